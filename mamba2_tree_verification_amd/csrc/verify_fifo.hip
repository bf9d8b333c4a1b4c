// verify_fifo.hip - ssm_tree_verify in the page's own form (flag
// SSM_TREE_VERIFY_FIFO): the breadth-first walk with a FIFO of live states.
//
// SpecMamba page sec. 3.2: the candidate tree is flattened breadth-first;
// the verifier takes a state from the front of a FIFO, forms each child's
// state from it, emits the child's output, queues the child's state when
// the child has children of its own, and releases the parent once its
// children are done.  Here:
//   h_v = dA_v h_parent + (dt_v x~_v) B_v^T,   y_v = C_v h_v + D x~_v
// with every child state materialised (no root projection), in fp32.
//
// Mapping.  One wave per (layer, sequence, 8 channels).  Lane (r, s) holds
// state row r, columns s N/8 .. s N/8 + N/8 - 1; y_v = C_v . h_v is an
// in-lane partial sum plus a 3-step butterfly over the row's 8 lanes.  The
// queue is a ring of K state slots in LDS indexed by the node's rank among
// internal nodes; the root state sits in slot K.  A tree whose peak queue
// occupancy exceeds K (capacity is a hint, results never depend on it)
// takes the fallback: each parent state is rebuilt by replaying the
// parent's root path from the root state, the same updates in the same
// order, so the results are identical.
//
// This is the reference form of the method on the GPU.  The root
// projection (verify.hip, verify_tt.hip, commit_verify.hip) computes the same outputs
// without materialising child states and is the default.
#include "common.h"

namespace ssmt {
namespace {

constexpr int kRows = 8;       // channels per wave
constexpr int kSegs = 8;       // lanes per channel row
constexpr int kRing = 8;       // queue capacity (states)

struct FifoLds {
  int parent, rank, cidx, depth, xt, dtx, dA, ring, total;
  // T = nodes, NPL = state values per lane
  __host__ __device__ FifoLds(int NPL) {
    int o = 0;
    parent = o; o += 4 * kMaxNodes;
    rank = o; o += 4 * kMaxNodes;      // slot to push to (internal: rank % K, leaf: scratch slot K + 1)
    cidx = o; o += 4 * kMaxNodes;      // conv input rows of taps 1..3 (node index or T + window row), 8 bits each
    depth = o; o += 4 * kMaxNodes;
    xt = o; o += 4 * kMaxNodes * kRows;   // conv outputs [T][8]
    dtx = o; o += 4 * kMaxNodes * kRows;  // dt * x~  [T][8]
    dA = o; o += 4 * kMaxNodes * kRows;   // exp(dt A) [T][8]
    ring = o; o += 4 * (kRing + 2) * kWave * NPL;  // [slot][value][lane]
    total = o;
  }
};

template <typename TIn, int NPL>
__device__ __forceinline__ void load_row(const TIn* p, float (&v)[NPL]) {
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = load_in(p, i);
}

// A lane's NPL consecutive inputs of one B or C row as raw words, loaded
// with the widest aligned vector loads and widened when used.
template <typename TIn, int NPL>
struct Row {
  static constexpr int NW = NPL * (int)sizeof(TIn) / 4;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const TIn* p) {
    if constexpr (NW % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
      }
    } else if constexpr (NW % 2 == 0) {
#pragma unroll
      for (int i = 0; i < NW / 2; ++i) {
        const uint2 q = reinterpret_cast<const uint2*>(p)[i];
        w[2 * i] = q.x; w[2 * i + 1] = q.y;
      }
    } else {
      w[0] = reinterpret_cast<const uint32_t*>(p)[0];
    }
  }
  __device__ __forceinline__ float get(int i) const {
    if constexpr (sizeof(TIn) == 2) return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
    return __uint_as_float(w[i]);
  }
};

}  // namespace

template <typename TIn, int NPL>
__global__ void __launch_bounds__(kWave) verify_fifo_kernel(VerifyArgs a) {
  const Dims d = a.d;
  const int T = d.T, N = d.N, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G;
  const int lane = threadIdx.x;
  const int r = lane / kSegs, s = lane % kSegs;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int c0 = blockIdx.x * kRows;
  const int c = c0 + r, h = c / P, g = h / (H / G);

  extern __shared__ __align__(16) unsigned char smem[];
  const FifoLds lo(NPL);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  int32_t* s_slot = reinterpret_cast<int32_t*>(smem + lo.rank);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);
  int32_t* s_depth = reinterpret_cast<int32_t*>(smem + lo.depth);
  float* s_xt = reinterpret_cast<float*>(smem + lo.xt);
  float* s_dtx = reinterpret_cast<float*>(smem + lo.dtx);
  float* s_dA = reinterpret_cast<float*>(smem + lo.dA);
  float* s_ring = reinterpret_cast<float*>(smem + lo.ring);
  auto slot_at = [&](int slot, int i) -> float& { return s_ring[(slot * NPL + i) * kWave + lane]; };
  __shared__ int s_peak;

  for (int i = lane; i < T; i += kWave) s_parent[i] = a.parent[(int64_t)b * T + i];
  __syncthreads();
  const bool valid = tree_is_valid(s_parent, T);
  if (blockIdx.x == 0 && l == 0 && lane == 0 && a.seq_status) a.seq_status[b] = valid ? SSM_TREE_OK : SSM_TREE_E_TREE;
  float* yo = a.y + unit * T * DI + c;
  if (!valid) {
    for (int i = lane; i < T * kRows; i += kWave) a.y[(unit * T + i / kRows) * DI + c0 + i % kRows] = __builtin_nanf("");
    return;
  }

  // ---- plan, one lane per node (T <= 64): queue slot, peak occupancy,
  // depth, conv input rows ----
  {
    const int v = lane;
    const int p = v < T ? s_parent[v] : -1;
    const uint64_t upto = (v == 63) ? ~0ull : ((1ull << (v + 1)) - 1);  // nodes 0..v
    // a parent leaves the queue at its first child (children are contiguous)
    const bool first_child = v < T && p >= 0 && (v == 0 || s_parent[v - 1] != p);
    const uint64_t pops = __ballot(first_child);
    s_slot[v] = 0;
    __syncthreads();
    if (first_child) s_slot[p] = 1;  // p has children: it is queued when formed
    __syncthreads();
    const bool internal = v < T && s_slot[v] == 1;
    __syncthreads();
    const uint64_t queued = __ballot(internal);
    const int rank = __popcll(queued & (upto >> 1));  // internal nodes before v
    if (v < T) s_slot[v] = internal ? rank % kRing : kRing + 1;
    // queue occupancy after node v: queued (internal, <= v) minus popped (parents whose first child is <= v)
    int occ = v < T ? __popcll(queued & upto) - __popcll(pops & upto) : 0;
    for (int off = 32; off > 0; off >>= 1) occ = max(occ, __shfl_xor(occ, off));
    if (v == 0) s_peak = occ;
    if (v < T) {
      int dep = 0;
      for (int u = v; u >= 0; u = s_parent[u]) ++dep;
      s_depth[v] = dep;
      int packed = 0;
      for (int jj = 1; jj < W; ++jj) {
        const int code = conv_input_code(s_parent, v, jj, W);
        packed |= (code >= 0 ? code : T + (-1 - code)) << (8 * (jj - 1));
      }
      s_cidx[v] = packed;
    }
  }
  __syncthreads();

  // ---- per (node, channel): conv output, dt * x~, dA ----
  const TIn* xg = reinterpret_cast<const TIn*>(a.x) + unit * T * DI;
  const TIn* wg = reinterpret_cast<const TIn*>(a.window) + unit * (int64_t)(W - 1) * DI;
  const TIn* dtr = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * H;
  for (int i = lane; i < T * kRows; i += kWave) {
    const int v = i / kRows, rr = i % kRows, cc = c0 + rr, hh = cc / P;
    const float* cw = a.prm.conv_w + ((int64_t)l * DI + cc) * W;
    float z = fmaf(cw[W - 1], load_in(xg, (int64_t)v * DI + cc), a.prm.conv_b ? a.prm.conv_b[(int64_t)l * DI + cc] : 0.0f);
    for (int jj = 1; jj < W; ++jj) {
      const int code = (s_cidx[v] >> (8 * (jj - 1))) & 255;
      const float u = code < T ? load_in(xg, (int64_t)code * DI + cc) : load_in(wg, (int64_t)(code - T) * DI + cc);
      z = fmaf(cw[W - 1 - jj], u, z);
    }
    const float xt = d.silu ? silu_f32(z) : z;
    const float dt = softplus_f32(load_in(dtr, (int64_t)v * H + hh) + a.prm.dt_bias[(int64_t)l * H + hh]);
    s_xt[v * kRows + rr] = xt;
    s_dtx[v * kRows + rr] = dt * xt;
    s_dA[v * kRows + rr] = expf(dt * a.prm.A[(int64_t)l * H + hh]);
  }
  // root state into slot K
  const float* h0p = reinterpret_cast<const float*>(a.state) + (unit * DI + c) * (int64_t)N + s * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) slot_at(kRing, i) = h0p[i];
  __syncthreads();

  const float Dh = a.prm.D[(int64_t)l * H + h];
  const TIn* Bg = reinterpret_cast<const TIn*>(a.B) + (unit * T * G + g) * (int64_t)N + s * NPL;
  const TIn* Cg = reinterpret_cast<const TIn*>(a.C) + (unit * T * G + g) * (int64_t)N + s * NPL;
  float hv[NPL], bv[NPL];

  // child v of the parent state hp: update, output (B and C rows prefetched)
  auto child = [&](int v, float (&hp)[NPL], const Row<TIn, NPL>& br, const Row<TIn, NPL>& cr) {
    const float dA = s_dA[v * kRows + r], dtx = s_dtx[v * kRows + r];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      hv[i] = fmaf(dA, hp[i], dtx * br.get(i));
      part = fmaf(cr.get(i), hv[i], part);
    }
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    part += __shfl_xor(part, 4);
    if (s == 0) yo[(int64_t)v * DI] = fmaf(Dh, s_xt[v * kRows + r], part);
  };

  float hp[NPL];
  // B and C rows two nodes ahead, in two register sets (even and odd nodes)
  Row<TIn, NPL> b0, c0r, b1, c1r;
  auto fetch = [&](int v, Row<TIn, NPL>& br, Row<TIn, NPL>& cr) {
    v = v < T ? v : T - 1;  // past the end: the last row again (branch-free)
    br.load(Bg + (int64_t)v * G * N);
    cr.load(Cg + (int64_t)v * G * N);
  };
  if (s_peak <= kRing) {
    // the page's walk: the parent's state comes off the queue (slot K: root)
    int cur = -2;
    auto step = [&](int v, Row<TIn, NPL>& br, Row<TIn, NPL>& cr) {
      const int p = s_parent[v];
      if (p != cur) {
        const int slot = p < 0 ? kRing : s_slot[p];
#pragma unroll
        for (int i = 0; i < NPL; ++i) hp[i] = slot_at(slot, i);
        cur = p;
      }
      child(v, hp, br, cr);
      fetch(v + 2, br, cr);
      // queue the child's state (leaves go to the scratch slot)
#pragma unroll
      for (int i = 0; i < NPL; ++i) slot_at(s_slot[v], i) = hv[i];
    };
    fetch(0, b0, c0r);
    fetch(1, b1, c1r);
    for (int v = 0; v < T; v += 2) {
      step(v, b0, c0r);
      if (v + 1 < T) step(v + 1, b1, c1r);
    }
  } else {
    // capacity exceeded: rebuild each parent state from the root along its path
    int cur = -2;
    for (int v = 0; v < T; ++v) {
      const int p = s_parent[v];
      if (p != cur) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) hp[i] = slot_at(kRing, i);
        // root path of p, root first
        const int dp = p < 0 ? 0 : s_depth[p];
        for (int k = 0; k < dp; ++k) {
          int u = p;
          for (int up = dp - 1 - k; up > 0; --up) u = s_parent[u];
          const float dA = s_dA[u * kRows + r], dtx = s_dtx[u * kRows + r];
          load_row<TIn, NPL>(Bg + (int64_t)u * G * N, bv);
#pragma unroll
          for (int i = 0; i < NPL; ++i) hp[i] = fmaf(dA, hp[i], dtx * bv[i]);
        }
        cur = p;
      }
      Row<TIn, NPL> br, cr;
      fetch(v, br, cr);
      child(v, hp, br, cr);
    }
  }
}

namespace {

template <typename TIn, int NPL>
int launch_fifo_t(const VerifyArgs& a, hipStream_t s) {
  const size_t lds = (size_t)FifoLds(NPL).total;
  if (allow_lds(verify_fifo_kernel<TIn, NPL>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  dim3 grid(a.d.d_in / kRows, a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((verify_fifo_kernel<TIn, NPL>), grid, dim3(kWave), lds, s, a);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

template <typename TIn>
int launch_fifo_in(const VerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_fifo_t<TIn, 2>(a, s);
    case 32: return launch_fifo_t<TIn, 4>(a, s);
    case 64: return launch_fifo_t<TIn, 8>(a, s);
    case 128: return launch_fifo_t<TIn, 16>(a, s);
    case 256: return launch_fifo_t<TIn, 32>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

}  // namespace

int launch_verify_fifo(const VerifyArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_fifo_in<bf16_t>(a, s) : launch_fifo_in<float>(a, s);
}

}  // namespace ssmt
