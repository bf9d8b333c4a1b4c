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
// projection (verify_mfma.hip, verify.hip) computes the same outputs
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

  // ---- plan: queue slots, peak occupancy, depth, conv rows (one lane) ----
  if (lane == 0) {
    int n_internal = 0, occ = 0, peak = 0, cur = -1;
    for (int v = 0; v < T; ++v) {
      const int p = s_parent[v];
      if (p != cur) {  // the next queued parent comes off the front
        if (p >= 0) --occ;
        cur = p;
      }
      const bool internal = (v + 1 < T) && [&] {
        for (int u = v + 1; u < T; ++u)
          if (s_parent[u] == v) return true;
        return false;
      }();
      s_slot[v] = internal ? (n_internal++) % kRing : kRing + 1;
      if (internal) peak = max(peak, ++occ);
      s_depth[v] = p >= 0 ? s_depth[p] + 1 : 1;
      int packed = 0;
      for (int jj = 1; jj < W; ++jj) {
        const int code = conv_input_code(s_parent, v, jj, W);
        packed |= (code >= 0 ? code : T + (-1 - code)) << (8 * (jj - 1));
      }
      s_cidx[v] = packed;
    }
    s_peak = peak;
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
  const float* h0p = a.state + (unit * DI + c) * (int64_t)N + s * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) slot_at(kRing, i) = h0p[i];
  __syncthreads();

  const float Dh = a.prm.D[(int64_t)l * H + h];
  const TIn* Bg = reinterpret_cast<const TIn*>(a.B) + (unit * T * G + g) * (int64_t)N + s * NPL;
  const TIn* Cg = reinterpret_cast<const TIn*>(a.C) + (unit * T * G + g) * (int64_t)N + s * NPL;
  float hv[NPL], bv[NPL], cv[NPL];

  // child v of a parent state held in hv's place: update, output, queue
  auto child = [&](int v, float (&hp)[NPL]) {
    const float dA = s_dA[v * kRows + r], dtx = s_dtx[v * kRows + r];
    load_row<TIn, NPL>(Bg + (int64_t)v * G * N, bv);
    load_row<TIn, NPL>(Cg + (int64_t)v * G * N, cv);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      hv[i] = fmaf(dA, hp[i], dtx * bv[i]);
      part = fmaf(cv[i], hv[i], part);
    }
    part += __shfl_xor(part, 1);
    part += __shfl_xor(part, 2);
    part += __shfl_xor(part, 4);
    if (s == 0) yo[(int64_t)v * DI] = fmaf(Dh, s_xt[v * kRows + r], part);
  };

  float hp[NPL];
  if (s_peak <= kRing) {
    // the page's walk: the parent's state comes off the queue (slot K: root)
    int cur = -2;
    for (int v = 0; v < T; ++v) {
      const int p = s_parent[v];
      if (p != cur) {
        const int slot = p < 0 ? kRing : s_slot[p];
#pragma unroll
        for (int i = 0; i < NPL; ++i) hp[i] = slot_at(slot, i);
        cur = p;
      }
      child(v, hp);
      // queue the child's state (leaves go to the scratch slot)
#pragma unroll
      for (int i = 0; i < NPL; ++i) slot_at(s_slot[v], i) = hv[i];
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
      child(v, hp);
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
