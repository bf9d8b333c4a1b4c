// verify_fifo.hip - ssm_tree_verify in the page's own form (flag
// SSM_TREE_VERIFY_FIFO): the breadth-first walk with a FIFO of live states.
//
// SpecMamba page sec. 3.2: the candidate tree is flattened breadth-first;
// the verifier takes a state from the front of a FIFO, forms each child's
// state from it, emits the child's output, queues the child's state when
// the child has children of its own, and releases the parent once its
// children are done.  Here:
//   h_v = dA_v h_parent + (dt_v x~_v) B_v^T,   y_v = C_v h_v + D x~_v
// with every child state materialised (no root projection), in fp32 on
// the vector ALU.
//
// Mapping.  One workgroup of 4 waves per (layer, sequence, 32 channels);
// wave w owns channels 8 w .. 8 w + 7 as four channel pairs, and lane
// (pair q, segment s) holds columns s N/16 .. s N/16 + N/16 - 1 of both
// channels of pair q.  The B and C segments a lane reads serve both of its
// channels.  y_v = C_v . h_v is an in-lane partial sum and a 4-step DPP
// reduction over the pair's 16 lanes (one DPP row).
//
// The FIFO lives in registers: K state slots per lane (K = 8 up to
// d_state 128, 4 at 256).  Parents leave the queue in breadth-first order,
// so the queued states always form a run of consecutive internal-node
// ranks, and rank mod K names a slot no queued state holds while the
// peak occupancy is at most K; the slot index is wave-uniform and picks
// the registers through a scalar branch.  A parent is copied out of its
// slot when its first child is formed (the slot is then free); leaves are
// never queued.  The root state is the parent of the first-level nodes.
// A tree whose peak occupancy exceeds K (capacity is a hint, results never
// depend on it) takes the fallback: each parent state is rebuilt by
// replaying the parent's root path from the root state, the same updates
// in the same order, so the results are identical.
//
// The plan (queue slots, peak, conv taps) and the per-(node, channel)
// scalars (conv output, dt x~, exp(dt A)) are formed once per workgroup
// into LDS; y is staged in LDS and leaves as whole row segments.
//
// This is the reference form of the method on the GPU.  The root
// projection (verify.hip, verify_tt.hip, commit_verify.hip) computes the
// same outputs without materialising child states and is the default.
#include "common.h"

namespace ssmt {
namespace {

constexpr int kFWaves = 4;
// s_waitcnt vmcnt(0), the other counters left alone (gfx9 encoding)
constexpr int kFifoWaitVm0 = 0x0F70;
constexpr int kFCh = 32;   // channels per workgroup (8 per wave)

// NS consecutive inputs of one B or C row as raw words, widened when used.
template <typename TIn, int NS>
struct SegRow {
  static constexpr int kBytes = NS * (int)sizeof(TIn);
  static constexpr int NW = kBytes >= 4 ? kBytes / 4 : 1;
  uint32_t w[NW];
  __device__ __forceinline__ void load(const TIn* p) {
    if constexpr (kBytes >= 16) {
#pragma unroll
      for (int i = 0; i < kBytes / 16; ++i) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
      }
    } else if constexpr (kBytes == 8) {
      const uint2 q = *reinterpret_cast<const uint2*>(p);
      w[0] = q.x; w[1] = q.y;
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = *reinterpret_cast<const unsigned short*>(p);
    }
  }
  __device__ __forceinline__ float get(int i) const {
    if constexpr (sizeof(TIn) == 2) return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
    return __uint_as_float(w[i]);
  }
};

// NS consecutive fp32 state values of one row
template <int NS>
__device__ __forceinline__ void load_state_seg(const float* p, float* out) {
  if constexpr (NS >= 4) {
#pragma unroll
    for (int i = 0; i < NS / 4; ++i) {
      const float4 q = reinterpret_cast<const float4*>(p)[i];
      out[4 * i] = q.x; out[4 * i + 1] = q.y; out[4 * i + 2] = q.z; out[4 * i + 3] = q.w;
    }
  } else if constexpr (NS == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    out[0] = q.x; out[1] = q.y;
  } else {
    out[0] = p[0];
  }
}

// v from another lane of the row; with 0 (the identity of the sum) as the
// old value the compiler folds the move into the add that takes it
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of a DPP row; every lane of the row gets it
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of the half row
  v += dpp<0x140>(v);  // row_mirror: the other half of the row
  return v;
}

// LDS layout of one workgroup: the tree tables, then per-(node, channel)
// tables sized by T (rounded up to a multiple of 4: the walk forms nodes
// four at a time), then the queue: K slots of the 32 channels' states,
// each lane's values as float4 (float2 at d_state 16) in lane order.
struct FifoLds {
  int parent, cidx, flag, word, depth, misc, xr, dt, sc, xt, y, path, ring, total;
  __host__ __device__ FifoLds(int T, int E, int K) {
    const int T4 = (T + 3) & ~3;
    int o = 0;
    parent = o; o += 4 * kMaxNodes;
    cidx = o; o += 4 * kMaxNodes;   // conv input rows of taps 1..3 (node index or T + window row), 8 bits each
    flag = o; o += 4 * kMaxNodes;   // node has children
    word = o; o += 4 * kMaxNodes;   // parent + 1 | (queue slot + 1) << 8 (slot 0: not queued)
    depth = o; o += 4 * kMaxNodes;
    misc = o; o += 16;              // peak queue occupancy, tree check flag
    xr = o; o += 4 * (T + 3) * kFCh; // raw x rows of the nodes, then the window rows (32 channels)
    dt = o; o += 4 * kFWaves * kWave; // dt_raw per (node, head of the workgroup) when they fit
    sc = o; o += 16 * T4 * kFCh / 2; // per (node, channel pair): exp(dt A), dt x~ of both channels
    xt = o; o += 4 * T * kFCh;      // conv output per (node, channel)
    y = o; o += 4 * T4 * kFCh;      // C . h per (node, channel)
    path = o; o += ((T * kMaxNodes + 15) / 16) * 16;  // root paths, top first (fallback only)
    ring = o; o += 4 * K * kFWaves * kWave * E;
    total = o;
  }
};

// queue capacity that keeps two workgroups per CU within 160 KiB of LDS
constexpr int kFifoLdsBudget = 80 * 1024;
constexpr int kFifoMaxSlots = 8;
__host__ __device__ inline int fifo_slots(int T, int E) {
  const int slot = 4 * kFWaves * kWave * E;
  const int k = (kFifoLdsBudget - FifoLds(T, E, 0).total) / slot;
  return k < 0 ? 0 : (k > kFifoMaxSlots ? kFifoMaxSlots : k);
}

}  // namespace

// The loads of one block of 32 channels that do not depend on the plan:
// its x and window rows (raw words), its dt_raw values, its parameters and
// its root state.  Issued a block ahead, they are in flight during the
// previous block's walk.
template <typename TIn, int NS>
struct FifoBlockLoads {
  static constexpr int kXW = kFCh * (int)sizeof(TIn) / 4;  // words per x row
  static constexpr int kXL = (kXW * (kMaxNodes + 3) + kFWaves * kWave - 1) / (kFWaves * kWave);
  uint32_t xw[kXL];
  float dtv, cw[4], cb, Ah, dtb, Dh;
  float h[2 * NS];
};

template <typename TIn, int NS>
__global__ void __launch_bounds__(kFWaves * kWave, NS * sizeof(TIn) <= 32 ? 2 : 1) verify_fifo_kernel(VerifyArgs a, int K, int NBK) {
  constexpr int E = 2 * NS;  // state values per lane (two channels)
  constexpr int EV = E >= 4 ? 4 : 2;  // values per LDS access
  typedef FifoBlockLoads<TIn, NS> BL;
  const Dims d = a.d;
  const int T = d.T, N = d.N, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G;
  const int T4 = (T + 3) & ~3;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qp = lane >> 4, s = lane & 15;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int blk0 = blockIdx.x * NBK;  // first 32-channel block of this workgroup
  const int pair = wave * 4 + qp;     // channel pair within a block
  const int ch = tid % kFCh;          // the channel whose conv and y this thread forms

  extern __shared__ __align__(16) unsigned char smem[];
  const FifoLds lo(T, E, K);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);
  int32_t* s_flag = reinterpret_cast<int32_t*>(smem + lo.flag);
  int32_t* s_word = reinterpret_cast<int32_t*>(smem + lo.word);
  int32_t* s_depth = reinterpret_cast<int32_t*>(smem + lo.depth);
  int32_t* s_misc = reinterpret_cast<int32_t*>(smem + lo.misc);
  float4* s_sc = reinterpret_cast<float4*>(smem + lo.sc);
  float* s_xt = reinterpret_cast<float*>(smem + lo.xt);
  float* s_y = reinterpret_cast<float*>(smem + lo.y);
  uint8_t* s_path = reinterpret_cast<uint8_t*>(smem + lo.path);
  float* s_ring = reinterpret_cast<float*>(smem + lo.ring);
  uint32_t* s_xr = reinterpret_cast<uint32_t*>(smem + lo.xr);
  float* s_dt = reinterpret_cast<float*>(smem + lo.dt);

  const TIn* dtr = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * H;
  const int xwords = BL::kXW * (T + W - 1);
  // heads of block blk's channels; their dt_raw values go through LDS when
  // one value per thread covers them
  auto heads = [&](int blk, int& h_lo, int& nh) {
    h_lo = blk * kFCh / P;
    nh = (blk * kFCh + kFCh - 1) / P - h_lo + 1;
  };
  // every load of block blk that does not depend on the plan (unconditional
  // loads from clamped indices; the surplus is never used)
  auto issue = [&](int blk, BL& L) __attribute__((always_inline)) {
    const int c0 = blk * kFCh, cc = c0 + ch, hh = cc / P;
    int h_lo, nh;
    heads(blk, h_lo, nh);
    const int dti = tid < T * nh ? tid : T * nh - 1;
    L.dtv = load_in(dtr, (int64_t)(dti / nh) * H + h_lo + dti % nh);
#pragma unroll
    for (int k = 0; k < BL::kXL; ++k) {
      int w = tid + k * kFWaves * kWave;
      w = w < xwords ? w : xwords - 1;
      const int r = w / BL::kXW, o = (w % BL::kXW) * (4 / (int)sizeof(TIn));
      const TIn* src = r < T ? reinterpret_cast<const TIn*>(a.x) + (unit * T + r) * (int64_t)DI + c0 + o
                             : reinterpret_cast<const TIn*>(a.window) + (unit * (W - 1) + (r - T)) * (int64_t)DI + c0 + o;
      L.xw[k] = *reinterpret_cast<const uint32_t*>(src);
    }
    const float* cwp = a.prm.conv_w + ((int64_t)l * DI + cc) * W;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) L.cw[jj] = cwp[jj < W ? jj : 0];
    L.cb = a.prm.conv_b ? a.prm.conv_b[(int64_t)l * DI + cc] : 0.0f;
    L.Ah = a.prm.A[(int64_t)l * H + hh];
    L.dtb = a.prm.dt_bias[(int64_t)l * H + hh];
    L.Dh = a.prm.D[(int64_t)l * H + hh];
    const float* h0p = reinterpret_cast<const float*>(a.state) + (unit * DI + c0 + 2 * pair) * (int64_t)N + s * NS;
    load_state_seg<NS>(h0p, L.h);
    load_state_seg<NS>(h0p + N, L.h + NS);
  };
  // B and C segments: node v's rows of block blk's group; four register
  // sets, node v's rows loaded while node v - 4 is formed
  auto group_rows = [&](int blk, const TIn*& Bg, const TIn*& Cg) {
    const int g = (blk * kFCh / P) / (H / G);
    Bg = reinterpret_cast<const TIn*>(a.B) + (unit * T * G + g) * (int64_t)N + s * NS;
    Cg = reinterpret_cast<const TIn*>(a.C) + (unit * T * G + g) * (int64_t)N + s * NS;
  };
  SegRow<TIn, NS> b0, cr0, b1, cr1, b2, cr2, b3, cr3;

  // ---- entry: the parent first (its wait counts the rest as in flight),
  // then the first block's loads and rows ----
  const int pv = a.parent[(int64_t)b * T + (tid < T ? tid : T - 1)];
  BL L;
  issue(blk0, L);
  {
    const TIn *Bg, *Cg;
    group_rows(blk0, Bg, Cg);
    b0.load(Bg); cr0.load(Cg);
    b1.load(Bg + (int64_t)(T > 1 ? 1 : 0) * G * N); cr1.load(Cg + (int64_t)(T > 1 ? 1 : 0) * G * N);
    b2.load(Bg + (int64_t)(T > 2 ? 2 : T - 1) * G * N); cr2.load(Cg + (int64_t)(T > 2 ? 2 : T - 1) * G * N);
    b3.load(Bg + (int64_t)(T > 3 ? 3 : T - 1) * G * N); cr3.load(Cg + (int64_t)(T > 3 ? 3 : T - 1) * G * N);
  }
  if (tid < T) s_parent[tid] = pv;
  if (tid < kMaxNodes) s_flag[tid] = 0;
  if (tid == 0) s_misc[1] = 0;
  __syncthreads();
  // BFS labelling check: parent[0] = -1, -1 <= parent[v] < v, non-decreasing
  if (tid < T) {
    const int p = s_parent[tid];
    if (tid == 0 ? p != -1 : (p < -1 || p >= tid || p < s_parent[tid - 1])) s_misc[1] = 1;
  }
  __syncthreads();
  const bool valid = s_misc[1] == 0;
  if (blockIdx.x == 0 && l == 0 && tid == 0 && a.seq_status) a.seq_status[b] = valid ? SSM_TREE_OK : SSM_TREE_E_TREE;
  if (!valid) {
    float* yo = a.y + unit * T * DI + blk0 * kFCh;
    for (int i = tid; i < T * kFCh * NBK; i += kFWaves * kWave)
      yo[(int64_t)(i / (kFCh * NBK)) * DI + i % (kFCh * NBK)] = __builtin_nanf("");
    return;
  }

  // ---- plan, once for every block: which nodes have children, conv input
  // rows, queue slots and peak occupancy ----
  if (tid < T) {
    const int v = tid, p = s_parent[v];
    if (p >= 0 && s_parent[v - 1] != p) s_flag[p] = 1;  // v is p's first child
    int packed = 0;
    for (int jj = 1; jj < W; ++jj) {
      const int code = conv_input_code(s_parent, v, jj, W);
      packed |= (code >= 0 ? code : T + (-1 - code)) << (8 * (jj - 1));
    }
    s_cidx[v] = packed;
  }
  __syncthreads();
  if (wave == 0) {
    const int v = lane;
    const int p = v < T ? s_parent[v] : -1;
    const bool internal = v < T && s_flag[v];
    const bool first_child = v < T && p >= 0 && s_parent[v - 1] != p;
    const uint64_t upto = (v == 63) ? ~0ull : ((1ull << (v + 1)) - 1);  // nodes 0..v
    const uint64_t queued = __ballot(internal);
    const uint64_t pops = __ballot(first_child);  // a parent leaves the queue at its first child
    const int rank = __popcll(queued & (upto >> 1));
    int occ = v < T ? __popcll(queued & upto) - __popcll(pops & upto) : 0;
    for (int off = 32; off > 0; off >>= 1) occ = max(occ, __shfl_xor(occ, off));
    if (v < T) s_word[v] = (p + 1) | ((internal && K > 0 ? rank % K + 1 : 0) << 8);
    // nodes T .. T4 - 1 pad the last group of four: children of the last
    // node's parent, never queued; what they form is never read
    if (v >= T && v < T4) s_word[v] = s_parent[T - 1] + 1;
    if (v == 0) s_misc[0] = occ;
  }
  __syncthreads();
  const bool over = s_misc[0] > K;  // past the queue capacity: replay fallback
  if (over) {
    build_paths(s_parent, T, s_depth, s_path);
    __syncthreads();
  }
  const int word = lane < T4 ? s_word[lane] : 0;
  auto slot_ptr = [&](int k, int j) { return s_ring + (((k * kFWaves + wave) * (E / EV) + j) * kWave + lane) * EV; };

  for (int bi = 0; bi < NBK; ++bi) {
    const int blk = blk0 + bi, c0 = blk * kFCh;
    const int nblk = bi + 1 < NBK ? blk + 1 : blk;  // the block whose loads go out during this walk
    int h_lo, nh;
    heads(blk, h_lo, nh);
    const bool dt_lds = T * nh <= kFWaves * kWave;
    // this block's x rows and dt_raw values to LDS; its parameters and root
    // state to registers (the previous block's y is out of LDS: barrier C)
    if (dt_lds && tid < T * nh) s_dt[tid] = L.dtv;
#pragma unroll
    for (int k = 0; k < BL::kXL; ++k)
      if (tid + k * kFWaves * kWave < xwords) s_xr[tid + k * kFWaves * kWave] = L.xw[k];
    float cw[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) cw[jj] = L.cw[jj];
    const float cb = L.cb, Ah = L.Ah, dtb = L.dtb, Dh = L.Dh;
    float hp[E];
#pragma unroll
    for (int i = 0; i < E; ++i) hp[i] = L.h[i];
    __syncthreads();  // A
    // per (node, channel): conv output, dt x~, exp(dt A); a thread keeps one
    // channel and takes every eighth node
    {
      float* scf = reinterpret_cast<float*>(s_sc);
      const int hh = (c0 + ch) / P;
      auto xrow = [&](int r) -> float {  // channel ch of row r (node, or T + window row)
        if constexpr (sizeof(TIn) == 2)
          return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(s_xr)[r * kFCh + ch] << 16);
        return __uint_as_float(s_xr[r * kFCh + ch]);
      };
      for (int v = tid / kFCh; v < T; v += kFWaves * kWave / kFCh) {
        float z = fmaf(cw[W - 1], xrow(v), cb);
        const int codes = s_cidx[v];
        for (int jj = 1; jj < W; ++jj) z = fmaf(cw[W - 1 - jj], xrow((codes >> (8 * (jj - 1))) & 255), z);
        const float xt = d.silu ? silu_f32(z) : z;
        const float dt =
            softplus_f32((dt_lds ? s_dt[v * nh + hh - h_lo] : load_in(dtr, (int64_t)v * H + hh)) + dtb);
        s_xt[v * kFCh + ch] = xt;
        *reinterpret_cast<float2*>(&scf[(v * kFCh / 2 + ch / 2) * 4 + (ch & 1) * 2]) =
            make_float2(expf(dt * Ah), dt * xt);
      }
    }
    __syncthreads();  // B
    issue(nblk, L);

    // ---- the walk (each wave on its own; no barriers) ----
    const TIn *Bg, *Cg, *Bn, *Cn;
    group_rows(blk, Bg, Cg);
    group_rows(nblk, Bn, Cn);
    // rows of node v + 4: this block's (clamped to T - 1), or past T4 the
    // next block's first four (so that its walk starts with them in place)
    auto fetch = [&](int v, SegRow<TIn, NS>& br, SegRow<TIn, NS>& cr) __attribute__((always_inline)) {
      const bool nx = v >= T4;
      const int r = nx ? v - T4 : (v < T ? v : T - 1);
      const int rr = r < T ? r : T - 1;
      br.load((nx ? Bn : Bg) + (int64_t)rr * G * N);
      cr.load((nx ? Cn : Cg) + (int64_t)rr * G * N);
    };
    int cur = -1;  // the parent whose state is in hp (-1: the root state)
    auto step = [&](int v, SegRow<TIn, NS>& br, SegRow<TIn, NS>& cr) __attribute__((always_inline)) {
      const int w = __builtin_amdgcn_readlane(word, v);
      const int p = (w & 0xFF) - 1;
      if (p != cur) {
        if (!over) {
          // the parent comes off the front of the queue
          const int ps = ((__builtin_amdgcn_readlane(word, p) >> 8) & 0xFF) - 1;
#pragma unroll
          for (int j = 0; j < E / EV; ++j) {
            if constexpr (EV == 4) {
              const float4 t = *reinterpret_cast<const float4*>(slot_ptr(ps, j));
              hp[4 * j] = t.x; hp[4 * j + 1] = t.y; hp[4 * j + 2] = t.z; hp[4 * j + 3] = t.w;
            } else {
              const float2 t = *reinterpret_cast<const float2*>(slot_ptr(ps, j));
              hp[2 * j] = t.x; hp[2 * j + 1] = t.y;
            }
          }
        } else {
          // rebuild the parent's state from the root along its path
          const float* h0p = reinterpret_cast<const float*>(a.state) + (unit * DI + c0 + 2 * pair) * (int64_t)N + s * NS;
          load_state_seg<NS>(h0p, hp);
          load_state_seg<NS>(h0p + N, hp + NS);
          for (int k = 0; k < s_depth[p]; ++k) {
            const int u = s_path[p * kMaxNodes + k];
            const float4 su = s_sc[u * kFCh / 2 + pair];
            SegRow<TIn, NS> bu;
            bu.load(Bg + (int64_t)u * G * N);
#pragma unroll
            for (int i = 0; i < NS; ++i) {
              hp[i] = fmaf(su.x, hp[i], su.y * bu.get(i));
              hp[NS + i] = fmaf(su.z, hp[NS + i], su.w * bu.get(i));
            }
          }
          __builtin_amdgcn_s_waitcnt(kFifoWaitVm0);  // no load of hp left in flight past this branch
        }
        cur = p;
      }
      const float4 sv = s_sc[v * kFCh / 2 + pair];
      float hv[E];
      float pa = 0.0f, pb = 0.0f;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const float bi_ = br.get(i), ci = cr.get(i);
        hv[i] = fmaf(sv.x, hp[i], sv.y * bi_);
        pa = fmaf(ci, hv[i], pa);
        hv[NS + i] = fmaf(sv.z, hp[NS + i], sv.w * bi_);
        pb = fmaf(ci, hv[NS + i], pb);
      }
      fetch(v + 4, br, cr);
      // queue the child's state when it has children of its own
      const int slot = ((w >> 8) & 0xFF) - 1;
      if (!over && slot >= 0) {
#pragma unroll
        for (int j = 0; j < E / EV; ++j) {
          if constexpr (EV == 4)
            *reinterpret_cast<float4*>(slot_ptr(slot, j)) =
                make_float4(hv[4 * j], hv[4 * j + 1], hv[4 * j + 2], hv[4 * j + 3]);
          else
            *reinterpret_cast<float2*>(slot_ptr(slot, j)) = make_float2(hv[2 * j], hv[2 * j + 1]);
        }
      }
      pa = row16_sum(pa);
      pb = row16_sum(pb);
      if (s == 0) *reinterpret_cast<float2*>(&s_y[v * kFCh + 2 * pair]) = make_float2(pa, pb);
    };
    for (int v = 0; v < T; v += 4) {
      step(v, b0, cr0);
      step(v + 1, b1, cr1);
      step(v + 2, b2, cr2);
      step(v + 3, b3, cr3);
    }
    __syncthreads();  // C

    // ---- y = C . h + D x~, whole row segments ----
    float* yo = a.y + unit * T * DI + c0;
    for (int i = tid; i < T * kFCh; i += kFWaves * kWave)  // channel i % 32 = ch
      yo[(int64_t)(i / kFCh) * DI + ch] = fmaf(Dh, s_xt[i], s_y[i]);
  }
}

namespace {

// blocks of 32 channels per workgroup: up to four, dividing the blocks of
// a (layer, sequence)
int fifo_blocks_per_workgroup(int d_in) {
  const int blocks = d_in / kFCh;
  for (int c = 4; c > 1; --c)
    if (blocks % c == 0) return c;
  return 1;
}

template <typename TIn, int NS>
int launch_fifo_t(const VerifyArgs& a, hipStream_t s) {
  const int K = fifo_slots(a.d.T, 2 * NS);
  const size_t lds = (size_t)FifoLds(a.d.T, 2 * NS, K).total;
  if (allow_lds(verify_fifo_kernel<TIn, NS>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  const int nbk = fifo_blocks_per_workgroup(a.d.d_in);
  dim3 grid(a.d.d_in / kFCh / nbk, a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((verify_fifo_kernel<TIn, NS>), grid, dim3(kFWaves * kWave), lds, s, a, K, nbk);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

template <typename TIn>
int launch_fifo_in(const VerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_fifo_t<TIn, 1>(a, s);
    case 32: return launch_fifo_t<TIn, 2>(a, s);
    case 64: return launch_fifo_t<TIn, 4>(a, s);
    case 128: return launch_fifo_t<TIn, 8>(a, s);
    case 256: return launch_fifo_t<TIn, 16>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

}  // namespace

int launch_verify_fifo(const VerifyArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_fifo_in<bf16_t>(a, s) : launch_fifo_in<float>(a, s);
}

}  // namespace ssmt
