// verify.hip - ssm_tree_verify kernel for gfx950.
//
// What is computed (SpecMamba page sec. 3.2; LightMamba section "why Mamba
// is hard to accelerate"): for every node v of a BFS-ordered draft tree,
//   h_v = dA_v h_parent + (dt_v x~_v) B_v^T,   y_v = h_v C_v + D x~_v,
// with h_parent the root state for root-level nodes.
//
// How it is computed on gfx950.  Unrolling the recurrence along the root
// path u_0 .. u_{m-1} = v of node v gives
//   h_v = a_v h0 + Delta_v,
//   a_v = prod_k dA_{u_k},
//   Delta_v = sum_k (prod_{k' > k} dA_{u_k'}) (dt x~)_{u_k} B_{u_k}^T,
// so every child state is its parent's state, decayed, plus one rank-1
// term: each node's state is carried as the shared root state h0 and the
// rank-1 factors along its path, and a child's factors are its parent's
// plus its own.  Then
//   y_v[c] = a_v (C_v . h0[c])                                          (1)
//          + sum_{u on path(v)} M_h[v][u] x~_u[c]                       (2)
//   M_h[v][u] = (prod of dA strictly below u on v's path) dt_u (C_v . B_u),
//               plus D_h on the diagonal.
// (1) is the only work per state element: each element of the root state
// is read once from HBM and multiplied by the T node vectors C_v (T FMAs per
// element, on VALU: an HBM-bound stream with T flops per 4 bytes).  (2)
// costs one FMA per (node, ancestor, channel); M and the T x T dots
// C_v . B_u do not depend on N.  Child states are never materialised, so y
// is the only output.
//
// Trees of at most 16 nodes whose heads are a multiple of 16 channels wide
// take the round's kernel in commit_verify.hip with nothing to commit, and
// trees of 17-64 nodes the matrix-core kernels of verify_tt.hip (same
// formula, both sums as MFMA contractions); this file's VALU kernel serves
// every other shape.
//
// Mapping.  A workgroup of NW waves owns one (layer, sequence) and NBLK
// consecutive blocks of NW*R*64 channels (rows of the root state) inside one
// B/C group; the tree prologue (paths, step sizes, C.B dots) runs once per
// workgroup.  A lane owns R rows of a block; all lanes of a wave walk the
// state index n together, so C_v[n] is wave-uniform and reaches v_fmac from
// scalar registers.  The root state is streamed in 16-column chunks:
// coalesced 16-byte loads kept two chunks ahead in registers, across block
// boundaries, then a swizzled LDS transpose so that each lane reads its own
// rows.
#include "common.h"

namespace ssmt {

namespace {

constexpr int kChunk = 16;  // state columns per streamed chunk
constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// C rows are read with scalar buffer loads (s_buffer_load_dwordx8): the
// offsets are wave-uniform, the values land in SGPRs and feed v_fmac
// directly, and a buffer resource holds the base so that only a 32-bit
// offset per load stays live.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
__device__ u32x8 scalar_buffer_load_x8(i32x4 rsrc, int byte_offset, int aux) __asm("llvm.amdgcn.s.buffer.load.v8i32");

// buffer resource over `bytes` bytes at `base` (raw dword access)
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;  // 32-bit data format, no swizzle, no stride
  return r;
}

// 16 consecutive values of a node's C row: raw dwords (loaded one node
// ahead) and their float values.
template <typename TIn>
struct CRow;

template <>
struct CRow<float> {
  struct raw { u32x8 lo, hi; };
  static __device__ __forceinline__ raw load(i32x4 rsrc, int off) {
    return raw{scalar_buffer_load_x8(rsrc, off, 0), scalar_buffer_load_x8(rsrc, off + 32, 0)};
  }
  static __device__ __forceinline__ float get(const raw& w, int i) { return __uint_as_float(i < 8 ? w.lo[i] : w.hi[i - 8]); }
};

template <>
struct CRow<bf16_t> {
  typedef u32x8 raw;
  static __device__ __forceinline__ raw load(i32x4 rsrc, int off) { return scalar_buffer_load_x8(rsrc, off, 0); }
  static __device__ __forceinline__ float get(const raw& w, int i) {
    return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
  }
};

// One input element as raw bits (loaded early, widened when used).
template <typename TIn>
__device__ __forceinline__ uint32_t load_bits(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ uint32_t load_bits<float>(const float* p, int64_t i) { return __float_as_uint(p[i]); }
template <>
__device__ __forceinline__ uint32_t load_bits<bf16_t>(const bf16_t* p, int64_t i) { return p[i].bits; }
template <typename TIn>
__device__ __forceinline__ float widen_bits(uint32_t b) { return sizeof(TIn) == 2 ? __uint_as_float(b << 16) : __uint_as_float(b); }

// Raw 4-element loads converted to float later, so that a thread can issue
// several before waiting on any.
template <typename TIn>
struct RawQuad;

template <>
struct RawQuad<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ type load(const void* base, int64_t off) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + off);
  }
  static __device__ __forceinline__ f32x4 widen(type r) { return r; }
};

template <>
struct RawQuad<bf16_t> {
  typedef uint2 type;
  static __device__ __forceinline__ type load(const void* base, int64_t off) {
    return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
  }
  static __device__ __forceinline__ f32x4 widen(type w) {
    f32x4 r;
    r.x = __uint_as_float(w.x << 16);
    r.y = __uint_as_float(w.x & 0xFFFF0000u);
    r.z = __uint_as_float(w.y << 16);
    r.w = __uint_as_float(w.y & 0xFFFF0000u);
    return r;
  }
};

}  // namespace

// One streamed chunk of R * 64 rows x 16 columns of the root state:
// transpose through LDS (swizzled to avoid bank conflicts), refill `gbuf`
// from `next` (the chunk this buffer serves next; the stream's last chunk
// again once past the end, so the loop stays branch-free) and
// accumulate acc[j][v] += C_v[n] h0[row j][n] over the 16 columns.  In the
// buffer `c_rsrc`, node 0's C values start at byte `c_off` and successive
// nodes' rows are `c_stride` bytes apart.
template <typename TIn, int R, int TMAX>
__device__ __forceinline__ void stream_chunk(f32x4 (&gbuf)[R * 4], const float* next, int64_t row_step,
                                             f32x4* lds4, int lane, i32x4 c_rsrc, int c_off,
                                             int c_stride, int T, float (&acc)[R][TMAX]) {
#pragma unroll
  for (int i = 0; i < R * 4; ++i) {
    const int row = i * 16 + (lane >> 2), q = lane & 3;
    lds4[row * 4 + (q ^ swz(row))] = gbuf[i];
  }
#pragma unroll
  for (int i = 0; i < R * 4; ++i) gbuf[i] = *reinterpret_cast<const f32x4*>(next + i * row_step);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float hv[R][kChunk];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int row = j * kWave + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 t = lds4[row * 4 + (q ^ swz(row))];
      hv[j][q * 4 + 0] = t.x;
      hv[j][q * 4 + 1] = t.y;
      hv[j][q * 4 + 2] = t.z;
      hv[j][q * 4 + 3] = t.w;
    }
  }
  // node by node, the next node's C row in flight while this one's FMAs
  // issue; the scheduling barriers keep the compiler from hoisting every
  // node's C values into scalar registers at once
  typename CRow<TIn>::raw w_next = CRow<TIn>::load(c_rsrc, c_off);
#pragma unroll
  for (int v = 0; v < TMAX; ++v) {
    const typename CRow<TIn>::raw w = w_next;
    if (v + 1 < TMAX) w_next = CRow<TIn>::load(c_rsrc, c_off + (v + 1 < T ? v + 1 : T - 1) * c_stride);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const float cval = CRow<TIn>::get(w, i);
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j][v] = fmaf(cval, hv[j][i], acc[j][v]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Launch geometry shared by the host (LDS sizing) and the kernel.
struct VerifyGeom {
  int NW;    // waves per workgroup
  int NBLK;  // channel blocks per workgroup
  int HWG;   // max heads touched by a workgroup's channel range
  int HB;    // max heads touched by one block
  int NC;    // columns of B and C staged per pass for the C.B dots
};

// LDS layout of one workgroup (byte offsets; identical on host and device)
template <int R, int TMAX, bool DENSE>
struct VerifyLds {
  static constexpr int kPairs = TMAX * (TMAX + 1) / 2;
  static constexpr int kWaveScratch = (R * kWave * kChunk > (TMAX + 3) * kWave) ? R * kWave * kChunk : (TMAX + 3) * kWave;
  int parent, depth, cidx, path, onk, dt, S, Dh, cb, pair, a, dA, M, dyn, total;
  __host__ __device__ VerifyLds(const VerifyGeom& g) {
    int o = 0;
    parent = o; o += 4 * kMaxNodes;
    depth = o; o += 4 * kMaxNodes;
    cidx = o; o += 4 * kMaxNodes;
    path = o; o += (TMAX * TMAX + 15) & ~15;
    onk = o; o += (TMAX * TMAX + 15) & ~15;
    dt = o; o += 4 * TMAX * g.HWG;
    S = o; o += 8 * TMAX * g.HWG;                              // float64
    Dh = o; o += 4 * ((g.HWG + 3) & ~3);
    cb = o; o += 4 * TMAX * TMAX;
    pair = o; o += (2 * kPairs + 15) & ~15;
    a = o; o += 3 * 4 * TMAX * g.HB;                           // three blocks in flight
    dA = o; o += DENSE ? 0 : 3 * 4 * TMAX * g.HB;
    M = o; o += DENSE ? 3 * 4 * g.HB * TMAX * TMAX : 0;
    dyn = o;
    const int stage = 2 * TMAX * (g.NC + 4);
    o += 4 * (g.NW * kWaveScratch > stage ? g.NW * kWaveScratch : stage);
    total = o;
  }
};

template <typename TIn, int R, int TMAX, bool DENSE>
__global__ void __launch_bounds__(kThreads) verify_proj_kernel(VerifyArgs a, VerifyGeom geo) {
  typedef VerifyLds<R, TMAX, DENSE> Lds;
  const Dims d = a.d;
  const int T = d.T, N = d.N, P = d.P, H = d.H, W = d.W, DI = d.d_in;
  const int NW = geo.NW, NBLK = geo.NBLK;
  const int BC = NW * R * kWave;                          // channels per block
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int c_wg = blockIdx.x * NBLK * BC;                // first channel of the workgroup
  const int g = c_wg / (DI / d.G);                        // B/C group of the workgroup
  const int h_wg = c_wg / P;                              // first head of the workgroup
  const int HWG = (c_wg + NBLK * BC - 1) / P - h_wg + 1;

  extern __shared__ __align__(16) unsigned char smem[];
  const Lds lo(geo);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  int32_t* s_depth = reinterpret_cast<int32_t*>(smem + lo.depth);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);   // xs rows of conv inputs 1..3, 8 bits each
  uint8_t* s_path = smem + lo.path;                                // [TMAX][TMAX] root path, top first
  uint8_t* s_onk = smem + lo.onk;                                  // [TMAX][TMAX] k + 1 if u = path(v)[k], else 0
  float* s_dt = reinterpret_cast<float*>(smem + lo.dt);            // [TMAX][HWG] dt
  // [TMAX][HWG] sum of dt * A over the root path, float64: on a deep path
  // with large steps S_v and S_u are large and close, and their difference
  // (the decay between u and v) must not lose its digits to rounding
  double* s_S = reinterpret_cast<double*>(smem + lo.S);
  float* s_D = reinterpret_cast<float*>(smem + lo.Dh);             // [HWG]
  float* s_cb = reinterpret_cast<float*>(smem + lo.cb);            // [TMAX][TMAX] C_v . B_(k-th path node)
  uint16_t* s_pair = reinterpret_cast<uint16_t*>(smem + lo.pair);  // (v << 8 | k)
  // per-block coefficients, buffer blk % 3: block k+1's are written during block
  // k's stream while block k's are read by its epilogue
  float* s_a = reinterpret_cast<float*>(smem + lo.a);              // [3][TMAX][HB] decay of the root state
  float* s_dA = reinterpret_cast<float*>(smem + lo.dA);            // [3][TMAX][HB] (path-walk epilogue)
  float* s_M = reinterpret_cast<float*>(smem + lo.M);              // [3][HB][TMAX][TMAX] (dense epilogue)
  float* s_dyn = reinterpret_cast<float*>(smem + lo.dyn);          // prologue staging, then per wave
  float* s_mine = s_dyn + wave * Lds::kWaveScratch;

  // ---- state stream: chunk s = (block s / NCH, columns (s % NCH) * 16) ----
  const int NCH = N / kChunk;
  const int total = NBLK * NCH;
  // lane -> (row lane/4 + 16 i, quad lane%4) of instruction i of a chunk
  const float* st_wave = reinterpret_cast<const float*>(a.state) + (unit * DI + c_wg + wave * R * kWave + (lane >> 2)) * (int64_t)N + (lane & 3) * 4;
  const int64_t row_step = (int64_t)16 * N;
  auto chunk_src = [&](int s) {
    const int blk = s / NCH, ch = s % NCH;
    return st_wave + (int64_t)blk * BC * N + ch * kChunk;
  };
  // two buffers when a block has an even number of chunks (chunk s in buffer
  // s % 2, refilled two chunks ahead), else one buffer refilled one ahead
  const bool two = (NCH % 2) == 0;
  f32x4 gA[R * 4], gB[R * 4];
  {
    const float* p = chunk_src(0);
#pragma unroll
    for (int i = 0; i < R * 4; ++i) gA[i] = *reinterpret_cast<const f32x4*>(p + i * row_step);
    if (two) {
      const float* q = chunk_src(1);
#pragma unroll
      for (int i = 0; i < R * 4; ++i) gB[i] = *reinterpret_cast<const f32x4*>(q + i * row_step);
    }
  }

  // ---- tree prologue, once per workgroup ----
  // unconditional (clamped) load: a branch here would make every T-derived
  // address look lane-dependent to the compiler and cost the scalar C loads
  const int par_in = a.parent[(int64_t)b * T + (tid < T ? tid : T - 1)];
  const int NC = geo.NC;
  const int q4 = NC / 4;
  const int nq = 2 * T * q4;  // quads per staging pass
  constexpr int kQ = 4;       // staged quads per thread issued before the first wait
  typename RawQuad<TIn>::type stq[kQ];
  float* sc = s_dyn;                          // [T][NC + 4]  C rows
  float* sb = s_dyn + TMAX * (NC + 4);        // [T][NC + 4]  B rows
  auto row_off = [&](int v, int n) { return ((unit * T + v) * d.G + g) * (int64_t)N + n; };
  auto stage_issue = [&](int n0) {
#pragma unroll
    for (int qi = 0; qi < kQ; ++qi) {
      const int i = tid + qi * nthr;
      const int r0 = i / q4, q = i % q4;
      const int r = r0 < 2 * T ? r0 : 2 * T - 1;
      stq[qi] = RawQuad<TIn>::load(r < T ? a.C : a.B, row_off(r < T ? r : r - T, n0 + q * 4));
    }
  };
  auto stage_store = [&](int n0) {
#pragma unroll
    for (int qi = 0; qi < kQ; ++qi) {
      const int i = tid + qi * nthr;
      const int r = i / q4, q = i % q4;
      if (r < 2 * T)
        *reinterpret_cast<f32x4*>((r < T ? sc + r * (NC + 4) : sb + (r - T) * (NC + 4)) + q * 4) =
            RawQuad<TIn>::widen(stq[qi]);
    }
    for (int i = tid + kQ * nthr; i < nq; i += nthr) {
      const int r = i / q4, q = i % q4;
      const auto raw = RawQuad<TIn>::load(r < T ? a.C : a.B, row_off(r < T ? r : r - T, n0 + q * 4));
      *reinterpret_cast<f32x4*>((r < T ? sc + r * (NC + 4) : sb + (r - T) * (NC + 4)) + q * 4) =
          RawQuad<TIn>::widen(raw);
    }
  };
  stage_issue(0);

  if (tid < T) s_parent[tid] = par_in;
  __syncthreads();
  const bool valid = tree_is_valid(s_parent, T);
  if (blockIdx.x == 0 && l == 0 && tid == 0 && a.seq_status) a.seq_status[b] = valid ? SSM_TREE_OK : SSM_TREE_E_TREE;
  if (!valid) {
    const float qnan = __builtin_nanf("");
    const int nch = NBLK * BC;
    for (int i = tid; i < T * nch; i += nthr) a.y[(unit * T + i / nch) * DI + c_wg + i % nch] = qnan;
    return;
  }
  // root paths and depths; conv input rows (node index, or T + window row)
  for (int v = tid; v < T; v += nthr) {
    int dep = 0;
    for (int u = v; u >= 0; u = s_parent[u]) ++dep;
    s_depth[v] = dep;
    int k = dep - 1;
    for (int u = v; u >= 0; u = s_parent[u]) s_path[v * TMAX + (k--)] = (uint8_t)u;
    int packed = 0;
    for (int j = 1; j < W; ++j) {
      const int code = conv_input_code(s_parent, v, j, W);
      packed |= (code >= 0 ? code : T + (-1 - code)) << (8 * (j - 1));
    }
    s_cidx[v] = packed;
  }
  const TIn* dtr = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * H;
  for (int i = tid; i < T * HWG; i += nthr) {
    const int v = i / HWG, hh = i % HWG, h = h_wg + hh;
    const float dt = softplus_f32(load_in(dtr, (int64_t)v * H + h) + a.prm.dt_bias[(int64_t)l * H + h]);
    s_dt[v * HWG + hh] = dt;
    s_S[v * HWG + hh] = (double)(dt * a.prm.A[(int64_t)l * H + h]);  // this node's own term for now
  }
  for (int i = tid; i < TMAX * TMAX; i += nthr) s_onk[i] = 0;
  for (int i = tid; i < HWG; i += nthr) s_D[i] = a.prm.D[(int64_t)l * H + h_wg + i];
  stage_store(0);
  __syncthreads();
  // cumulative log-decay along each root path (parents precede children)
  for (int hh = tid; hh < HWG; hh += nthr)
    for (int v = 0; v < T; ++v)
      if (s_parent[v] >= 0) s_S[v * HWG + hh] += s_S[s_parent[v] * HWG + hh];
  for (int v = tid; v < T; v += nthr)
    for (int k = 0; k < s_depth[v]; ++k) s_onk[v * TMAX + s_path[v * TMAX + k]] = (uint8_t)(k + 1);
  // (node, ancestor) pairs: node v owns slots [sum of earlier depths, + depth(v))
  for (int v = tid; v < T; v += nthr) {
    int off = 0;
    for (int w = 0; w < v; ++w) off += s_depth[w];
    for (int k = 0; k < s_depth[v]; ++k) s_pair[off + k] = (uint16_t)(v << 8 | k);
  }
  int npairs = 0;
  for (int w = 0; w < T; ++w) npairs += s_depth[w];
  __syncthreads();
  // C_v . B_u for every pair, one thread per pair, accumulated in n order
  for (int n0 = 0; n0 < N; n0 += NC) {
    if (n0) {
      __syncthreads();
      stage_issue(n0);
      stage_store(n0);
      __syncthreads();
    }
    for (int p = tid; p < npairs; p += nthr) {
      const int v = s_pair[p] >> 8, k = s_pair[p] & 255;
      const int u = s_path[v * TMAX + k];
      const f32x4* cr = reinterpret_cast<const f32x4*>(sc + v * (NC + 4));
      const f32x4* br = reinterpret_cast<const f32x4*>(sb + u * (NC + 4));
      float acc0 = n0 ? s_cb[v * TMAX + k] : 0.0f;
      for (int q = 0; q < q4; ++q) {
        const f32x4 cv = cr[q], bv = br[q];
        acc0 = fmaf(cv.x, bv.x, acc0);
        acc0 = fmaf(cv.y, bv.y, acc0);
        acc0 = fmaf(cv.z, bv.z, acc0);
        acc0 = fmaf(cv.w, bv.w, acc0);
      }
      s_cb[v * TMAX + k] = acc0;
    }
  }
  // the staging area becomes the per-wave scratch once every pair is done
  __syncthreads();

  const TIn* xin = reinterpret_cast<const TIn*>(a.x) + unit * T * DI;
  const TIn* win = reinterpret_cast<const TIn*>(a.window) + unit * (W - 1) * (int64_t)DI;
  f32x4* lds4 = reinterpret_cast<f32x4*>(s_mine);
  float acc[R][TMAX];
  uint32_t xr[R][TMAX + 3];  // the block's raw x (nodes, then window rows), in flight during the stream
  float wt[R][5];            // the block's conv weights (input jj = jj-th ancestor) and bias, likewise

  // Per-block coefficients a_v, and M_h[v][u] (dense) or dA (path walk):
  // slice `part` of `nparts` of them, so that they can be spread over a
  // block's chunks.
  auto block_coeffs = [&](int blk, int part, int nparts) {
    const int c0 = c_wg + blk * BC;
    const int hb0 = c0 / P - h_wg;  // first head of the block, workgroup-relative
    const int HBk = (c0 + BC - 1) / P - c0 / P + 1;
    const int buf = blk % 3;
    float* sa = s_a + buf * TMAX * geo.HB;
    for (int i = tid + part * nthr; i < T * HBk; i += nparts * nthr) {
      const int v = i / HBk, hb = i % HBk;
      const double Sv = s_S[v * HWG + hb0 + hb];
      sa[v * geo.HB + hb] = expf((float)Sv);
      if constexpr (!DENSE) {
        const int p = s_parent[v];
        s_dA[buf * TMAX * geo.HB + v * geo.HB + hb] = expf((float)(p >= 0 ? Sv - s_S[p * HWG + hb0 + hb] : Sv));
      }
    }
    if constexpr (DENSE) {
      float* sm = s_M + buf * geo.HB * TMAX * TMAX;
      // every column of the rows read, zero past T as well as off the path:
      // the product below runs over all TMAX columns
      for (int i = tid + part * nthr; i < HBk * T * TMAX; i += nparts * nthr) {
        const int hb = i / (T * TMAX), v = (i / TMAX) % T, u = i % TMAX;
        const int k1 = u < T ? s_onk[v * TMAX + u] : 0;
        float val = 0.0f;
        if (k1) {
          const int hw = hb0 + hb;
          val = expf((float)(s_S[v * HWG + hw] - s_S[u * HWG + hw])) * s_dt[u * HWG + hw] * s_cb[v * TMAX + k1 - 1];
          if (u == v) val += s_D[hw];
        }
        sm[(hb * TMAX + v) * TMAX + u] = val;
      }
    }
  };

  // Per-row epilogue of one block: conv outputs, path corrections, y.
  auto block_epilogue = [&](int blk) {
    const int c_blk = c_wg + blk * BC;
    const int c_row0 = c_blk + wave * R * kWave;
    float* xs = s_mine;  // [(T + W - 1)][64] raw x of the nodes, then the window rows
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int c = c_row0 + j * kWave + lane;
      const int hb = c / P - c_blk / P;  // block-relative head
      const int hw = c / P - h_wg;       // workgroup-relative head
      // raw x of every node and the window rows, prefetched at block start
#pragma unroll
      for (int v = 0; v < TMAX + 3; ++v)
        if (v < T + W - 1) xs[v * kWave + lane] = widen_bits<TIn>(xr[j][v]);
      const float* wj = wt[j];  // prefetched: wj[jj] weighs conv input jj (0 = the node itself)
      const float cbias = wt[j][4];
      const float* sa = s_a + (blk % 3) * TMAX * geo.HB;
      float* yo = a.y + unit * T * DI + c;
      if constexpr (DENSE) {
        // conv outputs of every node in registers; the input rows are wave-uniform
        float xt[TMAX];
#pragma unroll
        for (int v = 0; v < TMAX; ++v) {
          xt[v] = 0.0f;
          if (v < T) {
            const int ci = __builtin_amdgcn_readfirstlane(s_cidx[v]);
            float z = fmaf(wj[0], xs[v * kWave + lane], cbias);
#pragma unroll
            for (int jj = 1; jj < 4; ++jj)
              if (jj < W) z = fmaf(wj[jj], xs[((ci >> (8 * (jj - 1))) & 255) * kWave + lane], z);
            xt[v] = d.silu ? silu_f32(z) : z;
          }
        }
        // the raw inputs are consumed: park the accumulators in their place,
        // then one node per iteration against the full row of M (zero off the
        // node's path), so that M is never held in registers at once
        float* accs = xs;
#pragma unroll
        for (int v = 0; v < TMAX; ++v) accs[v * kWave + lane] = acc[j][v];
        const float* Mh = s_M + ((blk % 3) * geo.HB + hb) * TMAX * TMAX;
        bool fin = true;
#pragma unroll
        for (int v = 0; v < TMAX; ++v) fin = fin && __builtin_isfinite(xt[v]);
        if (__ballot(!fin) == 0) {
#pragma unroll 4
          for (int v = 0; v < T; ++v) {
            const f32x4* Mrow = reinterpret_cast<const f32x4*>(Mh + v * TMAX);
            float yv = sa[v * geo.HB + hb] * accs[v * kWave + lane];
#pragma unroll
            for (int u4 = 0; u4 < TMAX / 4; ++u4) {
              const f32x4 m = Mrow[u4];
              yv = fmaf(m.x, xt[4 * u4 + 0], yv);
              yv = fmaf(m.y, xt[4 * u4 + 1], yv);
              yv = fmaf(m.z, xt[4 * u4 + 2], yv);
              yv = fmaf(m.w, xt[4 * u4 + 3], yv);
            }
            yo[(int64_t)v * DI] = yv;
          }
        } else {
          // a non-finite conv output among the wave's channels: the zero
          // weight of a node off v's root path would still make y_v NaN, so
          // each node sums over its own root path alone, as the definition
          // has it
          for (int v = 0; v < T; ++v) {
            const float* Mrow = Mh + v * TMAX;
            float yv = sa[v * geo.HB + hb] * accs[v * kWave + lane];
#pragma unroll
            for (int u = 0; u < TMAX; ++u)
              if (u < T && s_onk[v * TMAX + u]) yv = fmaf(Mrow[u], xt[u], yv);
            yo[(int64_t)v * DI] = yv;
          }
        }
      } else {
        // deep trees: conv in place over LDS (descending, so every input is
        // still raw), then Horner along each root path
        for (int v = T - 1; v >= 0; --v) {
          const int ci = s_cidx[v];
          float z = fmaf(wj[0], xs[v * kWave + lane], cbias);
#pragma unroll
          for (int jj = 1; jj < 4; ++jj)
            if (jj < W) z = fmaf(wj[jj], xs[((ci >> (8 * (jj - 1))) & 255) * kWave + lane], z);
          xs[v * kWave + lane] = d.silu ? silu_f32(z) : z;
        }
        const float Dh = s_D[hw];
#pragma unroll
        for (int v = 0; v < TMAX; ++v) {
          if (v < T) {
            const int m = s_depth[v];
            float S = 0.0f;
            for (int k = 0; k < m; ++k) {
              const int u = s_path[v * TMAX + k];
              S = fmaf(S, s_dA[(blk % 3) * TMAX * geo.HB + u * geo.HB + hb],
                       (s_dt[u * HWG + hw] * s_cb[v * TMAX + k]) * xs[u * kWave + lane]);
            }
            yo[(int64_t)v * DI] = fmaf(sa[v * geo.HB + hb], acc[j][v], S) + Dh * xs[v * kWave + lane];
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  // this (layer, sequence)'s C rows as a scalar buffer: node v, group g,
  // column n at byte ((v * G + g) * N + n) * sizeof(input)
  const i32x4 c_rsrc = make_rsrc(reinterpret_cast<const TIn*>(a.C) + unit * T * d.G * N,
                                 (uint32_t)(T * d.G * N * (int)sizeof(TIn)));
  const int c_goff = g * N * (int)sizeof(TIn);
  const int c_stride = d.G * N * (int)sizeof(TIn);
  block_coeffs(0, 0, 1);
  for (int blk = 0; blk < NBLK; ++blk) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int c = c_wg + blk * BC + wave * R * kWave + j * kWave + lane;
#pragma unroll
      for (int v = 0; v < TMAX + 3; ++v) {
        const int vv = v < T + W - 1 ? v : T + W - 2;  // clamped: every load is in bounds
        const TIn* src = vv < T ? xin + (int64_t)vv * DI : win + (int64_t)(vv - T) * DI;
        xr[j][v] = load_bits(src, c);
      }
      const float* cw = a.prm.conv_w + ((int64_t)l * DI + c) * W;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wt[j][jj] = cw[jj < W ? W - 1 - jj : 0] * (jj < W ? 1.0f : 0.0f);
      wt[j][4] = a.prm.conv_b ? a.prm.conv_b[(int64_t)l * DI + c] : 0.0f;
#pragma unroll
      for (int v = 0; v < TMAX; ++v) acc[j][v] = 0.0f;
    }
    const bool more = blk + 1 < NBLK;
    if (two) {
      for (int ch = 0; ch < NCH; ch += 2) {
        const int s = blk * NCH + ch;
        stream_chunk<TIn, R, TMAX>(gA, chunk_src(min(s + 2, total - 1)), row_step, lds4, lane, c_rsrc,
                                   c_goff + ch * kChunk * (int)sizeof(TIn), c_stride, T, acc);
        if (more) block_coeffs(blk + 1, ch, NCH);
        stream_chunk<TIn, R, TMAX>(gB, chunk_src(min(s + 3, total - 1)), row_step, lds4, lane, c_rsrc,
                                   c_goff + (ch + 1) * kChunk * (int)sizeof(TIn), c_stride, T, acc);
        if (more) block_coeffs(blk + 1, ch + 1, NCH);
      }
    } else {
      for (int ch = 0; ch < NCH; ++ch) {
        const int s = blk * NCH + ch;
        stream_chunk<TIn, R, TMAX>(gA, chunk_src(min(s + 1, total - 1)), row_step, lds4, lane, c_rsrc,
                                   c_goff + ch * kChunk * (int)sizeof(TIn), c_stride, T, acc);
        if (more) block_coeffs(blk + 1, ch, NCH);
      }
    }
    // this block's coefficients (written during the previous block) are
    // complete, and every wave is past the epilogue whose buffer the next
    // block's coefficients reuse
    __syncthreads();
    block_epilogue(blk);
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------

namespace {

constexpr size_t kLdsCap = 160 * 1024;
constexpr size_t kLdsDenseCap = 80 * 1024;  // two workgroups per CU

// heads that a range of `ch` channels starting at a multiple of `ch` can touch
int heads_of_range(int ch, int P) { return (ch % P == 0) ? ch / P : (P % ch == 0 ? 1 : ch / P + 2); }

template <typename TIn, int R, int TMAX, bool DENSE>
int launch_t(const VerifyArgs& a, const VerifyGeom& geo, size_t lds, hipStream_t s) {
  dim3 grid(a.d.d_in / (geo.NBLK * geo.NW * R * kWave), a.d.Bsz, a.d.L);
  if (allow_lds(verify_proj_kernel<TIn, R, TMAX, DENSE>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  hipLaunchKernelGGL((verify_proj_kernel<TIn, R, TMAX, DENSE>), grid, dim3(geo.NW * kWave), lds, s, a, geo);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

template <int R, int TMAX, bool DENSE>
size_t lds_bytes(VerifyGeom& geo) {
  while (geo.NC > 16 && (size_t)VerifyLds<R, TMAX, DENSE>(geo).total > 72 * 1024) geo.NC /= 2;
  return (size_t)VerifyLds<R, TMAX, DENSE>(geo).total;
}

// Workgroup shape: the most waves whose block stays inside one B/C group,
// then as many blocks per workgroup as keep at least 512 workgroups in the
// grid (the tree prologue is paid once per workgroup) with LDS that fits;
// the dense correction matrix when it fits, the path walk otherwise.
template <typename TIn, int R, int TMAX>
int launch_r(const VerifyArgs& a, hipStream_t s) {
  const int per_group = a.d.d_in / a.d.G;
  const int64_t units = (int64_t)a.d.L * a.d.Bsz;
  for (int nw : {4, 2, 1}) {
    const int BC = nw * R * kWave;
    if (per_group % BC) continue;
    const int nblk_max = per_group / BC;
    for (int nblk = nblk_max; nblk >= 1; --nblk) {
      if (nblk_max % nblk) continue;
      if (nblk > 1 && units * (a.d.d_in / (nblk * BC)) < 512) continue;
      VerifyGeom geo{nw, nblk, heads_of_range(nblk * BC, a.d.P), heads_of_range(BC, a.d.P), a.d.N};
      if constexpr (TMAX <= 32) {
        VerifyGeom gd = geo;
        const size_t lds = lds_bytes<R, TMAX, true>(gd);
        if (lds <= kLdsDenseCap) return launch_t<TIn, R, TMAX, true>(a, gd, lds, s);
      }
      const size_t lds = lds_bytes<R, TMAX, false>(geo);
      if (lds <= kLdsCap) return launch_t<TIn, R, TMAX, false>(a, geo, lds, s);
    }
  }
  return SSM_TREE_E_DIMS;
}

template <typename TIn>
int launch_in(const VerifyArgs& a, hipStream_t s) {
  const int T = a.d.T;
  const bool r2 = (a.d.d_in / a.d.G) % (2 * kWave) == 0;
  if (T <= 32 && r2) {
    const int st = T <= 8 ? launch_r<TIn, 2, 8>(a, s) : T <= 16 ? launch_r<TIn, 2, 16>(a, s) : launch_r<TIn, 2, 32>(a, s);
    if (st != SSM_TREE_E_DIMS) return st;
  }
  if (T <= 8) return launch_r<TIn, 1, 8>(a, s);
  if (T <= 16) return launch_r<TIn, 1, 16>(a, s);
  if (T <= 32) return launch_r<TIn, 1, 32>(a, s);
  return launch_r<TIn, 1, 64>(a, s);
}

}  // namespace

int launch_verify_fifo(const VerifyArgs& a, bool bf16, hipStream_t s);

// SSM_TREE_CONV_XBC and the gate: taken on the fused round's shapes, whose
// kernel then runs with nothing to commit (see ssm_tree_verify).
bool commit_verify_fused_applies(const Dims& d);
bool tt_verify_applies(const Dims& d);
bool tt_verify_fits(const Dims& d, bool bf16, bool opt);
int launch_verify_tt(const VerifyArgs& a, bool bf16, hipStream_t s);

// A bfloat16 root state (SSM_TREE_STATE_BF16) is read by the matrix-core
// kernels only: no FIFO walk, no options.
bool verify_options_supported(const Dims& d, bool gate, bool bf16) {
  if (d.sbf16)
    return d.T == 0 || (!d.fifo && !d.xbc && !gate &&
                        (commit_verify_fused_applies(d) || (tt_verify_applies(d) && tt_verify_fits(d, bf16, false))));
  // the options: trees of 1-16 nodes on the fused round's kernel, 17-64 on
  // the options' instantiation of verify_tt_kernel
  return (!d.xbc && !gate) ||
         (!d.fifo && (commit_verify_fused_applies(d) || (tt_verify_applies(d) && tt_verify_fits(d, bf16, true))));
}

// trees of 1-16 nodes: the round's kernel with nothing to commit (one
// workgroup per 64 channels of a (layer, sequence))
int launch_verify_oneshot(const VerifyArgs& a, bool bf16, hipStream_t s);

int launch_verify(const VerifyArgs& a, bool bf16, hipStream_t s) {
  if (a.d.fifo) return launch_verify_fifo(a, bf16, s);
  if (commit_verify_fused_applies(a.d)) return launch_verify_oneshot(a, bf16, s);
  if (tt_verify_applies(a.d)) {
    const int st = launch_verify_tt(a, bf16, s);
    // E_DIMS: its LDS does not fit this shape, nothing launched (the vector
    // ALU kernel below takes neither the options nor a bf16 state)
    if (st != SSM_TREE_E_DIMS || a.d.sbf16 || a.d.xbc || a.z) return st;
  }
  if (a.d.sbf16) return SSM_TREE_E_DIMS;
  return bf16 ? launch_in<bf16_t>(a, s) : launch_in<float>(a, s);
}

}  // namespace ssmt
