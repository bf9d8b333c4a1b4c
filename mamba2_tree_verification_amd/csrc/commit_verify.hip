// commit_verify.hip - ssm_tree_commit of the last step's accepted path fused
// with ssm_tree_verify of the next tree, in one pass over the root state.
//
// Per (layer, sequence): the root state is read once, advanced along the
// accepted path of the previous tree (SpecMamba page sec. 3.1: recompute
// from the stored per-token dt, B and x; the replay in closed form, a
// decayed state plus rank-4 updates on the matrix cores), written once,
// and the next
// tree's outputs are formed from the new state while it is still in
// registers (the root projection of verify.hip:
//   y_v = a_v (C_v . h) + sum_{u on path(v)} M[v][u] x~_u).
// Results equal ssm_tree_commit followed by ssm_tree_verify on the
// committed state and window, up to fp32 rounding.  A sequence whose commit
// fails (invalid previous tree or path) passes its state and window through
// unchanged to the outputs, and its next tree is verified from them.
//
// Mapping.  One workgroup of 4 waves per (layer, sequence, 64 channels);
// wave w owns channels 16 w .. 16 w + 15.  Lane (j + 16 k) holds columns
// 16 gg + 4 k .. + 3 of channel j for every column group gg, which is both
// a coalesced 16-byte load and the B-operand layout of
// v_mfma_f32_16x16x4_f32, so the committed state feeds C . h on the
// matrix cores directly.
//
// Latency.  A workgroup's life is short (64 KiB of state in and out), so
// the number of dependent trips to memory decides the throughput.  There
// are two: every load that does not depend on the accepted path is issued
// at entry (both trees' parent[], the next tree's x, B, C and dt rows, the
// previous tree's dt rows, window, parameters, and the state last, so that
// waiting for the small rows does not wait for it); the path's x and
// B rows are gathered right after, from the unvalidated path, while one
// wave validates the trees and the path with ballots, one forms C_v . B_u
// and one the next tree's ancestor sets and conv taps.  Everything after
// that runs from LDS.  y is staged in LDS and leaves as whole 256-byte row
// segments.  Trees of at most 16 nodes, heads a multiple of 16 channels
// wide.
#include <string.h>

#include "common.h"

namespace ssmt {

hipError_t launch_window_bc(const WindowBcArgs& a, bool bf16, hipStream_t s);

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCvRows = 64;   // channels per workgroup
constexpr int kCvWaves = 4;
constexpr int kCvT = 16;      // node capacity
constexpr int kBcThreads = 256;  // bc_conv_kernel (one thread per entry of the 16 x 16 C . B table)
constexpr int kBcMaxN = 256;     // d_state bound of its LDS rows
static_assert(kBcThreads == kCvT * kCvT, "C . B table mapping");
// floats of one (sequence, group) block of the xBC workspace: the next
// tree's convolved B and C rows, the path's B rows, the C . B table
__host__ __device__ constexpr int bc_block_floats(int T, int N) { return T * 3 * N + kCvT * kCvT; }
constexpr int kRowPad = 16;   // bytes of padding per staged B / C row (LDS banks)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// 16x16x32 bf16 products, fp32 accumulate; the operands as raw bits
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TIn>
__device__ __forceinline__ f32x4 load4(const TIn* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  f32x4 r;
  r.x = __uint_as_float(w.x << 16);
  r.y = __uint_as_float(w.x & 0xFFFF0000u);
  r.z = __uint_as_float(w.y << 16);
  r.w = __uint_as_float(w.y & 0xFFFF0000u);
  return r;
}

// four consecutive input elements as raw bits
template <int E>
struct Raw4;
template <>
struct Raw4<2> {
  typedef u32x2 T;
};
template <>
struct Raw4<4> {
  typedef u32x4 T;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// LDS layout (byte offsets).  ys reuses the x staging of both trees, which
// is dead once the conv outputs exist; dtx reuses the next tree's B rows,
// dead once C . B is formed.
// Heads a 64-channel slab touches (P a multiple of 16): one when P is a
// multiple of 64, four at P = 16, otherwise at most two.
__host__ __device__ constexpr int slab_heads(int P) { return P % 64 == 0 ? 1 : (P == 16 ? 4 : 2); }

struct CvLds {
  int pparent, path, parent, misc, anc, cidx, dAp, dtp, dt, S, Sd, av, Mt, D, cbt, cw, cb, win, xn, xp, ys, C, B, dtx,
      Bp, xt, total, row;
  // the options' own arrays (offset 0 when unused)
  int z, Bpt;
  // vo: verify only (nothing committed: no previous tree's rows)
  __host__ __device__ CvLds(int N, int E, int P, bool xbc = false, bool gate = false, bool vo = false) {
    int o = 0;
    row = N * E + kRowPad;                    // staged B / C row stride
    pparent = o; o += 4 * kCvT;
    path = o; o += 4 * kCvT;
    parent = o; o += 4 * kCvT;
    misc = o; o += 16;                        // [0] path length applied, [1] commit status, [2] next tree ok, [3] raw length
    anc = o; o += 4 * kCvT;                   // next tree: root-path bitmask per node
    cidx = o; o += 4 * kCvT;                  // next tree: conv inputs of taps 1..3 (node, or T + window row)
    dAp = o; o += 4 * kCvT * 4;               // previous tree: dA per node and head
    dtp = o; o += 4 * kCvT * 4;               // previous tree: dt per node and head
    dt = o; o += 4 * 4 * kCvT;                // next tree: dt per head and node
    S = o; o += 4 * 4 * kCvT;                 // next tree: dt * A per head and node
    Sd = o; o += 8 * 4 * kCvT;                // next tree: S_v = sum of dt * A over the root path, float64
    av = o; o += 4 * 4 * kCvT;                // next tree: a_v = exp(S_v) per head and node
    Mt = o; o += 4 * slab_heads(P) * kCvT * kCvT;  // next tree: exp(S_v - S_u) dt_u, u on v's root path, else 0
    D = o; o += 16;
    cbt = o; o += xbc ? 0 : 4 * kCvT * kCvT;  // next tree: C_v . B_u (with the xBC conv, in the workspace)
    cw = o; o += 4 * 4 * kCvRows;             // conv weights per channel, tap order of the parameters
    cb = o; o += 4 * kCvRows;                 // conv bias per channel
    win = o; o += align16(3 * kCvRows * E);   // old window rows (raw)
    xn = o; o += kCvT * kCvRows * E;          // next tree x (raw)
    // previous tree x of the path nodes (raw); with bf16 inputs it also backs
    // the second half of the y staging, so verify-only keeps it then
    xp = o; o += (vo && E == 4) ? 0 : kCvT * kCvRows * E;
    ys = xn;                                  // y staging [node][channel] fp32 (4 KiB: xn, then xp or C)
    C = o; o += kCvT * row;                   // next tree C rows (raw, padded)
    B = o;                                    // next tree B rows (raw, padded) ...
    dtx = o;                                  // ... then dt * x~ per path node and channel, fp32
    o += kCvT * row > 4 * kCvT * kCvRows ? kCvT * row : 4 * kCvT * kCvRows;
    Bp = o; o += vo ? 0 : kCvT * row;         // previous tree B rows of the path nodes (raw, padded)
    xt = o; o += 4 * kCvRows * kCvT;          // next tree conv outputs, MFMA B-operand layout
    z = Bpt = 0;
    if (gate && !xbc) { z = o; o += kCvT * kCvRows * E; }  // gate input rows (raw)
    if (xbc) {
      // The raw B and C rows of both trees are not read (the next tree's
      // convolved rows go from the workspace to the registers of the lanes
      // that take them): dt * x~ takes the C rows' place, and the path's
      // convolved B rows (fp32, from the workspace) follow it over the B
      // and Bp rows, which always have room for them.
      dtx = C;
      Bpt = C + 4 * kCvT * kCvRows;
      // the gate rows arrive after the commit, over the same space (dead by
      // then; it is never smaller than 4 KiB)
      if (gate) z = C;
    }
    total = o;
  }
};

}  // namespace

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool finite4(f32x4 v) {
  return __builtin_isfinite(v.x) && __builtin_isfinite(v.y) && __builtin_isfinite(v.z) && __builtin_isfinite(v.w);
}

// OPT: an instantiation of its own for the Mamba2-convention options (the
// xBC conv, the gate), so that the plain path keeps its registers and LDS.
// VO: verify only (ssm_tree_verify): no previous tree, nothing committed,
// no state or window written.
// (verify only with bf16 inputs holds 7 waves per SIMD: its LDS leaves room
// for 7 workgroups per CU; the options' instance with bf16 inputs and
// d_state 128 is held to 6, which its registers allow without spilling)
template <typename TIn, typename TS, int NG, bool OPT, bool VO>
__global__ void __launch_bounds__(kCvWaves * kWave)
    __attribute__((amdgpu_waves_per_eu(VO && sizeof(TIn) == 2 && NG <= 8 ? 7 : (OPT && sizeof(TIn) == 2 && NG == 8 ? 6 : 1)))) commit_verify_kernel(CommitVerifyArgs a) {
  typedef StateQuad<TS> SQ;
  constexpr int N = 16 * NG;
  constexpr int E = (int)sizeof(TIn);
  typedef typename Raw4<E>::T RawQ;
  constexpr int kChunks = N * E / 16;                           // 16-byte chunks per B / C row
  constexpr int kCPT = (kCvT * kChunks + kCvWaves * kWave - 1) / (kCvWaves * kWave);  // chunks per thread
  const Dims d = a.d;
  const int T = d.T, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane & 15, k = lane >> 4;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int c0 = blockIdx.x * kCvRows;
  const int h_lo = c0 / P;
  const int HW = (c0 + kCvRows - 1) / P - h_lo + 1;  // heads touched (<= 4: P is a multiple of 16)
  const int g = c0 / (DI / G);
  const int CH = d.CH;  // conv channels = window row length
  const bool xbc = OPT && d.xbc, gate = OPT && a.z != nullptr;

  extern __shared__ __align__(16) unsigned char smem[];
  const CvLds lo(N, E, P, xbc, gate, VO);
  int32_t* s_pparent = reinterpret_cast<int32_t*>(smem + lo.pparent);
  int32_t* s_path = reinterpret_cast<int32_t*>(smem + lo.path);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  int32_t* s_misc = reinterpret_cast<int32_t*>(smem + lo.misc);
  int32_t* s_anc = reinterpret_cast<int32_t*>(smem + lo.anc);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);
  float* s_dAp = reinterpret_cast<float*>(smem + lo.dAp);
  float* s_dtp = reinterpret_cast<float*>(smem + lo.dtp);
  float* s_dt = reinterpret_cast<float*>(smem + lo.dt);
  float* s_S = reinterpret_cast<float*>(smem + lo.S);
  double* s_Sd = reinterpret_cast<double*>(smem + lo.Sd);
  float* s_a = reinterpret_cast<float*>(smem + lo.av);
  float* s_Mt = reinterpret_cast<float*>(smem + lo.Mt);
  float* s_D = reinterpret_cast<float*>(smem + lo.D);
  float* s_cbt = reinterpret_cast<float*>(smem + lo.cbt);
  float* s_cw = reinterpret_cast<float*>(smem + lo.cw);
  float* s_cb = reinterpret_cast<float*>(smem + lo.cb);
  TIn* s_win = reinterpret_cast<TIn*>(smem + lo.win);
  TIn* s_xn = reinterpret_cast<TIn*>(smem + lo.xn);
  TIn* s_xp = reinterpret_cast<TIn*>(smem + lo.xp);
  float* s_ys = reinterpret_cast<float*>(smem + lo.ys);
  unsigned char* s_C = smem + lo.C;
  unsigned char* s_B = smem + lo.B;
  float* s_dtx = reinterpret_cast<float*>(smem + lo.dtx);
  unsigned char* s_Bp = smem + lo.Bp;
  float* s_xt = reinterpret_cast<float*>(smem + lo.xt);
  const int rs = lo.row;
  TIn* s_z = reinterpret_cast<TIn*>(smem + lo.z);
  float* s_Bpt = reinterpret_cast<float*>(smem + lo.Bpt);
  // SSM_TREE_CONV_XBC: the group's convolved rows, [T][2 N] of the next tree
  // (B then C) and [T][N] of the path, formed ahead of this kernel
  const float* bcw_n = xbc ? a.bcw + (unit * G + g) * (int64_t)bc_block_floats(T, N) : nullptr;
  const float* bcw_p = xbc ? bcw_n + (int64_t)T * 2 * N : nullptr;
  const float* bcw_cb = xbc ? bcw_p + (int64_t)T * N : nullptr;

  // ======== trip 1: everything that does not depend on the path ========

  int r_pp = 0, r_path = 0, r_par = 0, r_len = 0;
  if (tid < T) {
    if constexpr (!VO) {
      r_pp = a.parent_prev[(int64_t)b * T + tid];
      r_path = a.path[(int64_t)b * T + tid];
    }
    r_par = a.parent[(int64_t)b * T + tid];
  }
  // verify-only use (the options of ssm_tree_verify): no path length means
  // nothing to commit, and no state or window output is written
  if (tid == kCvWaves * kWave - 1) r_len = (!VO && (!OPT || a.path_len)) ? a.path_len[b] : 0;

  // x rows: thread (v, q) holds channels 4 q .. 4 q + 3 of node v
  const int xv = tid >> 4, xq = (tid & 15) * 4;
  RawQ rx{};
  if (xv < T)
    rx = *reinterpret_cast<const RawQ*>(reinterpret_cast<const TIn*>(a.x) + (unit * T + xv) * DI + c0 + xq);
  // B and C rows of the next tree, 16-byte chunks
  u32x4 rc[kCPT], rb[kCPT];
  const unsigned char* Cg = reinterpret_cast<const unsigned char*>(a.C) + ((unit * T) * G + g) * (int64_t)N * E;
  const unsigned char* Bg = reinterpret_cast<const unsigned char*>(a.B) + ((unit * T) * G + g) * (int64_t)N * E;
#pragma unroll
  for (int it = 0; it < kCPT; ++it) {
    const int ci = tid + it * kCvWaves * kWave, v = ci / kChunks, q = ci % kChunks;
    if (v < T && !xbc) {
      rc[it] = *reinterpret_cast<const u32x4*>(Cg + (int64_t)v * G * N * E + q * 16);
      rb[it] = *reinterpret_cast<const u32x4*>(Bg + (int64_t)v * G * N * E + q * 16);
    }
  }
  // per-head scalars: wave 0 the next tree's dt, wave 1 the previous tree's
  const int sv = (lane >> 2), sh = lane & 3;
  // dt_raw as raw bits, widened only after the state loads are out (a
  // conversion here would make waves 0 and 1 wait for it first)
  uint32_t r_dt = 0;
  float r_A = 0.0f, r_bias = 0.0f, r_D = 0.0f;
  if ((wave == 0 || (!VO && wave == 1)) && sv < T && sh < HW) {
    const int64_t di = unit * T * H + (int64_t)sv * H + h_lo + sh;
    const void* src = wave == 0 ? a.dt_raw : a.dt_prev;
    r_dt = E == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(src)[di] : reinterpret_cast<const uint32_t*>(src)[di];
    r_A = a.prm.A[(int64_t)l * H + h_lo + sh];
    r_bias = a.prm.dt_bias[(int64_t)l * H + h_lo + sh];
  }
  if (wave == 0 && lane < HW) r_D = a.prm.D[(int64_t)l * H + h_lo + lane];
  // wave 2: old window rows; wave 3: conv weights and bias
  TIn r_win[3];
  float r_cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, r_cb = 0.0f;
  if (wave == 2) {
    const TIn* win_in = reinterpret_cast<const TIn*>(a.window_in) + unit * (W - 1) * (int64_t)CH + c0 + lane;
#pragma unroll
    for (int r = 0; r < 3; ++r)
      if (r < W - 1) r_win[r] = win_in[(int64_t)r * CH];
  } else if (wave == 3) {
    const float* cw = a.prm.conv_w + ((int64_t)l * CH + c0 + lane) * W;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (jj < W) r_cw[jj] = cw[jj];
    if (a.prm.conv_b) r_cb = a.prm.conv_b[(int64_t)l * CH + c0 + lane];
  }
  // the options: gate rows
  RawQ rz{};
  if constexpr (OPT) {
    if (gate && !xbc && xv < T)
      rz = *reinterpret_cast<const RawQ*>(reinterpret_cast<const TIn*>(a.z) + (unit * T + xv) * DI + c0 + xq);
  }

  // the state last: the small rows above reach LDS while it is still in flight
  // (loads complete in issue order)
  // Columns of quad gg in lane j + 16 k: 16 gg + 4 k .. + 3, or with a bf16
  // state (and an even number of column groups) 32 (gg / 2) + 8 k + 4 (gg % 2)
  // .. + 3, so that a pair of quads is 8 consecutive columns and the state
  // moves in 16-byte accesses.  C, B and the state take the same columns of
  // a lane (the contractions only need them to agree).
  constexpr bool kWide = sizeof(TS) == 2 && NG % 2 == 0 && !OPT;
  auto colq = [&](int gg) { return kWide ? 32 * (gg >> 1) + 8 * k + 4 * (gg & 1) : 16 * gg + 4 * k; };
  const TS* sin = reinterpret_cast<const TS*>(a.state_in) + (unit * DI + c0 + wave * 16 + j) * (int64_t)N;
  typename SQ::Raw hraw[NG];
  // A float32 state moves in whole 128-byte lines: per pair of column groups
  // p a wave loads its 16 rows with two instructions, lane (8 r + c) taking
  // the 16-byte chunk c of columns 32 p .. 32 p + 31 of row r (and of row
  // 8 + r), non-temporal (streamed past the caches) like commit_kernel's.
  // The quads change to the operand layout through LDS before the commit.
  // (Half a line per row per instruction, the operand layout, streams the
  // state about a fifth slower in the round.  Verify only reads the state,
  // and there the change of layout cost more than it saved.)
  constexpr bool kCoal = sizeof(TS) == 4 && NG % 2 == 0 && !VO;
  const int lr = lane >> 3, lc = lane & 7;  // row within eight, chunk of the 128-byte line
  const TS* sinw = reinterpret_cast<const TS*>(a.state_in) + (unit * DI + c0 + wave * 16) * (int64_t)N;
  if constexpr (kCoal) {
#pragma unroll
    for (int pp = 0; pp < NG / 2; ++pp) {
      hraw[2 * pp] = SQ::load_nt(sinw + lr * N + 32 * pp + 4 * lc);
      hraw[2 * pp + 1] = SQ::load_nt(sinw + (8 + lr) * N + 32 * pp + 4 * lc);
    }
  } else if constexpr (kWide) {
#pragma unroll
    for (int gp = 0; gp < NG / 2; ++gp) {
      const u32x4* src = reinterpret_cast<const u32x4*>(sin + colq(2 * gp));
      const u32x4 w = VO ? __builtin_nontemporal_load(src) : *src;
      hraw[2 * gp] = u32x2{w.x, w.y};
      hraw[2 * gp + 1] = u32x2{w.z, w.w};
    }
  } else {
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) hraw[gg] = VO ? SQ::load_nt(sin + colq(gg)) : SQ::load(sin + colq(gg));
  }
  asm volatile("" : "+v"(r_dt));  // (keeps dt_raw's widening below the state loads)

  // to LDS
  if (tid < T) {
    if constexpr (!VO) {
      s_pparent[tid] = r_pp;
      s_path[tid] = r_path;
    }
    s_parent[tid] = r_par;
  }
  if (tid == kCvWaves * kWave - 1) s_misc[3] = r_len;
  if (xv < T) *reinterpret_cast<RawQ*>(s_xn + xv * kCvRows + xq) = rx;
#pragma unroll
  for (int it = 0; it < kCPT; ++it) {
    const int ci = tid + it * kCvWaves * kWave, v = ci / kChunks, q = ci % kChunks;
    if (v < T && !xbc) {
      *reinterpret_cast<u32x4*>(s_C + v * rs + q * 16) = rc[it];
      *reinterpret_cast<u32x4*>(s_B + v * rs + q * 16) = rb[it];
    }
  }
  if ((wave == 0 || (!VO && wave == 1)) && sv < T && sh < HW) {
    const float dt = softplus_f32(__uint_as_float(E == 2 ? r_dt << 16 : r_dt) + r_bias);
    if (wave == 0) {
      s_dt[sh * kCvT + sv] = dt;
      s_S[sh * kCvT + sv] = dt * r_A;
    } else {
      s_dtp[sv * 4 + sh] = dt;
      s_dAp[sv * 4 + sh] = expf(dt * r_A);
    }
  }
  if (wave == 0 && lane < HW) s_D[lane] = r_D;
  if (wave == 2) {
#pragma unroll
    for (int r = 0; r < 3; ++r)
      if (r < W - 1) s_win[r * kCvRows + lane] = r_win[r];
  } else if (wave == 3) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) s_cw[lane * 4 + jj] = r_cw[jj];
    s_cb[lane] = r_cb;
  }
  if constexpr (OPT) {
    if (gate && !xbc && xv < T) *reinterpret_cast<RawQ*>(s_z + xv * kCvRows + xq) = rz;
  }
  __syncthreads();

  // ======== trip 2: the path's x and B rows, gathered before validation ========
  const int len_raw = s_misc[3];
  const int lg = len_raw < 0 ? 0 : (len_raw > T ? T : len_raw);
  RawQ rxp{};
  if (xv < lg) {
    const int v = s_path[xv];
    const int vs = (v >= 0 && v < T) ? v : 0;  // an invalid path is discarded below
    rxp = *reinterpret_cast<const RawQ*>(reinterpret_cast<const TIn*>(a.x_prev) + (unit * T + vs) * DI + c0 + xq);
  }
  u32x4 rbp[kCPT];
  const unsigned char* Bpg = reinterpret_cast<const unsigned char*>(a.B_prev) + ((unit * T) * G + g) * (int64_t)N * E;
#pragma unroll
  for (int it = 0; it < kCPT; ++it) {
    const int ci = tid + it * kCvWaves * kWave, q = ci / kChunks, ch = ci % kChunks;
    if (q < lg && !xbc) {
      const int v = s_path[q];
      const int vs = (v >= 0 && v < T) ? v : 0;
      rbp[it] = *reinterpret_cast<const u32x4*>(Bpg + (int64_t)vs * G * N * E + ch * 16);
    }
  }
  // with the xBC conv: the path's convolved B rows (positions past a failed
  // commit's length 0 are loaded but never read)
  constexpr int kQPT = (kCvT * N / 4 + kCvWaves * kWave - 1) / (kCvWaves * kWave);
  f32x4 rbq[OPT ? kQPT : 1];
  if constexpr (OPT) {
#pragma unroll
    for (int it = 0; it < kQPT; ++it) {
      const int ci = tid + it * kCvWaves * kWave;
      if (xbc && ci < lg * (N / 4)) rbq[it] = *reinterpret_cast<const f32x4*>(bcw_p + 4 * ci);
    }
  }

  if (wave == 0) {
    // both trees and the path, by ballot
    bool bad_p = false, bad_n = false, bad_path = false;
    if (lane < T) {
      int p;
      if constexpr (!VO) {
        p = s_pparent[lane];
        bad_p = lane == 0 ? p != -1 : (p < -1 || p >= lane || p < s_pparent[lane - 1]);
      }
      p = s_parent[lane];
      bad_n = lane == 0 ? p != -1 : (p < -1 || p >= lane || p < s_parent[lane - 1]);
    }
    if (lane < lg) {
      const int v = s_path[lane];
      bad_path = v < 0 || v >= T || s_pparent[v] != (lane == 0 ? -1 : s_path[lane - 1]);
    }
    const bool prev_ok = __ballot(bad_p) == 0, tree_ok = __ballot(bad_n) == 0;
    const bool path_ok = len_raw >= 0 && len_raw <= T && __ballot(bad_path) == 0;
    const int st = !prev_ok ? SSM_TREE_E_TREE : (!path_ok ? SSM_TREE_E_PATH : SSM_TREE_OK);
    if (lane == 0) {
      s_misc[0] = st == SSM_TREE_OK ? len_raw : 0;
      s_misc[1] = st;
      s_misc[2] = tree_ok ? 1 : 0;
      if (blockIdx.x == 0 && l == 0) {
        if (!VO && a.commit_status) a.commit_status[b] = st;
        if (a.verify_status) a.verify_status[b] = tree_ok ? SSM_TREE_OK : SSM_TREE_E_TREE;
      }
    }
  } else if (wave == 1 && !xbc) {
    // C_v . B_u of the next tree: lane (u + 16 q) ends with CB[4 q + r][u]
    // (with the xBC conv the table is in the workspace)
    f32x4 cbm = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool live = j < T;
    if constexpr (E == 2) {
      // bf16 rows are exact bf16 operands: one 16x16x32 product per pair
      // of column groups
      const TIn* cr = reinterpret_cast<const TIn*>(s_C + j * rs) + 4 * k;
      const TIn* br = reinterpret_cast<const TIn*>(s_B + j * rs) + 4 * k;
#pragma unroll
      for (int gp = 0; gp < (NG + 1) / 2; ++gp) {
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(cr + 32 * gp);
        const u32x2 b0 = *reinterpret_cast<const u32x2*>(br + 32 * gp);
        const u32x2 c1 = 2 * gp + 1 < NG ? *reinterpret_cast<const u32x2*>(cr + 32 * gp + 16) : u32x2{0u, 0u};
        const u32x2 b1 = 2 * gp + 1 < NG ? *reinterpret_cast<const u32x2*>(br + 32 * gp + 16) : u32x2{0u, 0u};
        u32x4 ca = u32x4{c0.x, c0.y, c1.x, c1.y};
        if (!live) ca = u32x4{0u, 0u, 0u, 0u};
        cbm = mfma32(ca, u32x4{b0.x, b0.y, b1.x, b1.y}, cbm);
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        f32x4 cq = load4<TIn>(reinterpret_cast<const TIn*>(s_C + j * rs) + 16 * gg + 4 * k);
        f32x4 bq = load4<TIn>(reinterpret_cast<const TIn*>(s_B + j * rs) + 16 * gg + 4 * k);
        if (!live) cq = bq = f32x4{0.f, 0.f, 0.f, 0.f};
        cbm = mfma4(cq.x, bq.x, cbm);
        cbm = mfma4(cq.y, bq.y, cbm);
        cbm = mfma4(cq.z, bq.z, cbm);
        cbm = mfma4(cq.w, bq.w, cbm);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) s_cbt[(4 * k + r) * kCvT + j] = cbm[r];
  } else if (wave == 2) {
    // next tree: root-path set and conv inputs.  Every step requires
    // -1 <= parent < node, so the walks end and stay in range even on an
    // invalid tree (whose outputs are discarded).
    if (lane < kCvT) {
      int m = 0, packed = 0;
      if (lane < T) {
        int u = lane, a1 = -1, a2 = -1, a3 = -1;  // ancestors 1, 2, 3
        int depth = 0;                            // nodes on the root path
        for (int s = 0; s < kCvT && u >= 0; ++s) {
          m |= 1 << u;
          ++depth;
          const int p = s_parent[u];
          u = (p >= 0 && p < u) ? p : -1;
          a1 = s == 0 ? u : a1;
          a2 = s == 1 ? u : a2;
          a3 = s == 2 ? u : a3;
        }
        // tap jj reads ancestor jj, or past the root window row W - 2 - (jj - depth)
#pragma unroll
        for (int jj = 1; jj < 4; ++jj) {
          const int an = jj == 1 ? a1 : (jj == 2 ? a2 : a3);
          const int code = an >= 0 ? an : T + (W - 2) - (jj - depth);
          if (jj < W) packed |= code << (8 * (jj - 1));
        }
      }
      s_anc[lane] = m;
      s_cidx[lane] = packed;
    }
    wave_sync();
    // then the decay table, while the state is still in flight
    // lane (head hh, node v): S_v = sum of dt * A over v's root path, in
    // float64, then a_v = exp(S_v) and row v of the decay table,
    // exp(S_v - S_u) dt_u for u on v's root path and 0 elsewhere.  The
    // differences are taken in float64: on a deep path with large steps
    // S_v and S_u are large and close, and a float32 difference would lose
    // the digits that matter (the float64 sums of the same float32 terms
    // cancel exactly, leaving the terms between u and v).
    const int hh = lane >> 4, v = lane & 15;
    const int m = s_anc[v];
    double S = 0.0;
    if (hh < HW) {
#pragma unroll 4
      for (int u = 0; u < kCvT; ++u) S += ((m >> u) & 1) ? (double)s_S[hh * kCvT + u] : 0.0;
      s_Sd[hh * kCvT + v] = S;
    }
    wave_sync();
    if (hh < HW) {
      constexpr double kLog2e = 1.4426950408889634;
      s_a[hh * kCvT + v] = __builtin_amdgcn_exp2f((float)(S * kLog2e));
      float* mt = s_Mt + (hh * kCvT + v) * kCvT;
      // (one quad at a time: the state of the whole workgroup is in flight in
      // registers meanwhile)
#pragma unroll 1
      for (int u4 = 0; u4 < kCvT / 4; ++u4) {
        f32x4 q;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int u = 4 * u4 + t;
          q[t] = ((m >> u) & 1)
                     ? __builtin_amdgcn_exp2f((float)((S - s_Sd[hh * kCvT + u]) * kLog2e)) * s_dt[hh * kCvT + u]
                     : 0.0f;
        }
        *reinterpret_cast<f32x4*>(mt + 4 * u4) = q;
      }
    }
  }
  if (xv < lg) *reinterpret_cast<RawQ*>(s_xp + xv * kCvRows + xq) = rxp;
#pragma unroll
  for (int it = 0; it < kCPT; ++it) {
    const int ci = tid + it * kCvWaves * kWave, q = ci / kChunks, ch = ci % kChunks;
    if (q < lg && !xbc) *reinterpret_cast<u32x4*>(s_Bp + q * rs + ch * 16) = rbp[it];
  }
  if constexpr (OPT) {
#pragma unroll
    for (int it = 0; it < kQPT; ++it) {
      const int ci = tid + it * kCvWaves * kWave;
      if (xbc && ci < lg * (N / 4)) *reinterpret_cast<f32x4*>(s_Bpt + 4 * ci) = rbq[it];
    }
  }
  __syncthreads();

  // ======== from LDS: the path's conv and the new window; the next tree's
  // S and conv outputs ========
  const int len = s_misc[0];  // 0 when the commit fails: state and window pass through unchanged
  // conv weights of channel `lane` by taps back (0 = the token itself)
  float wx[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) wx[jj] = jj < W ? s_cw[lane * 4 + W - 1 - jj] : 0.0f;
  const float cbias = s_cb[lane];
  // the path's conv: its inputs are raw rows only, so its positions are
  // independent; wave w takes positions q = w, w + 4, ... (lane = channel).
  // Tap jj of position q reads element q + W - 1 - jj of (old window rows,
  // path x rows).
  {
    const int hh = (c0 + lane) / P - h_lo;
    for (int q = wave; q < len; q += kCvWaves) {
      const float xv = load_in(s_xp, q * kCvRows + lane);
      float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        if (jj < W) {
          const int e = q + W - 1 - jj;
          u[jj] = e < W - 1 ? load_in(s_win, e * kCvRows + lane) : load_in(s_xp, (e - (W - 1)) * kCvRows + lane);
        }
      }
      float z = fmaf(wx[0], xv, cbias);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj)
        if (jj < W) z = fmaf(wx[jj], u[jj], z);
      const float xt = d.silu ? silu_fast(z) : z;
      s_dtx[q * kCvRows + lane] = s_dtp[s_path[q] * 4 + hh] * xt;
    }
  }
  if (wave == 0) {
    const int c = c0 + lane;
    // new window row r (oldest first) = element len + r of (old window, path x), bit for bit
    if (!VO && W > 1 && (!OPT || a.window_out)) {
      TIn* win_out = reinterpret_cast<TIn*>(a.window_out) + unit * (W - 1) * (int64_t)CH + c;
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        if (r < W - 1) {
          const int e = len + r;
          win_out[(int64_t)r * CH] = e < W - 1 ? s_win[e * kCvRows + lane] : s_xp[(e - (W - 1)) * kCvRows + lane];
        }
      }
    }
  }
  // the next tree's conv outputs: thread (wave, lane) takes channel lane of
  // nodes wave, wave + 4, wave + 8, wave + 12 (each node uniform in its
  // wave, so its tap sources are resolved once)
  static_assert(kCvT == 4 * kCvWaves && kCvRows == kWave, "x~ mapping");
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int v = wave + kCvWaves * it;
    float xt = 0.0f;
    if (v < T) {
      const int codes = s_cidx[v];
      float u[4];
      u[0] = load_in(s_xn, v * kCvRows + lane);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        u[jj] = 0.0f;
        if (jj < W) {
          const int code = (codes >> (8 * (jj - 1))) & 255;
          const TIn* src;
          if (code < T) {
            src = s_xn + code * kCvRows;
          } else {  // committed window row code - T
            const int e = len + code - T;
            src = e < W - 1 ? s_win + e * kCvRows : s_xp + (e - (W - 1)) * kCvRows;
          }
          u[jj] = load_in(src, lane);
        }
      }
      float z = fmaf(wx[0], u[0], cbias);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj)
        if (jj < W) z = fmaf(wx[jj], u[jj], z);
      xt = d.silu ? silu_fast(z) : z;
    }
    // MFMA B-operand layout: channel row lane, quad v / 4 swizzled
    s_xt[lane * kCvT + 4 * ((v >> 2) ^ ((lane >> 2) & 3)) + (v & 3)] = xt;
  }
  __syncthreads();

  // ======== commit along the path, new state, next tree's y ========
  {
    const int row = wave * 16 + j;
    const int hh = (c0 + wave * 16) / P - h_lo;  // the wave's head (P is a multiple of 16)
    f32x4 hq[NG];
    // the wave's 1 KiB for the state's change of layout: the next tree's and
    // the path's x rows are dead here (the y staging takes them back after a
    // barrier), [row 0..15][16-byte chunk 0..3] of one column group
    f32x4* s_tw = reinterpret_cast<f32x4*>(smem + lo.xn) + wave * 64;
    if constexpr (kCoal) {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        if ((lc >> 2) == (gg & 1)) {
          s_tw[lr * 4 + (lc & 3)] = hraw[gg & ~1];
          s_tw[(8 + lr) * 4 + (lc & 3)] = hraw[gg | 1];
        }
        wave_sync();
        hq[gg] = s_tw[j * 4 + k];
        wave_sync();
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) hq[gg] = SQ::to_f32(hraw[gg]);
    }
    if (!VO && len > 0) {
      // the replay along the path in closed form: with a_q = exp(dt_q A)
      // and c_q = a_{q+1} ... a_{len-1},
      //   h_new = (a_0 ... a_{len-1}) h + sum_q c_q (dt_q x~_q) B_q,
      // the sum as rank-4 updates on the matrix cores: the state quads are
      // the accumulator (lane j + 16 k, element t: row 4 k + t of the tile
      // whose columns are channels), A = the path's B rows (lane j + 16 k
      // brings B_{s4+k} at the column of row j), B = c_q dt_q x~_q of
      // channel j.  Lane q < len forms c_q.
      float cl = 1.0f;
      for (int i = len - 1; i > lane; --i) cl *= s_dAp[s_path[i] * 4 + hh];
      const float a_all = __shfl(cl, 0) * s_dAp[s_path[0] * 4 + hh];
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) hq[gg] *= a_all;
      // column of tile row m in quad gg (the state quads' own columns)
      auto colrow = [&](int gg, int m) {
        return kWide ? 32 * (gg >> 1) + 8 * (m >> 2) + 4 * (gg & 1) + (m & 3) : 16 * gg + m;
      };
      for (int s4 = 0; s4 < len; s4 += 4) {
        const int q = s4 + k;
        const bool on = q < len;
        const float cq = __shfl(cl, q);
        const float wv = on ? cq * s_dtx[q * kCvRows + row] : 0.0f;
        const TIn* bp = reinterpret_cast<const TIn*>(s_Bp + (on ? q : 0) * rs);
        const float* bpt = s_Bpt + (on ? q : 0) * N;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const int col = colrow(gg, j);
          const float av = on ? (xbc ? bpt[col] : load_in(bp, col)) : 0.0f;
          hq[gg] = mfma4(av, wv, hq[gg]);
        }
      }
    }
    // the committed state as stored (a bfloat16 state is rounded): the
    // next tree is verified from exactly what the two-call round would read
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      hraw[gg] = SQ::from_f32(hq[gg]);
      hq[gg] = SQ::to_f32(hraw[gg]);
    }
    if (!VO && (!OPT || a.state_out)) {
      TS* so = reinterpret_cast<TS*>(a.state_out) + (unit * DI + c0 + row) * (int64_t)N;
      if constexpr (kCoal) {
        // back to whole lines through the same LDS, non-temporal
        TS* sow = reinterpret_cast<TS*>(a.state_out) + (unit * DI + c0 + wave * 16) * (int64_t)N;
#pragma unroll
        for (int pp = 0; pp < NG / 2; ++pp) {
          f32x4 oa = f32x4{0.f, 0.f, 0.f, 0.f}, ob = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            s_tw[j * 4 + k] = hq[2 * pp + hs];
            wave_sync();
            if ((lc >> 2) == hs) {
              oa = s_tw[lr * 4 + (lc & 3)];
              ob = s_tw[(8 + lr) * 4 + (lc & 3)];
            }
            wave_sync();
          }
          SQ::store_nt(sow + lr * N + 32 * pp + 4 * lc, oa);
          SQ::store_nt(sow + (8 + lr) * N + 32 * pp + 4 * lc, ob);
        }
      } else if constexpr (kWide) {
#pragma unroll
        for (int gp = 0; gp < NG / 2; ++gp)
          *reinterpret_cast<u32x4*>(so + colq(2 * gp)) =
              u32x4{hraw[2 * gp].x, hraw[2 * gp].y, hraw[2 * gp + 1].x, hraw[2 * gp + 1].y};
      } else {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) SQ::store(so + colq(gg), hraw[gg]);
      }
    }

    // with the xBC conv the gate rows are loaded now, under the products,
    // and staged after the commit's arrays are done with (thread (v, q) as
    // in trip 1)
    const int zv = tid >> 4, zq = (tid & 15) * 4;  // (= xv, xq)
    RawQ rzl{};
    if constexpr (OPT) {
      if (xbc && gate && zv < T)
        rzl = *reinterpret_cast<const RawQ*>(reinterpret_cast<const TIn*>(a.z) + (unit * T + zv) * DI + c0 + zq);
    }
    // C . h on the matrix cores: lane (c + 16 q) ends with (C_{4q+r} . h_c)
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool live = j < T;
    // with the xBC conv, node j's convolved C row (node 0's for the lanes
    // past the tree, whose products are zeroed), and the C . B table
    // (C_v . B_u at [v][u]) in the workspace instead of LDS
    const float* ccj = OPT && xbc ? bcw_n + (live ? j : 0) * 2 * N + N : nullptr;
    const float* cbt = OPT && xbc ? bcw_cb : s_cbt;
    const f32x4 cbr = *reinterpret_cast<const f32x4*>(cbt + j * kCvT + 4 * k);
    // bf16 C rows and a bf16 state are exact bf16 operands: one 16x16x32
    // product per pair of column groups (lane j + 16 k feeds columns
    // 16 gg + 4 k .. + 3 of both groups, the same slots in C and in h)
    constexpr bool kBf16Ch = E == 2 && sizeof(TS) == 2 && !OPT;
    if constexpr (kBf16Ch) {
#pragma unroll
      for (int gp = 0; gp < (NG + 1) / 2; ++gp) {
        const TIn* cq0 = reinterpret_cast<const TIn*>(s_C + j * rs);
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(cq0 + colq(2 * gp));
        const u32x2 c1 = 2 * gp + 1 < NG ? *reinterpret_cast<const u32x2*>(cq0 + colq((2 * gp + 1) % NG)) : u32x2{0u, 0u};
        const u32x2 h0 = hraw[2 * gp];
        const u32x2 h1 = 2 * gp + 1 < NG ? hraw[(2 * gp + 1) % NG] : u32x2{0u, 0u};
        u32x4 ca = u32x4{c0.x, c0.y, c1.x, c1.y};
        if (!live) ca = u32x4{0u, 0u, 0u, 0u};
        acc = mfma32(ca, u32x4{h0.x, h0.y, h1.x, h1.y}, acc);
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        f32x4 cq;
        if constexpr (OPT) {
          if (xbc) {
            // the convolved C values of node j, columns 16 gg + 4 k .. + 3
            cq = *reinterpret_cast<const f32x4*>(ccj + 16 * gg + 4 * k);
          } else {
            cq = load4<TIn>(reinterpret_cast<const TIn*>(s_C + j * rs) + colq(gg));
          }
        } else {
          cq = load4<TIn>(reinterpret_cast<const TIn*>(s_C + j * rs) + colq(gg));
        }
        if (!live) cq = f32x4{0.f, 0.f, 0.f, 0.f};
        acc = mfma4(cq.x, hq[gg].x, acc);
        acc = mfma4(cq.y, hq[gg].y, acc);
        acc = mfma4(cq.z, hq[gg].z, acc);
        acc = mfma4(cq.w, hq[gg].w, acc);
      }
    }
    // then the path terms M[v][u] x~_u, with the diagonal D
    const int i = j;
    const f32x4 mq = *reinterpret_cast<const f32x4*>(s_Mt + (hh * kCvT + i) * kCvT + 4 * k);
    const f32x4 aq = *reinterpret_cast<const f32x4*>(s_a + hh * kCvT + 4 * k);
    const int ancm = s_anc[i];
    const float Dh = s_D[hh];
    f32x4 mop, y;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float mv = ((ancm >> (4 * k + t)) & 1) ? mq[t] * cbr[t] : 0.0f;
      mop[t] = (4 * k + t == i) ? mv + Dh : mv;
      y[t] = aq[t] * acc[t];
    }
    const f32x4 xq = *reinterpret_cast<const f32x4*>(s_xt + row * kCvT + 4 * (k ^ ((row >> 2) & 3)));
    if (__ballot(!finite4(xq)) == 0) {
      y = mfma4(mop.x, xq.x, y);
      y = mfma4(mop.y, xq.y, y);
      y = mfma4(mop.z, xq.z, y);
      y = mfma4(mop.w, xq.w, y);
    } else {
      // A non-finite conv output in the wave's tile: in the product, the
      // zero weight of a node off v's root path would still turn it into
      // NaN in y_v.  Each node's sum runs over its own root path alone
      // instead, as the definition has it.
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int v = 4 * k + t;
        const int av = s_anc[v];
        const float* mrow = s_Mt + (hh * kCvT + v) * kCvT;
        float yy = y[t];
        for (int u = 0; u < kCvT; ++u) {
          const float cb = cbt[v * kCvT + u];  // C_v . B_u
          if ((av >> u) & 1) {
            const float mv = mrow[u] * cb;
            const float xu = s_xt[row * kCvT + 4 * ((u >> 2) ^ ((row >> 2) & 3)) + (u & 3)];
            yy = fmaf(u == v ? mv + Dh : mv, xu, yy);
          }
        }
        y[t] = yy;
      }
    }
    const bool tree_ok = s_misc[2] != 0;
    if constexpr (kCoal) __syncthreads();  // every wave is done with its layout buffer
    if constexpr (OPT) {
      if (xbc && gate) {
        if constexpr (!kCoal) __syncthreads();  // every wave is done with dt * x~ and the path rows
        if (zv < T) *reinterpret_cast<RawQ*>(s_z + zv * kCvRows + zq) = rzl;
        __syncthreads();
      }
    }
    // lane (c + 16 k) holds nodes 4 k + r of channel row
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float yv = y[r];
      if constexpr (OPT)
        if (gate) yv *= silu_fast(load_in(s_z, (4 * k + r) * kCvRows + row));
      s_ys[(4 * k + r) * kCvRows + row] = tree_ok ? yv : __builtin_nanf("");
    }
  }
  __syncthreads();
  {
    const int v = tid / 16, q = tid % 16;  // node row, 16-byte chunk of the 256-byte row segment
    if (v < T)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(s_ys + v * kCvRows + 4 * q),
                                  reinterpret_cast<f32x4*>(a.y + (unit * T + v) * DI + c0 + 4 * q));
  }
}

// ---------------------------------------------------------------------------
// SSM_TREE_CONV_XBC: the convolved B and C rows, once per sequence and group
// ---------------------------------------------------------------------------
//
// Every workgroup of a (layer, sequence) needs the same convolved B and C
// rows of its group (the conv of SSM layers that pass x, B and C through
// conv1d together, Mamba2).  They are formed here once, in fp32, into the
// workspace the round then reads:
//   next tree [T][2N]: node v's B channels (columns 0..N-1) and C channels
//             (N..2N-1) convolved over v's taps: v itself, its ancestors,
//             and past the root the rows of the committed window (the old
//             window's rows, then the accepted path's rows);
//   path      [T][N]: the accepted path's B channels convolved along (old
//             window rows, path rows), positions q < len;
//   C.B       [16][16]: C_v . B_u of the next tree's convolved rows (zero
//             past T), which every wave of the round would otherwise form.
// SiLU follows when set.  The commit length follows the round's own checks
// (0 when the previous tree or the path is not valid, or with nothing to
// commit), so the window taps agree with what the round commits.  One
// workgroup per (group, sequence, layer); each thread owns channels.
template <typename TIn>
__global__ void __launch_bounds__(kBcThreads) bc_conv_kernel(CommitVerifyArgs a) {
  const Dims d = a.d;
  const int T = d.T, W = d.W, N = d.N, G = d.G, DI = d.d_in, CH = d.CH, GN = G * N;
  const int g = blockIdx.x, b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int tid = threadIdx.x;
  __shared__ int32_t s_parent[kCvT], s_pparent[kCvT], s_path[kCvT], s_code[kCvT][3], s_len;
  // the next tree's convolved rows, [node][column] with an odd stride (the
  // C . B dots below read 16 rows at one column on distinct banks)
  constexpr int kRs = 2 * kBcMaxN + 1;
  __shared__ float s_rows[kCvT * kRs];
  const bool commit = a.path_len != nullptr;
  if (tid < T) {
    s_parent[tid] = a.parent[(int64_t)b * T + tid];
    s_pparent[tid] = commit ? a.parent_prev[(int64_t)b * T + tid] : -1;
    s_path[tid] = commit ? a.path[(int64_t)b * T + tid] : 0;
  }
  __syncthreads();
  const bool prev_ok = !commit || tree_is_valid(s_pparent, T);
  if (tid == 0) {
    const int len_raw = commit ? a.path_len[b] : 0;
    bool ok = prev_ok && len_raw >= 0 && len_raw <= T;
    for (int q = 0; ok && q < len_raw; ++q) {
      const int v = s_path[q];
      ok = v >= 0 && v < T && s_pparent[v] == (q == 0 ? -1 : s_path[q - 1]);
    }
    s_len = ok ? len_raw : 0;
  }
  if (tid < T) {
    // taps 1..3 of node tid: an ancestor, or past the root T + the row of
    // the committed window counted from its oldest (a walk that stays in
    // range on an invalid tree, whose outputs the round discards)
    int u = tid, depth = 0, an[3] = {-1, -1, -1};
    for (int s = 0; s < kCvT && u >= 0; ++s) {
      ++depth;
      const int p = s_parent[u];
      u = (p >= 0 && p < u) ? p : -1;
      if (s < 3) an[s] = u;
    }
#pragma unroll
    for (int jj = 1; jj < 4; ++jj) s_code[tid][jj - 1] = an[jj - 1] >= 0 ? an[jj - 1] : T + (W - 2) - (jj - depth);
  }
  __syncthreads();
  const int len = s_len;
  const TIn* win = reinterpret_cast<const TIn*>(a.window_in) + unit * (W - 1) * (int64_t)CH + DI;
  float* out_n = a.bcw + (unit * G + g) * (int64_t)bc_block_floats(T, N);
  float* out_p = out_n + (int64_t)T * 2 * N;
  float* out_cb = out_p + (int64_t)T * N;
  // column c < 2 N: B channel c (c < N) or C channel c - N of group g
  for (int c = tid; c < 2 * N; c += kBcThreads) {
    const bool isB = c < N;
    const int n = isB ? c : c - N;
    const int wch = isB ? g * N + n : GN + g * N + n;  // among the window's B, C channels
    const float* cw = a.prm.conv_w + ((int64_t)l * CH + DI + wch) * W;
    float w[4];  // by taps back: w[jj] weighs the input jj steps before the token
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) w[jj] = jj < W ? cw[W - 1 - jj] : 0.0f;
    const float bias = a.prm.conv_b ? a.prm.conv_b[(int64_t)l * CH + DI + wch] : 0.0f;
    const TIn* rows = reinterpret_cast<const TIn*>(isB ? a.B : a.C) + (unit * T * G + g) * (int64_t)N + n;
    const TIn* prow = reinterpret_cast<const TIn*>(isB ? a.B_prev : a.C_prev) + (unit * T * G + g) * (int64_t)N + n;
    // element e of (old window rows, path rows): the committed window's rows
    // are elements len .. len + W - 2
    auto elem = [&](int e) {
      return e < W - 1 ? load_in(win, (int64_t)e * CH + wch) : load_in(prow, (int64_t)s_path[e - (W - 1)] * GN);
    };
    // (results go to LDS first: no global store between the nodes' loads)
#pragma unroll 4
    for (int v = 0; v < T; ++v) {
      float acc = fmaf(w[0], load_in(rows, (int64_t)v * GN), bias);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        if (jj < W) {
          const int code = s_code[v][jj - 1];
          acc = fmaf(w[jj], code < T ? load_in(rows, (int64_t)code * GN) : elem(len + code - T), acc);
        }
      }
      s_rows[v * kRs + c] = d.silu ? silu_fast(acc) : acc;
    }
    if (isB) {
      for (int q = 0; q < len; ++q) {
        float acc = bias;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (jj < W) acc = fmaf(w[jj], elem(q + W - 1 - jj), acc);
        out_p[(int64_t)q * N + n] = d.silu ? silu_fast(acc) : acc;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < T * 2 * N; i += kBcThreads) out_n[i] = s_rows[(i / (2 * N)) * kRs + i % (2 * N)];
  // C_v . B_u, thread (v, u) of the 16 x 16 table (zero past the tree)
  {
    const int v = tid / kCvT, u = tid % kCvT;
    float acc = 0.0f;
    if (v < T && u < T) {
      const float* cv = s_rows + v * kRs + N;
      const float* bu = s_rows + u * kRs;
      for (int n = 0; n < N; ++n) acc = fmaf(cv[n], bu[n], acc);
    }
    out_cb[tid] = acc;
  }
}

// bytes of the convolved rows a round with SSM_TREE_CONV_XBC on trees of up
// to 16 nodes needs (0 otherwise)
size_t bc_workspace_bytes(const Dims& d) {
  if (!d.xbc || d.T < 1 || d.T > kCvT) return 0;
  return (size_t)d.L * d.Bsz * d.G * bc_block_floats(d.T, d.N) * sizeof(float);
}

hipError_t launch_bc_conv(const CommitVerifyArgs& a, bool bf16, hipStream_t s) {
  dim3 grid(a.d.G, a.d.Bsz, a.d.L);
  if (bf16)
    hipLaunchKernelGGL((bc_conv_kernel<bf16_t>), grid, dim3(kBcThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bc_conv_kernel<float>), grid, dim3(kBcThreads), 0, s, a);
  return hipGetLastError();
}

namespace {

template <typename TIn, typename TS, int NG, bool OPT, bool VO = false>
int launch_cv_o(const CommitVerifyArgs& a, hipStream_t s) {
  const size_t lds =
      (size_t)CvLds(16 * NG, (int)sizeof(TIn), a.d.P, OPT && a.d.xbc, OPT && a.z != nullptr, VO).total;
  if (allow_lds(commit_verify_kernel<TIn, TS, NG, OPT, VO>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  if (OPT && a.d.xbc) {  // the convolved B and C rows first
    if (!a.bcw) return SSM_TREE_E_NULL;
    if (launch_bc_conv(a, sizeof(TIn) == 2, s) != hipSuccess) return SSM_TREE_E_HIP;
  }
  dim3 grid(a.d.d_in / kCvRows, a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((commit_verify_kernel<TIn, TS, NG, OPT, VO>), grid, dim3(kCvWaves * kWave), lds, s, a);
  if (hipGetLastError() != hipSuccess) return SSM_TREE_E_HIP;
  if (!VO && a.d.xbc && a.window_out) {  // the window's B and C rows, after every reader of the old ones
    WindowBcArgs w{a.d, a.parent_prev, a.path, a.path_len, a.B_prev, a.C_prev, a.window_in, a.window_out, 1};
    if (launch_window_bc(w, sizeof(TIn) == 2, s) != hipSuccess) return SSM_TREE_E_HIP;
  }
  return SSM_TREE_OK;
}

template <typename TIn, int NG>
int launch_cv_t(const CommitVerifyArgs& a, hipStream_t s) {
  if (a.d.sbf16)  // (no options with a bfloat16 state)
    return (a.d.xbc || a.z) ? SSM_TREE_E_DIMS : launch_cv_o<TIn, bf16_t, NG, false>(a, s);
  return (a.d.xbc || a.z) ? launch_cv_o<TIn, float, NG, true>(a, s) : launch_cv_o<TIn, float, NG, false>(a, s);
}

template <typename TIn>
int launch_cv_in(const CommitVerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_cv_t<TIn, 1>(a, s);
    case 32: return launch_cv_t<TIn, 2>(a, s);
    case 64: return launch_cv_t<TIn, 4>(a, s);
    case 128: return launch_cv_t<TIn, 8>(a, s);
    case 256: return launch_cv_t<TIn, 16>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

// verify only: the plain instantiation with nothing to commit
template <typename TIn, int NG>
int launch_vo_t(const CommitVerifyArgs& a, hipStream_t s) {
  return a.d.sbf16 ? launch_cv_o<TIn, bf16_t, NG, false, true>(a, s) : launch_cv_o<TIn, float, NG, false, true>(a, s);
}

template <typename TIn>
int launch_vo_in(const CommitVerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_vo_t<TIn, 1>(a, s);
    case 32: return launch_vo_t<TIn, 2>(a, s);
    case 64: return launch_vo_t<TIn, 4>(a, s);
    case 128: return launch_vo_t<TIn, 8>(a, s);
    case 256: return launch_vo_t<TIn, 16>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

}  // namespace

// ssm_tree_verify on the fused round's shapes without the options: the
// round's kernel with nothing to commit (one workgroup per 64 channels of a
// (layer, sequence), the root state read once and never written).
int launch_verify_oneshot(const VerifyArgs& v, bool bf16, hipStream_t s) {
  CommitVerifyArgs a;
  memset(&a, 0, sizeof(a));
  a.d = v.d;
  a.prm = v.prm;
  a.window_in = v.window;
  a.state_in = v.state;
  a.parent = v.parent;
  a.x = v.x;
  a.B = v.B;
  a.C = v.C;
  a.dt_raw = v.dt_raw;
  a.y = v.y;
  a.verify_status = v.seq_status;
  return bf16 ? launch_vo_in<bf16_t>(a, s) : launch_vo_in<float>(a, s);
}

bool commit_verify_fused_applies(const Dims& d) { return d.T >= 1 && d.T <= kCvT && d.P % 16 == 0; }

// SSM_TREE_CONV_XBC and the gate: taken by the kernel's OPT instantiation,
// with a float32 state.
bool commit_verify_options_supported(const Dims& d, bool gate) { return !d.sbf16 || (!d.xbc && !gate); }

int launch_commit_verify(const CommitVerifyArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_cv_in<bf16_t>(a, s) : launch_cv_in<float>(a, s);
}

}  // namespace ssmt
