// verify_mfma.hip - ssm_tree_verify for trees of at most 16 nodes, on the
// gfx950 matrix cores.
//
// Same arithmetic as the root projection in verify.hip (SpecMamba page
// sec. 3.2 recurrence, unrolled along each root path):
//   y_v[c] = a_v(h) (C_v . h0[c]) + sum_u M_h[v][u] x~_u[c],
//   M_h[v][u] = exp(S_v - S_u) dt_u (C_v . B_u) for u on v's root path
//               (u = v included), plus D_h when u = v;  a_v = exp(S_v),
//   S_v = sum of dt * A over v's root path.
// Both sums are dense contractions once the tree is padded to 16 nodes:
//   Y1 = C (16 x N) . h0^T (N x channels)        -- the HBM-bound stream
//   Y  = diag(a) Y1 + M_h (16 x 16) . X~ (16 x channels)
// and both run on v_mfma_f32_16x16x4_f32 (fp32 in, fp32 accumulate).
//
// MFMA operand layout (16x16x4, one block): lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16]; the 16x16 result D[i][j] sits in lane j + 16 (i / 4),
// element i % 4.  The contraction index may be permuted freely as long as A
// and B agree, so for state columns n = 16 gg + 4 k + t a lane (j + 16 k)
// takes the four consecutive columns 16 gg + 4 k .. + 3 of channel j with one
// 16-byte load and feeds them to four MFMAs (t = 0..3): the root state goes
// from HBM to the matrix cores with no LDS transpose, and two loads of a wave
// (gg and gg + 1) cover whole 128-byte lines.
//
// Work split.  A work item is one (layer, sequence, 64-channel slab); every
// wave owns a contiguous range of items and runs on its own (no workgroup
// barrier anywhere).  The root state of its range is one flat stream of
// 1 KiB pieces (16 channels x 16 columns) kept RD pieces ahead in registers,
// across tile, slab and sequence boundaries.  Per item the wave computes the
// conv outputs of its 64 channels and S, dt of its heads; per (layer,
// sequence) and B/C group it loads C into MFMA operand registers and forms
// the 16 x 16 dots C_v . B_u with 32 more MFMAs.
#include "common.h"

namespace ssmt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;            // node rows of an MFMA tile
constexpr int kSlab = 64;            // channels per work item
constexpr int kXRows = kTile + 3;    // conv input rows: nodes, then window rows

// per-wave LDS region (byte offsets)
template <int E>  // input element size
struct WaveLds {
  // two buffers (item parity): [kXRows + 1][64] raw x, then the item's conv
  // outputs [64][16] (swizzled) in place
  static constexpr int xs = 0;
  static constexpr int xs_bytes = (kXRows + 1) * kSlab * E > kSlab * kTile * 4 ? (kXRows + 1) * kSlab * E : kSlab * kTile * 4;
  static constexpr int parent = xs + 2 * xs_bytes;
  static constexpr int anc = parent + 4 * kTile;       // bit u of anc[v]: u is on v's root path (v included)
  static constexpr int cidx = anc + 4 * kTile;         // conv input rows 1..3 of node v, 8 bits each
  static constexpr int S = cidx + 4 * kTile;           // [4 heads][16] cumulative dt * A, times log2(e)
  static constexpr int dt = S + 4 * 4 * kTile;         // [4 heads][16]
  static constexpr int D = dt + 4 * 4 * kTile;         // [4 heads]
  static constexpr int cb = D + 16;                    // [16][16] C.B transpose
  static constexpr int bytes = cb + 4 * kTile * kTile;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
// 16x16x32 bf16 products, fp32 accumulate; the operands as raw bits
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// four consecutive input elements widened to float
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

template <typename TIn>
__device__ __forceinline__ uint32_t raw_bits(const TIn* p);
template <>
__device__ __forceinline__ uint32_t raw_bits<float>(const float* p) { return __float_as_uint(*p); }
template <>
__device__ __forceinline__ uint32_t raw_bits<bf16_t>(const bf16_t* p) { return p->bits; }
template <typename TIn>
__device__ __forceinline__ float from_bits(uint32_t b) { return sizeof(TIn) == 2 ? __uint_as_float(b << 16) : __uint_as_float(b); }

// two consecutive input elements, raw
template <typename TIn>
struct Pair;
template <>
struct Pair<float> {
  typedef uint2 type;
  static __device__ __forceinline__ float get(const float* s, int i) { return s[i]; }
};
template <>
struct Pair<bf16_t> {
  typedef uint32_t type;
  static __device__ __forceinline__ float get(const bf16_t* s, int i) { return __uint_as_float((uint32_t)s[i].bits << 16); }
};

// An opaque copy of a wave-uniform value: derived addresses are recomputed
// where they are used instead of being hoisted (and spilled) out of the loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ int opaque_lane() {
  int v = threadIdx.x;
  asm volatile("" : "+v"(v));
  return v & 63;
}

}  // namespace

// NG = N / 16 column groups per state row; RD = pieces kept in flight; WPG
// waves per workgroup (one workgroup per CU).  ILV (heads a multiple of 64
// channels wide): tile tl of an item holds channels 4 j + tl, so that across
// its four tiles a lane owns four adjacent channels and y leaves in 16-byte
// stores of whole 256-byte row segments; otherwise tile tl holds channels
// 16 tl + j (one head per tile) and y leaves per tile.
template <typename TIn, typename TS, int NG, int RD, int WPG, bool ILV>
__global__ void __launch_bounds__(WPG * 64) verify_mfma_kernel(VerifyArgs a, int items_per_wg) {
  constexpr int N = 16 * NG;
  typedef WaveLds<sizeof(TIn)> Lw;
  static_assert(RD <= 4 * NG && (4 * NG) % RD == 0, "an item's pieces must fill whole ring cycles");
  const Dims d = a.d;
  const int T = d.T, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int NS = DI / kSlab;                        // slabs per (layer, sequence)
  const int total = d.L * d.Bsz * NS;  // work items (the host keeps this below 2^31)
  const int wg_begin = blockIdx.x * items_per_wg;
  const int wg_end = min(total, wg_begin + items_per_wg);
  const int j = lane & 15, k = lane >> 4;

  extern __shared__ __align__(16) unsigned char smem[];
  // The workgroup's items are handed out one at a time from an LDS counter:
  // the hardware issues the oldest waves first, so equal static shares would
  // leave the youngest waves finishing long after the others.
  int* s_next = reinterpret_cast<int*>(smem + WPG * Lw::bytes);
  if (threadIdx.x == 0) *s_next = wg_begin;
  __syncthreads();
  auto grab = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(s_next, 1);
    return __builtin_amdgcn_readlane(v, 0);
  };
  unsigned char* ws = smem + wave * Lw::bytes;
  auto xs_buf = [&](int it) { return reinterpret_cast<float*>(ws + Lw::xs + (it & 1) * Lw::xs_bytes); };
  int32_t* s_par = reinterpret_cast<int32_t*>(ws + Lw::parent);
  int32_t* s_anc = reinterpret_cast<int32_t*>(ws + Lw::anc);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(ws + Lw::cidx);
  float* s_S = reinterpret_cast<float*>(ws + Lw::S);
  float* s_dt = reinterpret_cast<float*>(ws + Lw::dt);
  float* s_D = reinterpret_cast<float*>(ws + Lw::D);
  float* s_cbt = reinterpret_cast<float*>(ws + Lw::cb);

  int cur = grab();
  if (cur >= wg_end) return;
  int nxt = grab();

  // ---- the state stream: piece i of an item = (tile i / NG, columns 16 (i % NG) ..) ----
  typedef StateQuad<TS> SQ;
  const TS* sbase = reinterpret_cast<const TS*>(a.state) + (int64_t)(ILV ? 4 * j : j) * N + 4 * k;
  auto piece = [&](int item, int i) {
    return SQ::load(sbase + ((int64_t)item * kSlab + (i / NG) * (ILV ? 1 : 16)) * N + (i % NG) * 16);
  };
  typename SQ::Raw ring[RD];  // raw: converted where the products take it
  // With bf16 inputs and a bf16 state (kRawC below) and an even number of
  // column groups, pieces go in pairs: lane j + 16 k loads the 8 consecutive
  // columns 32 p + 8 k .. + 7 of column-group pair p with one 16-byte load,
  // and C and B take the same columns (colq).  ring2 holds RD / 2 pairs.
  constexpr bool kWide = sizeof(TIn) == 2 && sizeof(TS) == 2 && NG % 2 == 0;
  auto colq = [&](int gg) { return kWide ? 32 * (gg >> 1) + 8 * k + 4 * (gg & 1) : 16 * gg + 4 * k; };
  const TS* sbase2 = reinterpret_cast<const TS*>(a.state) + (int64_t)(ILV ? 4 * j : j) * N + 8 * k;
  auto pair = [&](int item, int p) {  // pieces 2 p and 2 p + 1
    const int i = 2 * p;
    return *reinterpret_cast<const u32x4*>(sbase2 + ((int64_t)item * kSlab + (i / NG) * (ILV ? 1 : 16)) * N +
                                           32 * ((i % NG) >> 1));
  };
  u32x4 ring2[kWide ? RD / 2 : 1];
  if constexpr (kWide) {
#pragma unroll
    for (int p = 0; p < RD / 2; ++p) ring2[p] = pair(cur, p);
  } else {
#pragma unroll
    for (int i = 0; i < RD; ++i) ring[i] = piece(cur, i);
  }

  // ---- per-item inputs, loaded one item ahead ----
  const TIn* xg = reinterpret_cast<const TIn*>(a.x);
  const TIn* wg = reinterpret_cast<const TIn*>(a.window);
  const TIn* dtr = reinterpret_cast<const TIn*>(a.dt_raw);
  const int HS = P >= kSlab ? 1 : kSlab / P;  // heads touched by a slab
  // raw x rows (nodes, then window rows) of the slab: lanes 0..31 hold rows
  // 2 m, lanes 32..63 rows 2 m + 1, two channels per lane
  typename Pair<TIn>::type xr[(kXRows + 1) / 2];
  // conv taps (0 = the node itself; taps >= W unused) and bias, raw: any
  // arithmetic on a prefetched value here would wait for the load at once
  float wt[5];
  uint32_t dtr_raw;                           // lane (head hl, node v): dt_raw
  float p_bias, p_A, p_D;                     // lane (hl, v): that head's parameters
  auto prefetch = [&](int item) {
    const int unit = item / NS;
    const int slab = item - unit * NS;
    const int l = unit / d.Bsz;
    const int ln = opaque_lane();
    const int c = slab * kSlab + ln;
    {
      const int Tq = opaque(T), DIq = opaque(DI), last = Tq + opaque(W) - 2;
      const TIn* xu = xg + (int64_t)unit * Tq * DIq + slab * kSlab + 2 * (ln & 31);
      const TIn* wu = wg + ((int64_t)unit * (W - 1) - Tq) * DIq + slab * kSlab + 2 * (ln & 31);  // row r >= T at r * DI
#pragma unroll
      for (int m = 0; m < (kXRows + 1) / 2; ++m) {
        int r = 2 * m + (ln >> 5);
        r = r < last ? r : last;  // clamped: every load is in bounds
        xr[m] = *reinterpret_cast<const typename Pair<TIn>::type*>((r < Tq ? xu : wu) + (int64_t)r * DIq);
      }
    }
    const float* cw = a.prm.conv_w + ((int64_t)l * DI + c) * W;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wt[jj] = cw[jj < W ? W - 1 - jj : 0];
    wt[4] = *(a.prm.conv_b ? a.prm.conv_b + (int64_t)l * DI + c : cw);  // no bias: replaced by 0 at use
    const int hl = ln >> 4, v = ln & 15;
    const int hh = min(slab * kSlab / P + (hl < HS ? hl : 0), H - 1);
    dtr_raw = raw_bits<TIn>(dtr + ((int64_t)unit * T + (v < T ? v : T - 1)) * H + hh);
    p_bias = a.prm.dt_bias[(int64_t)l * H + hh];
    p_A = a.prm.A[(int64_t)l * H + hh];
    p_D = a.prm.D[(int64_t)l * H + hh];
  };
  // Take delivery of item it's prefetched inputs: raw x into its LDS buffer,
  // the rest marked as arrived.  Placed in straight-line code a fixed number
  // of memory operations after the prefetch, so that the compiler's wait is
  // exact (a wait after a branch join degrades to draining the stream).
  auto deliver = [&](int par) {
    const int ln = opaque_lane();
    TIn* s_xr = reinterpret_cast<TIn*>(xs_buf(par));
#pragma unroll
    for (int m = 0; m < (kXRows + 1) / 2; ++m)
      *reinterpret_cast<typename Pair<TIn>::type*>(s_xr + (2 * m + (ln >> 5)) * kSlab + 2 * (ln & 31)) = xr[m];
#pragma unroll
    for (int q = 0; q < 5; ++q) asm volatile("" : "+v"(wt[q]));
    asm volatile("" : "+v"(dtr_raw), "+v"(p_bias), "+v"(p_A), "+v"(p_D));
  };
  prefetch(cur);
  deliver(0);

  // ---- per (layer, sequence) and group state ----
  int cur_unit = -1;
  int cur_group = -1;
  bool ok = false;
  // bf16 inputs with a bf16 state: C and the state are exact bf16 operands,
  // and C . h0 takes one 16x16x32 product per pair of column groups (lane
  // i + 16 k feeds columns 16 gg + 4 k .. + 3 of both, the same slots in C
  // and in the state); C stays as raw bits
  constexpr bool kRawC = sizeof(TIn) == 2 && sizeof(TS) == 2;
  f32x4 cop[NG];  // lane (i + 16 k): C_i[16 gg + 4 k .. + 3], zero for i >= T
  su32x2 craw[NG];  // the same as raw bits (kRawC)
  f32x4 cbop;     // lane (i + 16 k): C_i . B_(4 k + t), zero off i's root path
  int ancm = 0;   // anc[i]
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    cop[gg] = f32x4{0.f, 0.f, 0.f, 0.f};
    craw[gg] = su32x2{0u, 0u};
  }
  cbop = f32x4{0.f, 0.f, 0.f, 0.f};

  // start of item it: tree bookkeeping on a new (layer, sequence), C operands
  // and C.B dots on a new group, conv outputs and S, dt of the slab's heads
  auto item_start = [&](int item, int par) {
    const int lane = opaque_lane();  // recomputed here rather than kept live across the stream
    const int j = lane & 15, k = lane >> 4;
    const int unit = item / NS;
    const int slab = item - unit * NS;
    const int l = unit / d.Bsz, b = unit - l * d.Bsz;
    const int g = slab * kSlab / (DI / G);
    float* s_xs = xs_buf(par);
    const TIn* s_xr = reinterpret_cast<const TIn*>(s_xs);  // [kXRows + 1][64] raw, delivered
    const bool new_unit = unit != cur_unit;
    if (new_unit) {
      cur_unit = unit;
      const int par = a.parent[(int64_t)b * T + (lane < T ? lane : T - 1)];
      const int prev = __shfl_up(par, 1);
      const bool bad = lane < T && (lane == 0 ? par != -1 : (par < -1 || par >= lane || par < prev));
      ok = __ballot(bad) == 0;
      if (ok) {
        if (lane < T) s_par[lane] = par;
        wave_sync();
        if (lane < kTile) {
          int m = 0, packed = 0;
          if (lane < T) {
            for (int u = lane; u >= 0; u = s_par[u]) m |= 1 << u;
            for (int jj = 1; jj < W; ++jj) {
              const int code = conv_input_code(s_par, lane, jj, W);
              packed |= (code >= 0 ? code : T + (-1 - code)) << (8 * (jj - 1));
            }
          }
          s_anc[lane] = m;  // zero for the padding rows
          s_cidx[lane] = packed;
        }
        wave_sync();
      }
    }
    if (slab == 0 && l == 0 && lane == 0 && a.seq_status) a.seq_status[b] = ok ? SSM_TREE_OK : SSM_TREE_E_TREE;
    if (!ok) return;
    if (new_unit || g != cur_group) {
      cur_group = g;
      const int i = lane & 15;
      const int ic = i < T ? i : T - 1;
      const float keep = i < T ? 1.0f : 0.0f;
      const TIn* cg = reinterpret_cast<const TIn*>(a.C) + (((int64_t)unit * T + ic) * G + g) * N + 4 * k;
      const TIn* bg = reinterpret_cast<const TIn*>(a.B) + (((int64_t)unit * T + ic) * G + g) * N + 4 * k;
      const TIn* cg0 = cg - 4 * k, *bg0 = bg - 4 * k;  // row starts (for colq)
      // CB[v][u] = C_v . B_u: A = C rows, B = B rows (lane j + 16 k holds B_j)
      f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kRawC) {
        su32x2 braw[NG];
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          craw[gg] = *reinterpret_cast<const su32x2*>(cg0 + colq(gg));
          braw[gg] = *reinterpret_cast<const su32x2*>(bg0 + colq(gg));
          if (i >= T) craw[gg] = braw[gg] = su32x2{0u, 0u};
        }
#pragma unroll
        for (int gp = 0; gp < (NG + 1) / 2; ++gp) {
          const su32x2 c1 = 2 * gp + 1 < NG ? craw[(2 * gp + 1) % NG] : su32x2{0u, 0u};
          const su32x2 b1 = 2 * gp + 1 < NG ? braw[(2 * gp + 1) % NG] : su32x2{0u, 0u};
          cb = mfma32(u32x4{craw[2 * gp].x, craw[2 * gp].y, c1.x, c1.y},
                      u32x4{braw[2 * gp].x, braw[2 * gp].y, b1.x, b1.y}, cb);
        }
      } else {
        f32x4 bop[NG];
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          cop[gg] = load4<TIn>(cg + 16 * gg) * keep;
          bop[gg] = load4<TIn>(bg + 16 * gg) * keep;
        }
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          cb = mfma4(cop[gg].x, bop[gg].x, cb);
          cb = mfma4(cop[gg].y, bop[gg].y, cb);
          cb = mfma4(cop[gg].z, bop[gg].z, cb);
          cb = mfma4(cop[gg].w, bop[gg].w, cb);
        }
      }
      // result layout: lane (u + 16 q) holds CB[4 q + r][u]; transpose through LDS
#pragma unroll
      for (int r = 0; r < 4; ++r) s_cbt[(4 * k + r) * 16 + j] = cb[r];
      wave_sync();
      const f32x4 row = *reinterpret_cast<const f32x4*>(s_cbt + i * 16 + 4 * k);
      ancm = s_anc[i];
#pragma unroll
      for (int t = 0; t < 4; ++t) cbop[t] = ((ancm >> (4 * k + t)) & 1) ? row[t] : 0.0f;
      wave_sync();
    }
    // conv outputs of the slab's 64 channels (lane = channel), nodes in registers
    wave_sync();
    int4 cq[4];  // every node's conv input rows, read at once
#pragma unroll
    for (int q = 0; q < 4; ++q) cq[q] = *reinterpret_cast<const int4*>(s_cidx + 4 * q);
    // tap reads without branches (every row holds an input or a clamped copy
    // of one; unused taps and nodes past T are dropped by selects, never
    // scaled by a zero weight), so that the reads need not wait one by one
    float xt[kTile];
    const float bias = a.prm.conv_b ? wt[4] : 0.0f;
#pragma unroll
    for (int v = 0; v < kTile; ++v) {
      const int ci = __builtin_amdgcn_readfirstlane(v % 4 == 0 ? cq[v / 4].x : v % 4 == 1 ? cq[v / 4].y
                                                                : v % 4 == 2 ? cq[v / 4].z : cq[v / 4].w);
      float z = fmaf(wt[0], Pair<TIn>::get(s_xr, v * kSlab + lane), bias);
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        const float u = Pair<TIn>::get(s_xr, ((ci >> (8 * (jj - 1))) & 255) * kSlab + lane);
        z = jj < W ? fmaf(wt[jj], u, z) : z;
      }
      xt[v] = z;
    }
    if (d.silu) {  // (a uniform branch: a select would run the transcendentals either way)
#pragma unroll
      for (int v = 0; v < kTile; ++v) xt[v] = xt[v] * __builtin_amdgcn_rcpf(1.0f + __expf(-xt[v]));
    }
#pragma unroll
    for (int v = 0; v < kTile; ++v) xt[v] = v < T ? xt[v] : 0.0f;
    // S and dt of the slab's heads: lane (hl, v)
    {
      const int hl = lane >> 4, v = lane & 15;
      const float dt = v < T ? softplus_f32(from_bits<TIn>(dtr_raw) + p_bias) : 0.0f;
      wave_sync();
      // conv outputs as the MFMA B operand: the channel in column j of tile tl
      // sits in row p = 16 tl + j, its quad q at p * 16 + 4 (q ^ ((p >> 2) & 3))
      const int p = ILV ? (lane & 3) * 16 + (lane >> 2) : lane;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(s_xs + p * 16 + 4 * (q ^ ((p >> 2) & 3))) =
            f32x4{xt[4 * q], xt[4 * q + 1], xt[4 * q + 2], xt[4 * q + 3]};
      if (hl < HS) s_S[hl * 16 + v] = dt * p_A;
      wave_sync();
      // S_v = sum of dt * A over v's root path, root first (zero terms skipped
      // in effect: adding +0 leaves the sum unchanged)
      const int hr = hl < HS ? hl : 0;
      f32x4 dq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) dq[q] = *reinterpret_cast<const f32x4*>(s_S + hr * 16 + 4 * q);
      const int m = v < T ? s_anc[v] : 0;
      float S = 0.0f;
#pragma unroll
      for (int u = 0; u < kTile; ++u) S += ((m >> u) & 1) ? dq[u / 4][u % 4] : 0.0f;
      wave_sync();
      if (hl < HS) {
        // stored in base-2 units: exp(S_v - S_u) = exp2(S2_v - S2_u)
        s_S[hl * 16 + v] = S * 1.4426950408889634f;
        s_dt[hl * 16 + v] = dt;
        if (v == 0) s_D[hl] = p_D;
      }
      wave_sync();
    }
  };

  // tile epilogue: y = diag(a) Y1 + M_h X~ for 16 channels; lane (c + 16 k)
  // returns nodes 4 k .. 4 k + 3 of its channel (NaN for an invalid tree)
  auto tile_end = [&](int item, int par, int tl, f32x4 acc) {
    const int lane = opaque_lane();
    const int j = lane & 15, k = lane >> 4;
    const int unit = item / NS;
    const int slab = item - unit * NS;
    const float* s_xs = xs_buf(par);
    const int hl = ILV ? 0 : (slab * kSlab + tl * 16) / P - slab * kSlab / P;
    const int i = lane & 15;
    const float Sv = s_S[hl * 16 + i];
    const f32x4 Sq = *reinterpret_cast<const f32x4*>(s_S + hl * 16 + 4 * k);
    const f32x4 dq = *reinterpret_cast<const f32x4*>(s_dt + hl * 16 + 4 * k);
    const float Dh = s_D[hl];
    f32x4 mop, y;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float m = ((ancm >> (4 * k + t)) & 1) ? __builtin_amdgcn_exp2f(Sv - Sq[t]) * dq[t] * cbop[t] : 0.0f;
      mop[t] = (4 * k + t == i) ? m + Dh : m;
      y[t] = __builtin_amdgcn_exp2f(Sq[t]) * acc[t];  // lane (c + 16 k) holds nodes 4 k + t
    }
    const int cl = tl * 16 + j;
    const f32x4 xq = *reinterpret_cast<const f32x4*>(s_xs + cl * 16 + 4 * (k ^ ((cl >> 2) & 3)));
    y = mfma4(mop.x, xq.x, y);
    y = mfma4(mop.y, xq.y, y);
    y = mfma4(mop.z, xq.z, y);
    y = mfma4(mop.w, xq.w, y);
    // selected, not branched: the body stays straight-line
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = ok ? y[r] : __builtin_nanf("");
    return y;
  };
  // y of one tile (channels 16 tl + j)
  auto store_tile = [&](int item, int tl, f32x4 y) {
    const int lane = opaque_lane();
    const int j = lane & 15, k = lane >> 4;
    const int unit = item / NS;
    float* yo = a.y + (int64_t)unit * T * DI + (item - unit * NS) * kSlab + tl * 16 + j;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * k + r < T) yo[(int64_t)(4 * k + r) * DI] = y[r];
  };
  // y of an interleaved item: lane (j + 16 k) holds channels 4 j .. 4 j + 3 of nodes 4 k + r
  auto store_item = [&](int item, const f32x4 (&ys)[4]) {
    const int lane = opaque_lane();
    const int j = lane & 15, k = lane >> 4;
    const int unit = item / NS;
    float* yo = a.y + (int64_t)unit * T * DI + (item - unit * NS) * kSlab + 4 * j;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * k + r < T)
        *reinterpret_cast<f32x4*>(yo + (int64_t)(4 * k + r) * DI) = f32x4{ys[0][r], ys[1][r], ys[2][r], ys[3][r]};
  };

  // ---- main loop: one work item (4 tiles of NG pieces) per iteration ----
  // After item_start the body is straight-line: the next item's inputs are
  // requested, then delivered two tiles later; the ring runs on into the
  // next item (the current one again when there is none).
  for (int par = 0;; par ^= 1) {
    const int after = grab();  // the item after next, known well before it is needed
    item_start(cur, par);
    const int nx = nxt < wg_end ? nxt : cur;
    prefetch(nx);
    f32x4 ys[4];
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kWide) {
#pragma unroll
        for (int gp = 0; gp < NG / 2; ++gp) {
          const int pp = tl * (NG / 2) + gp;  // pair index within the item, static
          acc = mfma32(u32x4{craw[2 * gp].x, craw[2 * gp].y, craw[2 * gp + 1].x, craw[2 * gp + 1].y},
                       ring2[pp % (RD / 2)], acc);
          ring2[pp % (RD / 2)] = pp + RD / 2 < 2 * NG ? pair(cur, pp + RD / 2) : pair(nx, pp + RD / 2 - 2 * NG);
        }
      } else if constexpr (kRawC) {
#pragma unroll
        for (int gp = 0; gp < (NG + 1) / 2; ++gp) {
          const int i = tl * NG + 2 * gp;  // static
          const bool two = 2 * gp + 1 < NG;
          const su32x2 c1 = two ? craw[(2 * gp + 1) % NG] : su32x2{0u, 0u};
          const su32x2 h0 = ring[i % RD];
          const su32x2 h1 = two ? ring[(i + 1) % RD] : su32x2{0u, 0u};
          acc = mfma32(u32x4{craw[2 * gp].x, craw[2 * gp].y, c1.x, c1.y}, u32x4{h0.x, h0.y, h1.x, h1.y}, acc);
          ring[i % RD] = i + RD < 4 * NG ? piece(cur, i + RD) : piece(nx, i + RD - 4 * NG);
          if (two)
            ring[(i + 1) % RD] = i + 1 + RD < 4 * NG ? piece(cur, i + 1 + RD) : piece(nx, i + 1 + RD - 4 * NG);
        }
      } else {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
          const int i = tl * NG + gg;  // static
          const f32x4 h = SQ::to_f32(ring[i % RD]);
          acc = mfma4(cop[gg].x, h.x, acc);
          acc = mfma4(cop[gg].y, h.y, acc);
          acc = mfma4(cop[gg].z, h.z, acc);
          acc = mfma4(cop[gg].w, h.w, acc);
          ring[i % RD] = i + RD < 4 * NG ? piece(cur, i + RD) : piece(nx, i + RD - 4 * NG);
        }
      }
      ys[tl] = tile_end(cur, par, tl, acc);
      if (!ILV) store_tile(cur, tl, ys[tl]);
      if (tl == 1) deliver(par ^ 1);
    }
    if (ILV) store_item(cur, ys);
    if (nxt >= wg_end) break;
    cur = nxt;
    nxt = after;
  }
}

namespace {

template <typename TIn, typename TS, int NG, int RD, bool ILV>
int launch_mfma_t(const VerifyArgs& a, hipStream_t s) {
  // sixteen waves per CU where registers and LDS allow, else twelve
  constexpr int kWpg = (sizeof(TIn) == 2 && NG <= 8) ? 16 : 12;
  auto kern = verify_mfma_kernel<TIn, TS, NG, RD, kWpg, ILV>;
  const size_t lds = (size_t)kWpg * WaveLds<sizeof(TIn)>::bytes + 16;
  if (allow_lds(kern, lds) != hipSuccess) return SSM_TREE_E_HIP;
  int dev = 0, n_cu = 0, resident = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&resident, reinterpret_cast<const void*>(kern), kWpg * kWave, lds) !=
          hipSuccess ||
      resident < 1)
    return SSM_TREE_E_HIP;
  const int64_t items = (int64_t)a.d.L * a.d.Bsz * (a.d.d_in / kSlab);
  if (items >= ((int64_t)1 << 30)) return SSM_TREE_E_DIMS;  // item indices are 32-bit in the kernel
  const int64_t groups = (int64_t)resident * n_cu;
  const int64_t ipg = (items + groups - 1) / groups;
  const int64_t wgs = (items + ipg - 1) / ipg;
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kWpg * kWave), lds, s, a, (int)ipg);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

template <typename TIn, typename TS, bool ILV>
int launch_mfma_n(const VerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_mfma_t<TIn, TS, 1, 4, ILV>(a, s);
    case 32: return launch_mfma_t<TIn, TS, 2, 8, ILV>(a, s);
    case 64: return launch_mfma_t<TIn, TS, 4, 8, ILV>(a, s);
    case 128: return launch_mfma_t<TIn, TS, 8, 8, ILV>(a, s);
    case 256: return launch_mfma_t<TIn, TS, 16, 4, ILV>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

template <typename TIn, typename TS>
int launch_mfma_in(const VerifyArgs& a, hipStream_t s) {
  return a.d.P % kSlab == 0 ? launch_mfma_n<TIn, TS, true>(a, s) : launch_mfma_n<TIn, TS, false>(a, s);
}

}  // namespace

// Trees of at most 16 nodes with heads of a multiple of 16 channels.
bool mfma_verify_applies(const Dims& d) { return d.T >= 1 && d.T <= kTile && d.P % 16 == 0 && d.d_in % kSlab == 0; }

int launch_verify_mfma(const VerifyArgs& a, bool bf16, hipStream_t s) {
  if (a.d.sbf16) return bf16 ? launch_mfma_in<bf16_t, bf16_t>(a, s) : launch_mfma_in<float, bf16_t>(a, s);
  return bf16 ? launch_mfma_in<bf16_t, float>(a, s) : launch_mfma_in<float, float>(a, s);
}

}  // namespace ssmt
