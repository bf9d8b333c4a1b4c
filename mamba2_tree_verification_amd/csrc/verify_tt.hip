// verify_tt.hip - ssm_tree_verify for trees of 17 to 64 nodes, on the gfx950
// matrix cores.
//
// The root projection of verify.hip (SpecMamba page sec. 3.2
// recurrence, unrolled along each root path):
//   y_v[c] = a_v (C_v . h0[c]) + sum_{u on path(v)} M_h[v][u] x~_u[c],
//   M_h[v][u] = exp(S_v - S_u) dt_u (C_v . B_u), plus D_h when u = v,
//   a_v = exp(S_v), S_v = sum of dt * A over v's root path,
// with the tree padded to TT tiles of 16 nodes.  At 64 nodes C . h0 is 32
// flop per state byte, above the fp32 matrix-core ridge (19.7 flop/B) and
// far above the vector ALU's (9.8 without packed fp32): the product runs on
// v_mfma_f32_16x16x4_f32 in TT row tiles, and M_h . X~ over the
// lower-triangular tile pairs (an ancestor's index is below its
// descendant's).
//
// Mapping.  A workgroup of 4 waves owns one (layer, sequence) and NBLK
// consecutive blocks of 64 channels inside one B/C group; wave w owns
// channels 16 w .. 16 w + 15 of a block, in the MFMA B-operand layout
// (lane j + 16 k holds columns 16 gg + 4 k .. + 3 of channel j).  The tree
// bookkeeping, the C rows and the C_v . B_u dots (formed once for the NBLK
// blocks, with B rows as the A operand so that the result lands in the
// layout the path terms read) stay in LDS.  Per block: conv outputs and the
// heads' S and dt, then C . h0 (the next block's state is loaded as soon as
// each column group has been consumed), the path terms, and y staged in LDS
// and stored as whole 256-byte row segments.
#include <type_traits>

#include "common.h"

namespace ssmt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// word 3 of a raw buffer resource on gfx9: 32-bit data format (untyped
// accesses, range-checked against the record count, no swizzle)
constexpr int kBufWord3 = 0x00020000;
// s_waitcnt vmcnt(0), the other counters left alone (gfx9 encoding)
constexpr int kWaitVm0 = 0x0F70;

constexpr int kTtRows = 64;   // channels per block
constexpr int kTtWaves = 4;
constexpr int kTtThreads = kTtWaves * kWave;
constexpr int kTtMaxT = 64;
// C.B and M are kept by lower-triangular tile pair (ti, tj), pair index
// ti (ti + 1) / 2 + tj, as 16 rows of 16 values; rows are 20 floats apart so
// that the 16 rows a wave reads at once fall on different LDS banks
constexpr int kPairStride = 20;
__host__ __device__ constexpr int pair_of(int ti, int tj) { return ti * (ti + 1) / 2 + tj; }
__host__ __device__ constexpr int pair_ti(int pi) {
  int ti = 0;
  while ((ti + 1) * (ti + 2) / 2 <= pi) ++ti;
  return ti;
}
__host__ __device__ constexpr int pair_tj(int pi) { return pi - pair_of(pair_ti(pi), 0); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 16 x 16 x 32 bf16 product: each lane brings 8 values of its A row and of
// its B column; only the pairing of A's and B's k slots matters for the sum,
// and both operands here fill their slots from the same state indices
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
// two bf16 (raw bits, in the high halves of lo and hi) packed into a dword
__device__ __forceinline__ uint32_t pack_hi(uint32_t lo, uint32_t hi) { return (lo >> 16) | (hi & 0xFFFF0000u); }
// eight fp32 values as the sum of three bf16 terms, by truncation: each
// remainder is exact in fp32, and the third term leaves less than 2^-21 of
// the value
__device__ __forceinline__ void split3(f32x4 p, f32x4 q, u32x4& t0, u32x4& t1, u32x4& t2) {
  uint32_t b0[8], b1[8], b2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = e < 4 ? p[e] : q[e - 4];
    const uint32_t h = __float_as_uint(v) & 0xFFFF0000u;
    const float r = v - __uint_as_float(h);
    const uint32_t m = __float_as_uint(r) & 0xFFFF0000u;
    b0[e] = h;
    b1[e] = m;
    b2[e] = __float_as_uint(r - __uint_as_float(m));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    t0[w] = pack_hi(b0[2 * w], b0[2 * w + 1]);
    t1[w] = pack_hi(b1[2 * w], b1[2 * w + 1]);
    t2[w] = pack_hi(b2[2 * w], b2[2 * w + 1]);
  }
}

// 4 x 4 transpose across the four lanes of a quad (lane index j & 3) and
// the four elements of q: element t of lane s ends as element s of lane t.
// Two butterfly stages: swap the off-diagonal 2 x 2 blocks between lanes
// 2 apart, then the off-diagonal elements of each 2 x 2 block between
// neighbouring lanes (DPP quad permutations)
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 m, int j) {
  const bool hi = (j & 2) != 0, lo = (j & 1) != 0;
  const float x0 = dpp_xor2(m.x), x1 = dpp_xor2(m.y), x2 = dpp_xor2(m.z), x3 = dpp_xor2(m.w);
  const float n0 = hi ? x2 : m.x, n1 = hi ? x3 : m.y, n2 = hi ? m.z : x0, n3 = hi ? m.w : x1;
  const float y0 = dpp_xor1(n0), y1 = dpp_xor1(n1), y2 = dpp_xor1(n2), y3 = dpp_xor1(n3);
  return f32x4{lo ? y1 : n0, lo ? n1 : y0, lo ? y3 : n2, lo ? n3 : y2};
}

template <typename TIn>
__device__ __forceinline__ f32x4 load4(const TIn* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<bf16_t>(const bf16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  f32x4 r;
  r.x = __uint_as_float(w.x << 16);
  r.y = __uint_as_float(w.x & 0xFFFF0000u);
  r.z = __uint_as_float(w.y << 16);
  r.w = __uint_as_float(w.y & 0xFFFF0000u);
  return r;
}

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

// an input element's raw bits in a 32-bit register, and back
template <typename TIn>
__device__ __forceinline__ uint32_t raw_bits(const TIn* p);
template <>
__device__ __forceinline__ uint32_t raw_bits<float>(const float* p) {
  return __float_as_uint(*p);
}
template <>
__device__ __forceinline__ uint32_t raw_bits<bf16_t>(const bf16_t* p) {
  return p->bits;
}
template <typename TIn>
__device__ __forceinline__ TIn from_bits(uint32_t r);
template <>
__device__ __forceinline__ float from_bits<float>(uint32_t r) {
  return __uint_as_float(r);
}
template <>
__device__ __forceinline__ bf16_t from_bits<bf16_t>(uint32_t r) {
  return bf16_t{(uint16_t)r};
}
// threadIdx.x through an empty asm: values derived from it inside a phase
// are recomputed there instead of being hoisted out of the block loop and
// kept live across it (which ran the kernel out of registers)
__device__ __forceinline__ int opaque_tid() {
  int v = threadIdx.x;
  asm volatile("" : "+v"(v));
  return v;
}

// softplus(z) = max(z, 0) + log1p(exp(-|z|)) with the hardware exp2 and
// log2; log1p(t) as log(u) t / (u - 1), u = 1 + t, which cancels the
// rounding of u (Goldberg's form), so small t keeps its relative accuracy;
// above 20 the result is z, as in the plain definition's usual cut-over
__device__ __forceinline__ float softplus_hw(float z) {
  const float t = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(z));
  const float u = 1.0f + t;
  const float lp =
      u == 1.0f ? t : __builtin_amdgcn_logf(u) * 0.6931471805599453f * t * __builtin_amdgcn_rcpf(u - 1.0f);
  return z > 20.0f ? z : fmaxf(z, 0.0f) + lp;
}


// the sum of acc over the root path of node (lane) v, given each node's
// parent up (-1 at a root) within one wave: pointer jumping, six rounds for
// paths of up to 64 nodes (round r adds the partial sum of the node 2^r
// steps up)
__device__ __forceinline__ double root_path_sum(double acc, int up, int v) {
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = up >= 0 ? up : v;
    const double acc_up = __shfl(acc, src);
    const int up_up = __shfl(up, src);
    if (up >= 0) {
      acc += acc_up;
      up = up_up;
    }
  }
  return acc;
}

// M[v][u0 .. u0 + 3] of one head: exp(S_v - S_u) dt_u (C_v . B_u) where u is
// on v's root path (ancestor bits ancv), zero elsewhere, plus D on the
// diagonal; S in base-2 units, fp64 (the difference is taken before rounding)
typedef double f64x2 __attribute__((ext_vector_type(2)));
// the LDS inputs of one M quad, loaded apart from the arithmetic so that a
// wave can have several quads' loads in flight
struct MQuadIn {
  double Sv;
  f64x2 sa, sb;
  f32x4 du, cb;
  uint32_t nib;
};
__device__ __forceinline__ MQuadIn m_load(int v, int u0, const double* S2h, const float* dth, uint64_t ancv,
                                          const float* cbr) {
  MQuadIn q;
  q.Sv = S2h[v];
  q.du = *reinterpret_cast<const f32x4*>(dth + u0);
  q.cb = *reinterpret_cast<const f32x4*>(cbr);
  q.sa = *reinterpret_cast<const f64x2*>(S2h + u0);
  q.sb = *reinterpret_cast<const f64x2*>(S2h + u0 + 2);
  q.nib = (uint32_t)(ancv >> u0) & 15u;
  return q;
}
template <bool kDiag>
__device__ __forceinline__ f32x4 m_compute(const MQuadIn& q, int v, int u0, float Dh) {
  f32x4 m;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const double su = t == 0 ? q.sa.x : (t == 1 ? q.sa.y : (t == 2 ? q.sb.x : q.sb.y));
    const float e = __builtin_amdgcn_exp2f((float)(q.Sv - su)) * q.du[t] * q.cb[t];
    const float mv = ((q.nib >> t) & 1) ? e : 0.0f;
    m[t] = kDiag && u0 + t == v ? mv + Dh : mv;
  }
  return m;
}
template <bool kDiag>
__device__ __forceinline__ f32x4 m_quad(int v, int u0, const double* S2h, const float* dth, uint64_t ancv,
                                        const float* cbr, float Dh) {
  return m_compute<kDiag>(m_load(v, u0, S2h, dth, ancv, cbr), v, u0, Dh);
}

// M of the block's head for the tile pairs slot, slot + 4, ... (at most 3 for
// 64 nodes): all loads first, then the arithmetic and the stores
template <int TT, int kSlot>
__device__ __forceinline__ void m_form_slot(float* s_m, const float* s_cbt, const uint64_t* s_anc,
                                            const double* S2w, const float* dtw, float Dh0, int r, int cq) {
  constexpr int kPairs = TT * (TT + 1) / 2;
  constexpr int kMine = (kPairs - kSlot + 3) / 4;
  MQuadIn in[kMine > 0 ? kMine : 1];
#pragma unroll
  for (int k = 0; k < kMine; ++k) {
    const int pi = kSlot + 4 * k;
    const int v = 16 * pair_ti(pi) + r, u0 = 16 * pair_tj(pi) + 4 * cq;
    in[k] = m_load(v, u0, S2w, dtw, s_anc[v], s_cbt + (16 * pi + r) * kPairStride + 4 * cq);
  }
#pragma unroll
  for (int k = 0; k < kMine; ++k) {
    const int pi = kSlot + 4 * k;
    const int v = 16 * pair_ti(pi) + r, u0 = 16 * pair_tj(pi) + 4 * cq;
    *reinterpret_cast<f32x4*>(s_m + (16 * pi + r) * kPairStride + 4 * cq) =
        pair_ti(pi) == pair_tj(pi) ? m_compute<true>(in[k], v, u0, Dh0) : m_compute<false>(in[k], v, u0, Dh0);
  }
}

// LDS layout (byte offsets)
struct TtLds {
  int parent, anc, cidx, misc, C, cbt, X, Y, Mo, So, S2, Ah, dt, D, cw, cb, nf, R, total, row, rawrow;
  // opt: the Mamba2-convention options' instantiation, whose B and C rows are
  // staged as float32 (convolved with the xBC conv), the raw rows apart
  __host__ __device__ TtLds(int N, int E, int TT, bool opt = false) {
    const int KT = 16 * TT, pair_bytes = 4 * 16 * kPairStride * pair_of(TT, 0);
    int o = 0;
    rawrow = N * E + 16;                       // raw B / C row stride (padded)
    row = opt ? N * 4 + 16 : rawrow;           // staged B / C row stride (padded)
    parent = o; o += 4 * kTtMaxT;
    anc = o; o += 8 * kTtMaxT;                 // root-path bitmask per node (64 bits)
    cidx = o; o += 4 * kTtMaxT;                // conv inputs of taps 1..3: row of the window-and-x rows
    misc = o; o += 16;                         // [0] tree ok
    C = o; o += KT * row;                      // C rows (raw)
    cbt = o; o += pair_bytes;                  // C_v . B_u by tile pair
    X = o;                                     // B rows (raw) until the dots exist, then conv outputs
    o += KT * row > 4 * kTtRows * kTtMaxT ? KT * row : 4 * kTtRows * kTtMaxT;
    // a block's 3 window rows (the last one at row 2) and x rows (node v at
    // row 3 + v), raw
    Y = o; o += ((3 + KT) * kTtRows * E + 15) / 16 * 16;
    Mo = o; o += pair_bytes;                   // M of the block's head by tile pair (one head per block)
    So = o; o += 4 * 4 * kTtMaxT;              // [head][node] dt * A
    // [head][node] S over the root path times log2(e), fp64; with one head
    // per block, [wave][node]: each wave's own copy of the head's
    S2 = o; o += 8 * 4 * kTtMaxT;
    Ah = o; o += 4 * 4 * kTtMaxT;              // [head][node] exp(S)
    dt = o; o += 4 * 8 * kTtMaxT;              // [block][node]; several heads per block: [parity][head][node]
    D = o; o += 32;                            // [block]; several heads per block: [parity][head]
    cw = o; o += 4 * 4 * kTtRows;              // [tap][channel], tap t = the node t steps up the path
    cb = o; o += 4 * kTtRows;
    nf = o; o += kTtRows * kTtMaxT / 4;        // [channel][node quad] codes of non-finite conv outputs
    R = o; o += opt ? 2 * KT * rawrow : 0;     // (opt) raw B rows, then raw C rows
    total = o;
  }
};

}  // namespace

// Non-finite conv outputs.  In the product M . X~ the zero weight of a node u
// off v's root path would still turn a non-finite x~_u into NaN in y_v.  So
// the conv stores such an entry as zero, with a bit beside it (nibble q of
// channel c: nodes 4 q .. 4 q + 3), and a block that has one (rare) then
// overwrites, after the product, every y_v whose root path holds a
// non-finite x~_u with NaN: by the definition's sum y_v is not finite there
// (NaN, or an infinity that NaN stands for).
__device__ __forceinline__ uint32_t nonfinite_quad(f32x4& q) {
  uint32_t bits = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bool nf = !__builtin_isfinite(q[t]);
    bits |= (nf ? 1u : 0u) << t;
    q[t] = nf ? 0.0f : q[t];
  }
  return bits;
}

// The nodes whose conv output in channel `row` is not finite, as a bit mask.
__device__ __forceinline__ uint64_t nonfinite_nodes(const uint8_t* nf, int row) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(nf + row * (kTtMaxT / 4));
  uint64_t m = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) m |= (uint64_t)((w[q >> 2] >> (8 * (q & 3))) & 15u) << (4 * q);
  return m;
}

// OPT: the Mamba2-convention options (the xBC conv, the gate) in an
// instantiation of their own: B and C rows staged as float32 (convolved over
// each node's path with the xBC conv), products on the float32 matrix
// cores, y gated by silu(z).
template <typename TIn, typename TS, int NG, int TT, bool OPT>
__global__ void __launch_bounds__(kTtThreads) verify_tt_kernel(VerifyArgs a, int NBLK) {
  typedef StateQuad<TS> SQ;
  typedef typename std::conditional<OPT, float, TIn>::type TR;  // element type of the staged B and C rows
  constexpr int N = 16 * NG;
  constexpr int E = (int)sizeof(TIn);
  constexpr int KT = 16 * TT;                      // node capacity
  typedef typename Raw4<E>::T RawQ;
  constexpr int kChunks = N * E / 16;              // 16-byte chunks per B / C row
  const Dims d = a.d;
  const int T = d.T, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G, CH = d.CH;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane & 15, k = lane >> 4;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int cw0 = blockIdx.x * NBLK * kTtRows;
  const int g = cw0 / (DI / G);

  extern __shared__ __align__(16) unsigned char smem[];
  const TtLds lo(N, E, TT, OPT);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + lo.anc);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);
  int32_t* s_misc = reinterpret_cast<int32_t*>(smem + lo.misc);
  unsigned char* s_C = smem + lo.C;
  float* s_cbt = reinterpret_cast<float*>(smem + lo.cbt);
  unsigned char* s_B = smem + lo.X;
  float* s_xt = reinterpret_cast<float*>(smem + lo.X);
  uint8_t* s_nf = smem + lo.nf;
  float* s_m = reinterpret_cast<float*>(smem + lo.Mo);
  TIn* s_xw = reinterpret_cast<TIn*>(smem + lo.Y);
  TIn* s_xr = s_xw + 3 * kTtRows;
  float* s_So = reinterpret_cast<float*>(smem + lo.So);
  double* s_S2 = reinterpret_cast<double*>(smem + lo.S2);
  float* s_Ah = reinterpret_cast<float*>(smem + lo.Ah);
  float* s_dt = reinterpret_cast<float*>(smem + lo.dt);
  float* s_D = reinterpret_cast<float*>(smem + lo.D);
  float* s_cw = reinterpret_cast<float*>(smem + lo.cw);
  float* s_cb = reinterpret_cast<float*>(smem + lo.cb);
  const int rs = lo.row;

  // ---- the first block's state, in flight during the tree prologue ----
  typename SQ::Raw hq[NG];  // raw until the products take it
  {
    const TS* sin = reinterpret_cast<const TS*>(a.state) + (unit * DI + cw0 + wave * 16 + j) * (int64_t)N + 4 * k;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) hq[gg] = SQ::load(sin + 16 * gg);
  }

  // ---- tree prologue: parent[], C and B rows ----
  if (tid < kTtMaxT) s_parent[tid] = tid < T ? a.parent[(int64_t)b * T + tid] : 0;
  const unsigned char* Cg = reinterpret_cast<const unsigned char*>(a.C) + ((unit * T) * G + g) * (int64_t)N * E;
  const unsigned char* Bg = reinterpret_cast<const unsigned char*>(a.B) + ((unit * T) * G + g) * (int64_t)N * E;
  // (with the options the raw rows go to a staging area of their own)
  unsigned char* rawB = OPT ? smem + lo.R : s_B;
  unsigned char* rawC = OPT ? smem + lo.R + KT * lo.rawrow : s_C;
  for (int ci = tid; ci < KT * kChunks; ci += kTtThreads) {
    const int v = ci / kChunks, q = ci % kChunks;
    u32x4 c4 = u32x4{0u, 0u, 0u, 0u}, b4 = c4;  // zero rows past T
    if (v < T) {
      c4 = *reinterpret_cast<const u32x4*>(Cg + (int64_t)v * G * N * E + q * 16);
      b4 = *reinterpret_cast<const u32x4*>(Bg + (int64_t)v * G * N * E + q * 16);
    }
    *reinterpret_cast<u32x4*>(rawC + v * lo.rawrow + q * 16) = c4;
    *reinterpret_cast<u32x4*>(rawB + v * lo.rawrow + q * 16) = b4;
  }
  __syncthreads();
  if (wave == 0) {
    // validation by ballot (lane = node), then per node the root-path set and
    // the conv taps; the walks require -1 <= parent < node at every step, so
    // they end and stay in range even on an invalid tree
    bool bad = false;
    if (lane < T) {
      const int p = s_parent[lane];
      bad = lane == 0 ? p != -1 : (p < -1 || p >= lane || p < s_parent[lane - 1]);
    }
    const bool ok = __ballot(bad) == 0;
    uint64_t m = 0;
    int packed = 0;
    if (lane < T) {
      int u = lane, a1 = -1, a2 = -1, a3 = -1, depth = 0;
      for (int s = 0; s < kTtMaxT && u >= 0; ++s) {
        m |= 1ull << u;
        ++depth;
        const int p = s_parent[u];
        u = (p >= 0 && p < u) ? p : -1;
        a1 = s == 0 ? u : a1;
        a2 = s == 1 ? u : a2;
        a3 = s == 2 ? u : a3;
      }
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        const int an = jj == 1 ? a1 : (jj == 2 ? a2 : a3);
        // past the root: window row (W - 2) - (jj - depth), stored at row
        // 2 - (jj - depth) of the window-and-x rows
        const int code = an >= 0 ? an + 3 : 2 - (jj - depth);
        if (jj < W) packed |= code << (8 * (jj - 1));
      }
    }
    s_anc[lane] = m;  // zero past T
    s_cidx[lane] = packed;
    if (lane == 0) {
      s_misc[0] = ok ? 1 : 0;
      if (blockIdx.x == 0 && l == 0 && a.seq_status) a.seq_status[b] = ok ? SSM_TREE_OK : SSM_TREE_E_TREE;
    }
  }
  if constexpr (OPT) {
    // the B and C rows as float32: with the xBC conv, each node's row
    // convolved over its root path (taps past the root read the committed
    // window's B and C channels), with SiLU when set; thread = state column
    // n of B (i < N) or of C
    __syncthreads();  // the tap codes
    const TIn* wing = reinterpret_cast<const TIn*>(a.window) + unit * (W - 1) * (int64_t)CH;
    for (int i = tid; i < 2 * N; i += kTtThreads) {
      const bool isC = i >= N;
      const int n = isC ? i - N : i;
      const unsigned char* raw = isC ? rawC : rawB;
      unsigned char* dst = isC ? s_C : s_B;
      float w[4] = {0.f, 0.f, 0.f, 0.f}, bias = 0.f, win[3] = {0.f, 0.f, 0.f};
      if (d.xbc) {
        const int ch = DI + (isC ? G * N : 0) + g * N + n;
        const float* cw = a.prm.conv_w + ((int64_t)l * CH + ch) * W;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = jj < W ? cw[W - 1 - jj] : 0.0f;  // by taps back
        if (a.prm.conv_b) bias = a.prm.conv_b[(int64_t)l * CH + ch];
#pragma unroll
        for (int r = 0; r < 3; ++r)
          if (r < W - 1) win[r] = load_in(wing, (int64_t)r * CH + ch);
      }
      for (int v = 0; v < KT; ++v) {
        float z = 0.0f;
        if (v < T) {
          const float u0 = load_in(reinterpret_cast<const TIn*>(raw + v * lo.rawrow), n);
          if (d.xbc) {
            const int codes = s_cidx[v];
            z = fmaf(w[0], u0, bias);
#pragma unroll
            for (int jj = 1; jj < 4; ++jj) {
              if (jj < W) {
                // code >= 3: node code - 3; else window row code + W - 4
                const int code = (codes >> (8 * (jj - 1))) & 255;
                const float u = code >= 3 ? load_in(reinterpret_cast<const TIn*>(raw + (code - 3) * lo.rawrow), n)
                                          : (code + W - 4 == 0 ? win[0] : (code + W - 4 == 1 ? win[1] : win[2]));
                z = fmaf(w[jj], u, z);
              }
            }
            if (d.silu) z = silu_fast(z);
          } else {
            z = u0;
          }
        }
        reinterpret_cast<float*>(dst + v * rs)[n] = z;
      }
    }
    __syncthreads();
  }
  // C_v . B_u over the lower-triangular tile pairs, B rows as the A operand
  // and C rows as the B operand: lane (i + 16 k) ends with
  // (B_{16 tj + 4k + t} . C_{16 ti + i}) = CB[16 ti + i][16 tj + 4 k + t]
  for (int pi = wave; pi < TT * (TT + 1) / 2; pi += kTtWaves) {
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= pi) ++ti;
    const int tj = pi - ti * (ti + 1) / 2;
    f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
    const TR* brow = reinterpret_cast<const TR*>(s_B + (16 * tj + j) * rs) + 4 * k;
    const TR* crow = reinterpret_cast<const TR*>(s_C + (16 * ti + j) * rs) + 4 * k;
    if constexpr (sizeof(TR) == 2) {
      // bf16 rows are exact bf16 operands: k slots = state indices
      // 16 g + 4 k .. + 3 of column groups g = 2 m, 2 m + 1
#pragma unroll
      for (int m = 0; m < (NG + 1) / 2; ++m) {
        const u32x2 b0 = *reinterpret_cast<const u32x2*>(brow + 32 * m);
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(crow + 32 * m);
        u32x2 b1 = u32x2{0u, 0u}, c1 = b1;
        if (2 * m + 1 < NG) {
          b1 = *reinterpret_cast<const u32x2*>(brow + 32 * m + 16);
          c1 = *reinterpret_cast<const u32x2*>(crow + 32 * m + 16);
        }
        cb = mfma32(u32x4{b0.x, b0.y, b1.x, b1.y}, u32x4{c0.x, c0.y, c1.x, c1.y}, cb);
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const f32x4 bq = load4<TR>(brow + 16 * gg);
        const f32x4 cq = load4<TR>(crow + 16 * gg);
        cb = mfma4(bq.x, cq.x, cb);
        cb = mfma4(bq.y, cq.y, cb);
        cb = mfma4(bq.z, cq.z, cb);
        cb = mfma4(bq.w, cq.w, cb);
      }
    }
    *reinterpret_cast<f32x4*>(s_cbt + (16 * pi + j) * kPairStride + 4 * k) = cb;
  }
  __syncthreads();  // the B rows are dead from here: their space holds the conv outputs
  const bool tree_ok = s_misc[0] != 0;

  const TIn* xg = reinterpret_cast<const TIn*>(a.x) + unit * T * (int64_t)DI;
  const TIn* wg = reinterpret_cast<const TIn*>(a.window) + unit * (W - 1) * (int64_t)CH;
  const TIn* dtg = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * (int64_t)H;
  // a 64-channel block inside one head (P a multiple of 64): the head's dt,
  // S and exp(S) are formed here for all the workgroup's blocks (wave =
  // block, lane = node), and M once per block for all four waves
  const bool shared_m = P % kTtRows == 0;
  if (shared_m) {
    const int tid = opaque_tid();
    const int bw = __builtin_amdgcn_readfirstlane(tid / kWave), v = tid % kWave;
    if (bw < NBLK) {
      const int h = (cw0 + bw * kTtRows) / P;
      float dtv = 0.0f;  // zero past T
      if (v < T) dtv = softplus_hw(load_in(dtg, (int64_t)v * H + h) + a.prm.dt_bias[(int64_t)l * H + h]);
      int up = v < T ? s_parent[v] : -1;
      up = (up >= 0 && up < v) ? up : -1;  // (an invalid tree's output is discarded; keep indices in range)
      // S in fp64: down a 64-node chain it reaches ~-70, and M takes
      // differences of two such sums
      const double s2 = root_path_sum((double)(dtv * a.prm.A[(int64_t)l * H + h]), up, v) * 1.4426950408889634;
      s_dt[bw * kTtMaxT + v] = dtv;
      s_S2[bw * kTtMaxT + v] = s2;
      s_Ah[bw * kTtMaxT + v] = __builtin_amdgcn_exp2f((float)s2);
      if (v == 0) s_D[bw] = a.prm.D[(int64_t)l * H + h];
    }
  }
  // per-block inputs, loaded a block ahead into registers: raw x quads,
  // and by role the window rows and conv parameters (threads < 64) and the
  // head scalars (thread = head x node)
  constexpr int kXQ = (KT * (kTtRows / 4) + kTtThreads - 1) / kTtThreads;
  RawQ pxr[kXQ];
  // (raw values only: arithmetic on a loaded value would wait for the load at once)
  uint32_t pwin[3] = {0u, 0u, 0u}, pdt = 0u;
  float pcw[4] = {0.f, 0.f, 0.f, 0.f}, pcb = 0.f, pbias = 0.f, pA = 0.f, pD = 0.f;
  auto prefetch = [&](int blk) {
    const int tid = opaque_tid();
    const int c0 = cw0 + blk * kTtRows;
    const int h_lo = c0 / P;
    const int HW = (c0 + kTtRows - 1) / P - h_lo + 1;
#pragma unroll
    for (int it = 0; it < kXQ; ++it) {
      const int qi = tid + it * kTtThreads;
      const int v = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
      // rows past T repeat row T - 1: no tap reads them, and their own conv
      // output is discarded (an unconditional load keeps the register free
      // of a reset that would wait on every load in flight)
      const int vr = v < T ? v : T - 1;
      pxr[it] = *reinterpret_cast<const RawQ*>(xg + (int64_t)vr * DI + c0 + c4);
    }
    if (tid < kTtRows) {
      const int c = c0 + tid;
#pragma unroll
      for (int r = 0; r < 3; ++r)
        if (r < W - 1) pwin[r] = raw_bits<TIn>(wg + (int64_t)r * CH + c);
      const float* cw = a.prm.conv_w + ((int64_t)l * CH + c) * W;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t < W) pcw[t] = cw[W - 1 - t];  // tap t weighs the node t steps up the path
      if (a.prm.conv_b) pcb = a.prm.conv_b[(int64_t)l * CH + c];
    }
    const int hh = tid / kTtMaxT, v = tid % kTtMaxT;  // 4 heads x 64 nodes
    if (!shared_m && hh < HW && v < T) {
      const int h = h_lo + hh;
      pdt = raw_bits<TIn>(dtg + (int64_t)v * H + h);
      pbias = a.prm.dt_bias[(int64_t)l * H + h];
      pA = a.prm.A[(int64_t)l * H + h];
    }
    if (!shared_m && tid < HW) pD = a.prm.D[(int64_t)l * H + h_lo + tid];
  };
  // a block's inputs from the prefetch registers into LDS: x and window
  // rows, conv parameters, and (blocks of several heads) the heads' dt, dt A
  // and D, dt and D double-buffered by block parity
  auto deliver = [&](int blk) {
    const int tid = opaque_tid();
    const int c0 = cw0 + blk * kTtRows;
    const int h_lo = c0 / P;
    const int HW = (c0 + kTtRows - 1) / P - h_lo + 1;
#pragma unroll
    for (int it = 0; it < kXQ; ++it) {
      const int qi = tid + it * kTtThreads;
      const int v = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
      if (qi < KT * (kTtRows / 4)) *reinterpret_cast<RawQ*>(s_xr + v * kTtRows + c4) = pxr[it];
    }
    if (tid < kTtRows) {
#pragma unroll
      for (int r = 0; r < 3; ++r)
        if (r < W - 1) s_xw[(4 - W + r) * kTtRows + tid] = from_bits<TIn>(pwin[r]);
#pragma unroll
      for (int r = 0; r < 3; ++r)  // rows above the window: read by unused taps (weight zero), so zero
        if (r < 4 - W) s_xw[r * kTtRows + tid] = from_bits<TIn>(0u);
#pragma unroll
      for (int t = 0; t < 4; ++t) s_cw[t * kTtRows + tid] = pcw[t];  // zero past W
      s_cb[tid] = pcb;
    }
    if (!shared_m) {
      const int hh = tid / kTtMaxT, v = tid % kTtMaxT;
      float dtv = 0.0f, so = 0.0f;
      if (hh < HW && v < T) {
        dtv = softplus_hw((sizeof(TIn) == 2 ? __uint_as_float(pdt << 16) : __uint_as_float(pdt)) + pbias);
        so = dtv * pA;
      }
      s_dt[((blk & 1) * 4 + hh) * kTtMaxT + v] = dtv;
      s_So[hh * kTtMaxT + v] = so;
      if (tid < HW) s_D[(blk & 1) * 4 + tid] = pD;
    }
  };
  // Order within a block: [S, conv, M] barrier [next block's delivery, C . h
  // (loading the next block's state), prefetch of the block after, path
  // terms and y] barrier.  Every wait on a prefetch register then covers
  // only loads issued at least a phase earlier (the wait counter also
  // counts the y stores).
  prefetch(0);
  deliver(0);
  if (NBLK > 1) prefetch(1);
  for (int blk = 0; blk < NBLK; ++blk) {
    const int c0 = cw0 + blk * kTtRows;
    const int h_lo = c0 / P;
    __syncthreads();  // the block's inputs are in LDS; the previous block's path terms are done
    if (!shared_m) {
      // S along each root path (base-2 units), accumulated in fp64: down a
      // 64-node chain it reaches ~-70, and the decay between two nodes is
      // the difference of two such sums, which fp32 would leave with ~1e-5
      // of cancellation error; fp64 keeps the difference exact to the fp32
      // rounding of its own terms.  Wave = head, lane = node.
      const int tid = opaque_tid();
      const int hh = tid / kTtMaxT, v = tid % kTtMaxT;
      int up = v < T ? s_parent[v] : -1;
      up = (up >= 0 && up < v) ? up : -1;  // (an invalid tree's output is discarded; keep indices in range)
      const double s2 = root_path_sum((double)s_So[hh * kTtMaxT + v], up, v) * 1.4426950408889634;  // zero past T
      s_S2[hh * kTtMaxT + v] = s2;
      s_Ah[hh * kTtMaxT + v] = __builtin_amdgcn_exp2f((float)s2);
    }
    uint32_t nf_any = 0;  // non-finite bits of this thread's conv outputs, or-ed
    {
      // causal conv over each node's root path, lane = channel, wave = node
      // quads wave, wave + 4, ...: a node's tap sources are the same for the
      // whole wave, and a quad leaves as one 16-byte store
      const int tid = opaque_tid();
      const int cl = tid & (kWave - 1);
      const int wq = __builtin_amdgcn_readfirstlane(tid / kWave);
      float wt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) wt[t] = s_cw[t * kTtRows + cl];
      const float cbv = s_cb[cl];
      // every tap read of the wave's TT node quads is issued before any
      // arithmetic or store (the stores could alias the reads as far as the
      // compiler can tell, which would serialise quad after quad); unused
      // taps (weight zero) and nodes past T read zeroed rows
      u32x4 codes4[TT];
#pragma unroll
      for (int it = 0; it < TT; ++it) codes4[it] = *reinterpret_cast<const u32x4*>(s_cidx + 4 * (wq + kTtWaves * it));
      float xs[TT][4][4];
#pragma unroll
      for (int it = 0; it < TT; ++it) {
        const int q = wq + kTtWaves * it;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t codes = __builtin_amdgcn_readfirstlane(codes4[it][r]);
          xs[it][r][0] = load_in(s_xr, (4 * q + r) * kTtRows + cl);
#pragma unroll
          for (int t = 1; t < 4; ++t)
            xs[it][r][t] = load_in(s_xw, ((codes >> (8 * (t - 1))) & 255) * kTtRows + cl);
        }
      }
#pragma unroll
      for (int it = 0; it < TT; ++it) {
        const int q = wq + kTtWaves * it;
        f32x4 xq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = fmaf(wt[0], xs[it][r][0], cbv);
#pragma unroll
          for (int t = 1; t < 4; ++t) z = fmaf(wt[t], xs[it][r][t], z);
          xq[r] = z;
        }
        if (d.silu) {  // (a uniform branch: a select would run the transcendentals either way)
#pragma unroll
          for (int r = 0; r < 4; ++r) xq[r] = silu_fast(xq[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) xq[r] = 4 * q + r < T ? xq[r] : 0.0f;
        const uint32_t nfb = nonfinite_quad(xq);
        s_nf[cl * (kTtMaxT / 4) + q] = (uint8_t)nfb;
        nf_any |= nfb;
        // conv outputs [channel][node] in the MFMA B-operand layout: quad q
        // (nodes 4 q .. 4 q + 3) of channel row cl sits at quad q ^ (cl & 15),
        // so that the 16 channels a wave reads at once fall on different banks
        *reinterpret_cast<f32x4*>(s_xt + cl * kTtMaxT + 4 * (q ^ (cl & 15))) = xq;
      }
    }

    // ---- M[v][u] of the block's head when shared: thread = (tile pair
    // slot, row, column quad) ----
    if (shared_m) {
      const int tid = opaque_tid();
      const int slot = __builtin_amdgcn_readfirstlane(tid / kWave), r = (tid >> 2) & 15, cq = tid & 3;
      const double* S2w = s_S2 + blk * kTtMaxT;
      const float* dtw = s_dt + blk * kTtMaxT;
      const float Dh0 = s_D[blk];
      // tile pairs dealt round the waves, each wave's list fixed at compile time
      switch (slot) {
        case 0: m_form_slot<TT, 0>(s_m, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
        case 1: m_form_slot<TT, 1>(s_m, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
        case 2: m_form_slot<TT, 2>(s_m, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
        default: m_form_slot<TT, 3>(s_m, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
      }
    }
    // conv outputs and M are complete; x rows, conv parameters and dt A are free
    const bool xt_nonfinite = __syncthreads_or(nf_any != 0) != 0;
    if (blk + 1 < NBLK) deliver(blk + 1);

    // ---- C . h0 on the matrix cores: lane (c + 16 q) ends with (C_{16 ti + 4q + r} . h_c) ----
    const int ln = opaque_tid() & (kWave - 1), j = ln & 15, k = ln >> 4;
    f32x4 acc[TT];
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) acc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool more = blk + 1 < NBLK;
    const TS* nsin = reinterpret_cast<const TS*>(a.state) + (unit * DI + c0 + kTtRows + wave * 16 + j) * (int64_t)N + 4 * k;
    if constexpr (sizeof(TR) == 2) {
      // bf16 C rows against the state, two column groups per product: a
      // bf16 state is an exact operand as it stands; an fp32 state is split
      // into three bf16 terms
#pragma unroll
      for (int m = 0; m < (NG + 1) / 2; ++m) {
        const bool two = 2 * m + 1 < NG;
        u32x4 h0, h1, h2;
        if constexpr (sizeof(TS) == 2) {
          const u32x2 lo = hq[2 * m], hi = two ? hq[2 * m + 1] : u32x2{0u, 0u};
          h0 = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          split3(hq[2 * m], two ? hq[2 * m + 1] : f32x4{0.f, 0.f, 0.f, 0.f}, h0, h1, h2);
        }
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) {
          const TR* crow = reinterpret_cast<const TR*>(s_C + (16 * ti + j) * rs) + 32 * m + 4 * k;
          const u32x2 c0 = *reinterpret_cast<const u32x2*>(crow);
          const u32x2 c1 = two ? *reinterpret_cast<const u32x2*>(crow + 16) : u32x2{0u, 0u};
          const u32x4 ca = u32x4{c0.x, c0.y, c1.x, c1.y};
          if constexpr (sizeof(TS) != 2) {
            acc[ti] = mfma32(ca, h2, acc[ti]);
            acc[ti] = mfma32(ca, h1, acc[ti]);
          }
          acc[ti] = mfma32(ca, h0, acc[ti]);
        }
        // these column groups are consumed: the next block's take their registers
        if (more) {
          hq[2 * m] = SQ::load(nsin + 32 * m);
          if (two) hq[2 * m + 1] = SQ::load(nsin + 32 * m + 16);
        }
        asm volatile("" ::: "memory");
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const f32x4 h = SQ::to_f32(hq[gg]);
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) {
          const f32x4 cq = load4<TR>(reinterpret_cast<const TR*>(s_C + (16 * ti + j) * rs) + 16 * gg + 4 * k);
          acc[ti] = mfma4(cq.x, h.x, acc[ti]);
          acc[ti] = mfma4(cq.y, h.y, acc[ti]);
          acc[ti] = mfma4(cq.z, h.z, acc[ti]);
          acc[ti] = mfma4(cq.w, h.w, acc[ti]);
        }
        // this column group is consumed: the next block's takes its registers
        if (more) hq[gg] = SQ::load(nsin + 16 * gg);
        // one column group's C operands at a time (hoisting all of them would
        // take 4 NG x 4 registers)
        asm volatile("" ::: "memory");
      }
    }

    if (blk + 2 < NBLK) prefetch(blk + 2);

    // ---- the path terms M[v][u] x~_u (u in tiles tj <= ti), with the diagonal D ----
    const int row = wave * 16 + j;                   // this lane's channel in the block
    const int hl = (c0 + wave * 16) / P - h_lo;      // the wave's head
    const float Dh = s_D[(blk & 1) * 4 + hl];
    const double* S2h = s_S2 + hl * kTtMaxT;
    const float* dth = s_dt + ((blk & 1) * 4 + hl) * kTtMaxT;
    const float* Ahh = s_Ah + (shared_m ? blk : hl) * kTtMaxT;
    float* yrow = a.y + unit * T * (int64_t)DI + c0 + row;
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) {
      const int vi = 16 * ti + j;                    // the M row (node) this lane supplies
      const uint64_t ancm = shared_m ? 0 : s_anc[vi];
      f32x4 y = *reinterpret_cast<const f32x4*>(Ahh + 16 * ti + 4 * k) * acc[ti];
#pragma unroll
      for (int tj = 0; tj <= ti; ++tj) {
        const int u0 = 16 * tj + 4 * k;
        const int pq = (16 * pair_of(ti, tj) + j) * kPairStride + 4 * k;  // this lane's quad of the pair
        const float* cbr = s_cbt + pq;
        const f32x4 mop = shared_m    ? *reinterpret_cast<const f32x4*>(s_m + pq)
                          : tj == ti ? m_quad<true>(vi, u0, S2h, dth, ancm, cbr, Dh)
                                     : m_quad<false>(vi, u0, S2h, dth, ancm, cbr, Dh);
        const f32x4 xq = *reinterpret_cast<const f32x4*>(s_xt + row * kTtMaxT + 4 * ((4 * tj + k) ^ (row & 15)));
        y = mfma4(mop.x, xq.x, y);
        y = mfma4(mop.y, xq.y, y);
        y = mfma4(mop.z, xq.z, y);
        y = mfma4(mop.w, xq.w, y);
      }
      // lane (c + 16 k) holds nodes 16 ti + 4 k + r of channel row: each
      // store covers 16 channels (64 bytes) of four nodes; the four waves
      // fill each node's 256-byte row segment
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 16 * ti + 4 * k + r;
        float yv = y[r];
        if constexpr (OPT)  // the gate: y silu(z)
          if (a.z) yv *= silu_fast(load_in(reinterpret_cast<const TIn*>(a.z) + (unit * T + v) * (int64_t)DI + c0 + row, 0));
        if (v < T) yrow[(int64_t)v * DI] = tree_ok ? yv : __builtin_nanf("");
      }
      // one node tile's operands at a time: hoisting the LDS reads of all
      // tiles above the loop would take most of the register file
      asm volatile("" ::: "memory");
    }
    if (xt_nonfinite) {  // (rare) y_v not finite where v's root path holds a non-finite x~_u
      const uint64_t nfm = nonfinite_nodes(s_nf, row);
      for (int v = 4 * k; v < T; v = (v & 3) == 3 ? v + 13 : v + 1)  // this lane's nodes 16 ti + 4 k + r
        if (s_anc[v] & nfm) yrow[(int64_t)v * DI] = __builtin_nanf("");
    }
  }
}

// ---------------------------------------------------------------------------
// The same verify with the waves split by role, for blocks that lie in one
// head (P a multiple of 64) and at least 8 blocks per workgroup.  Waves 0-3
// (producers) run the vector work of block ph: the conv and M, then deliver
// block ph + 1's inputs and issue block ph + 3's loads (two register sets).
// Waves 4-7 (consumers) run the matrix work: C . h0 of block ph, then the
// path terms and y of block ph - 1.  Conv outputs, M, the x rows and the
// conv parameters are double-buffered by block parity, so one barrier per
// phase separates writers from readers, and each SIMD holds one wave of each
// role whose vector and matrix instructions overlap.  Every phase of a
// role's loop issues the same memory operations (unconditional loads from
// clamped addresses, stores past the range dropped by buffer resources),
// so the compiler's waits count them and loads stay in flight across the
// barrier.
//
// With CM the kernel is also the round of ssm_tree_commit_verify (SpecMamba
// page sec. 3.1, the accepted path recomputed from the stored dt, B and x):
// the previous tree's path is committed into each block's state before its
// C . h0, in closed form on the matrix cores,
//   h_new^T = exp(P_last) h^T + Bp^T W,  W[q][c] = exp(P_last - P_q) dt_q x~_q[c],
// P_q the fp64 prefix sum of dt * A along the path (the producers form W
// for the first 16 positions, the consumers for the rest), the state and
// the committed window are written, and the next tree is verified from the
// committed state.
// ---------------------------------------------------------------------------

namespace {

constexpr int kWsWaves = 8;
constexpr int kWsThreads = kWsWaves * kWave;
constexpr int kWsMaxBlk = 20;   // blocks per workgroup, the round (an even count)
constexpr int kWsMaxBlkV = 40;  // blocks per workgroup, verify alone (its per-block tables have room)
// the commit's first 16 path positions: their weighted conv outputs are
// formed by the producers, [channel][position] with a padded stride (the 16
// lanes that read one position read 16 channels on distinct banks)
constexpr int kWqPos = 16;
constexpr int kWqStride = kWqPos + 1;

struct TtWsLds {
  int parent, anc, cidx, misc, C, cbt, X, Y, Mo, S2, Ah, dt, D, cw, cb, nf, nff, total, row, xbuf, ybuf, mbuf, cwbuf;
  // cm: the commit's own arrays (offset 0 when unused)
  int pparent, path, Pr, wt, at, Wq;
  __host__ __device__ TtWsLds(int N, int E, int TT, bool cm, int nblk) {
    const int KT = 16 * TT, pair_bytes = 4 * 16 * kPairStride * pair_of(TT, 0);
    int o = 0;
    row = N * E + 16;
    parent = o; o += 4 * kTtMaxT;
    anc = o; o += 8 * kTtMaxT;
    cidx = o; o += 4 * kTtMaxT;
    misc = o; o += 16;
    C = o; o += KT * row;
    cbt = o; o += pair_bytes;
    // two conv-output buffers [channel][node]; the B rows (KT rows) sit here
    // until the C . B dots exist
    xbuf = 4 * kTtRows * kTtMaxT;
    X = o; o += 2 * xbuf > KT * row ? 2 * xbuf : KT * row;
    ybuf = ((3 + KT) * kTtRows * E + 15) / 16 * 16;  // window and x rows, raw
    Y = o; o += 2 * ybuf;
    mbuf = pair_bytes;
    Mo = o; o += 2 * mbuf;
    S2 = o; o += 8 * nblk * kTtMaxT;        // [block][node] fp64
    Ah = o; o += 4 * nblk * kTtMaxT;        // [block][node]
    dt = o; o += 4 * nblk * kTtMaxT;        // [block][node]
    D = o; o += 4 * nblk;
    cwbuf = 4 * 4 * kTtRows;
    cw = o; o += 2 * cwbuf;                  // [parity][tap][channel]
    cb = o; o += 2 * 4 * kTtRows;            // [parity][channel]
    nf = o; o += 2 * kTtRows * kTtMaxT / 4;  // [parity][channel][node quad] codes of non-finite conv outputs
    nff = o; o += 4 * (nblk + 1);            // [phase] whether the block's conv outputs hold a non-finite value
    pparent = path = Pr = wt = at = Wq = 0;
    if (cm) {
      pparent = o; o += 4 * kTtMaxT;         // the committed tree's parent[]
      path = o; o += 4 * kTtMaxT;            // the accepted path
      Pr = o; o += 2 * ybuf;                 // [parity] old window rows and the path's x rows, raw
      wt = o; o += 4 * nblk * kTtMaxT;       // [block][path position] exp(P_last - P_q) dt_q
      at = o; o += 4 * nblk;                 // [block] exp(P_last)
      Wq = o; o += 2 * 4 * kTtRows * kWqStride;  // [parity][channel][position < 16] weight * x~ (producers)
      // the path's B rows (raw, zero past its length) take the C rows' place
      // once the matrix-core operands hold those
    }
    total = o;
  }
};

}  // namespace

template <typename TIn, typename TS, int NG, int TT, bool CM>
__global__ void __launch_bounds__(kWsThreads) verify_tt_ws_kernel(CommitVerifyArgs a, int NBLK) {
  typedef StateQuad<TS> SQ;
  constexpr int N = 16 * NG;
  constexpr int E = (int)sizeof(TIn);
  constexpr int KT = 16 * TT;
  typedef typename Raw4<E>::T RawQ;
  constexpr int kChunks = N * E / 16;
  const Dims d = a.d;
  const int T = d.T, P = d.P, H = d.H, W = d.W, DI = d.d_in, G = d.G, CH = d.CH;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool producer = wave < 4;
  const int rw = wave & 3;  // the wave's index within its role
  const int j = lane & 15, k = lane >> 4;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int cw0 = blockIdx.x * NBLK * kTtRows;
  const int g = cw0 / (DI / G);

  // the commit's path B rows replace the C rows, which the consumers then
  // hold in registers
  static_assert(!CM || (E == 2 && NG <= 8), "commit: bf16 inputs, d_state <= 128");

  extern __shared__ __align__(16) unsigned char smem[];
  const TtWsLds lo(N, E, TT, CM, NBLK);
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem + lo.parent);
  int32_t* s_pparent = reinterpret_cast<int32_t*>(smem + lo.pparent);
  int32_t* s_path = reinterpret_cast<int32_t*>(smem + lo.path);
  float* s_wt = reinterpret_cast<float*>(smem + lo.wt);
  float* s_at = reinterpret_cast<float*>(smem + lo.at);
  auto s_pr = [&](int par) { return reinterpret_cast<TIn*>(smem + lo.Pr + par * lo.ybuf); };
  int32_t* s_nff = reinterpret_cast<int32_t*>(smem + lo.nff);
  auto s_wq = [&](int par) { return reinterpret_cast<float*>(smem + lo.Wq + par * 4 * kTtRows * kWqStride); };
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + lo.anc);
  int32_t* s_cidx = reinterpret_cast<int32_t*>(smem + lo.cidx);
  int32_t* s_misc = reinterpret_cast<int32_t*>(smem + lo.misc);
  unsigned char* s_C = smem + lo.C;
  float* s_cbt = reinterpret_cast<float*>(smem + lo.cbt);
  unsigned char* s_B = smem + lo.X;
  double* s_S2 = reinterpret_cast<double*>(smem + lo.S2);
  float* s_Ah = reinterpret_cast<float*>(smem + lo.Ah);
  float* s_dt = reinterpret_cast<float*>(smem + lo.dt);
  float* s_D = reinterpret_cast<float*>(smem + lo.D);
  const int rs = lo.row;
  auto s_xt = [&](int par) { return reinterpret_cast<float*>(smem + lo.X + par * lo.xbuf); };
  auto s_nf = [&](int par) { return smem + lo.nf + par * (kTtRows * kTtMaxT / 4); };
  auto s_xw = [&](int par) { return reinterpret_cast<TIn*>(smem + lo.Y + par * lo.ybuf); };
  auto s_m = [&](int par) { return reinterpret_cast<float*>(smem + lo.Mo + par * lo.mbuf); };
  auto s_cw = [&](int par) { return reinterpret_cast<float*>(smem + lo.cw + par * lo.cwbuf); };
  auto s_cb = [&](int par) { return reinterpret_cast<float*>(smem + lo.cb + par * 4 * kTtRows); };

  // ---- consumers: the first block's state, in flight during the prologue ----
  typename SQ::Raw hq[NG];
  if (!producer) {
    const TS* sin = reinterpret_cast<const TS*>(a.state_in) + (unit * DI + cw0 + rw * 16 + j) * (int64_t)N + 4 * k;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) hq[gg] = SQ::load(sin + 16 * gg);
  }
  // ---- every wave's blocks (wave, wave + 8): the nodes' dt_raw (lane =
  // node) and the head's parameters, issued at entry so that the head data
  // below waits on no load ----
  constexpr int kHB = ((CM ? kWsMaxBlk : kWsMaxBlkV) + kWsWaves - 1) / kWsWaves;
  uint32_t hdt[kHB], hdtp[kHB];
  float hbias[kHB], hA[kHB], hD[kHB];
  {
    const TIn* dtg0 = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * (int64_t)H;
#pragma unroll
    for (int i = 0; i < kHB; ++i) {
      const int bw = wave + kWsWaves * i;
      const int h = (cw0 + (bw < NBLK ? bw : 0) * kTtRows) / P;
      hdt[i] = raw_bits<TIn>(dtg0 + (int64_t)(lane < T ? lane : T - 1) * H + h);
      hbias[i] = a.prm.dt_bias[(int64_t)l * H + h];
      hA[i] = a.prm.A[(int64_t)l * H + h];
      hD[i] = a.prm.D[(int64_t)l * H + h];
      hdtp[i] = 0u;
    }
  }

  const TIn* xg = reinterpret_cast<const TIn*>(a.x) + unit * T * (int64_t)DI;
  const TIn* wg = reinterpret_cast<const TIn*>(a.window_in) + unit * (W - 1) * (int64_t)CH;
  // buffer resources over this unit's y rows and committed window: an offset
  // past the range drops the store, so that stores of padded nodes or unused
  // window rows need no branch (a branch around a store changes the count
  // of outstanding memory operations from phase to phase, and the compiler
  // then waits for all of them before the next block's state is used)
  constexpr int kOutOfRange = 0x7FFFFFF0;
  const __amdgpu_buffer_rsrc_t y_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.y + unit * T * (int64_t)DI, (short)0, T * DI * 4, kBufWord3);
  const __amdgpu_buffer_rsrc_t wo_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      CM && W > 1 ? reinterpret_cast<TIn*>(a.window_out) + unit * (W - 1) * (int64_t)CH : nullptr, (short)0,
      CM && W > 1 ? (W - 1) * CH * E : 0, kBufWord3);
  // ---- tree prologue (all waves): parent[], C and B rows ----
  if (tid < kTtMaxT) s_parent[tid] = tid < T ? a.parent[(int64_t)b * T + tid] : 0;
  if (tid <= NBLK) s_nff[tid] = 0;
  if constexpr (CM) {
    if (tid < kTtMaxT) {
      s_pparent[tid] = tid < T ? a.parent_prev[(int64_t)b * T + tid] : 0;
      s_path[tid] = tid < T ? a.path[(int64_t)b * T + tid] : 0;
    }
    if (tid == kWsThreads - 1) s_misc[3] = a.path_len[b];
  }
  const unsigned char* Cg = reinterpret_cast<const unsigned char*>(a.C) + ((unit * T) * G + g) * (int64_t)N * E;
  const unsigned char* Bg = reinterpret_cast<const unsigned char*>(a.B) + ((unit * T) * G + g) * (int64_t)N * E;
  for (int ci = tid; ci < KT * kChunks; ci += kWsThreads) {
    const int v = ci / kChunks, q = ci % kChunks;
    u32x4 c4 = u32x4{0u, 0u, 0u, 0u}, b4 = c4;
    if (v < T) {
      c4 = *reinterpret_cast<const u32x4*>(Cg + (int64_t)v * G * N * E + q * 16);
      b4 = *reinterpret_cast<const u32x4*>(Bg + (int64_t)v * G * N * E + q * 16);
    }
    *reinterpret_cast<u32x4*>(s_C + v * rs + q * 16) = c4;
    *reinterpret_cast<u32x4*>(s_B + v * rs + q * 16) = b4;
  }
  __syncthreads();
  // ---- producers' per-block inputs, a block ahead in registers ----
  constexpr int kXQ = (KT * (kTtRows / 4) + kTtThreads - 1) / kTtThreads;  // (256 producer threads)
  // the commit: the old window rows and the path's x rows, rows 0..2 and
  // 3.. of the block's path buffer (the window right-aligned: element e of
  // (old window, path rows) sits at row 4 - W + e)
  constexpr int kPQ = CM ? ((3 + KT) * (kTtRows / 4) + kTtThreads - 1) / kTtThreads : 1;
  // one block's prefetched inputs; two sets, so that a block's loads are
  // issued two phases before its delivery
  struct PRegs {
    RawQ x[kXQ];
    RawQ p[kPQ];
    uint32_t win[3];
    uint32_t q7[CM ? 7 : 1];  // the rows of this thread's channel that its 4 path positions tap
    float cw[4], cb;
  };
  PRegs pra, prb;
  // path length applied (0 when nothing is committed): first the length as
  // given, clamped, so that blocks 0 and 1 are fetched before the path is
  // validated; a failed commit (rare) sets 0 and fetches them again
  int clen = CM ? (s_misc[3] < 0 ? 0 : (s_misc[3] > T ? T : s_misc[3])) : 0;
  auto spath = [&](int q) {  // a path node, clamped into the tree (an invalid path is refetched)
    const int v = s_path[q];
    return (v >= 0 && v < T) ? v : 0;
  };
  const TIn* xpg = CM ? reinterpret_cast<const TIn*>(a.x_prev) + unit * T * (int64_t)DI : nullptr;
  // Every prefetch load is unconditional, from a clamped address where its
  // value is not needed (selected away at delivery): a load under a branch
  // makes the compiler wait for it where the branches join, which turned
  // the one-phase lead into a wait inside the same phase.  Unused lanes of
  // a load all read one address.
  const int pch = opaque_tid() & (kTtRows - 1);  // the channel of the per-channel rows (all four waves)
  // The sources of a thread's path and window rows are the same for every
  // block but for the block's channel offset: resolved once here (through
  // the path in LDS), so that a prefetch issues its loads without waiting on
  // LDS reads.  Each points at the row's element for channel offset 0 of
  // block 0 (plus the thread's channel within the block).
  // (as element offsets from x_prev's unit, or from the window's where bit
  // it of pwin_rows is set: 32-bit offsets keep the registers down)
  int psrc[kPQ];
  uint32_t pwin_rows = 0;
  const TIn* wsrc[3];
  int qsrc[CM ? 7 : 1];  // (offsets as psrc; window rows flagged by bit 8 + m of pwin_rows)
  auto resolve_sources = [&]() {
    pwin_rows = 0;
    const int ptid = opaque_tid();
#pragma unroll
    for (int it = 0; it < kPQ; ++it) {
      psrc[it] = cw0;  // (unused rows: row 0 of the previous tree's x)
      if constexpr (CM) {
        const int qi = ptid + it * kTtThreads;
        const int rr = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
        if (rr >= 3 && rr < 3 + clen) psrc[it] = spath(rr - 3) * DI + cw0 + c4;
        if (rr < 3 && rr >= 4 - W) {
          psrc[it] = (rr - (4 - W)) * CH + cw0 + c4;
          pwin_rows |= 1u << it;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int c = cw0 + pch;
      wsrc[r] = xg + c;  // (unused taps)
      if (r < W - 1) {
        wsrc[r] = wg + (int64_t)r * CH + c;
        if constexpr (CM) {  // the committed window: element clen + r of (old window, path rows)
          const int e = clen + r;
          wsrc[r] = e < W - 1 ? wg + (int64_t)e * CH + c : xpg + (int64_t)spath(e - (W - 1)) * DI + c;
        }
      }
    }
    // the commit's first 16 path positions, producer thread (channel pch,
    // positions 4 pg .. 4 pg + 3, pg = its wave): they tap element
    // q + W - 1 - t of (old window, path rows), i.e. rows 4 pg .. 4 pg + 6 of
    // the block's path buffer (row 4 - W + e holds element e)
    const int pg = ptid >> 6;
#pragma unroll
    for (int m = 0; m < (CM ? 7 : 1); ++m) {
      qsrc[m] = cw0 + pch;  // (unused rows)
      if constexpr (CM) {
        const int rr = 4 * pg + m;
        if (rr >= 3 && rr < 3 + clen) qsrc[m] = spath(rr - 3) * DI + cw0 + pch;
        if (rr < 3 && rr >= 4 - W) {
          qsrc[m] = (rr - (4 - W)) * CH + cw0 + pch;
          pwin_rows |= 1u << (8 + m);
        }
      }
    }
  };
  resolve_sources();
  const float* cwb = a.prm.conv_w + ((int64_t)l * CH + cw0 + pch) * W;
  const float* cbb = a.prm.conv_b ? a.prm.conv_b + (int64_t)l * CH + cw0 + pch : cwb;
  auto prefetch = [&](int blk, PRegs& R) {
    const int ptid = opaque_tid();  // < 256
    const int c0 = cw0 + blk * kTtRows, boff = blk * kTtRows;
#pragma unroll
    for (int it = 0; it < kXQ; ++it) {
      const int qi = ptid + it * kTtThreads;
      const int v = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
      const int vr = v < T ? v : T - 1;  // rows past T repeat row T - 1 (never a tap source)
      R.x[it] = *reinterpret_cast<const RawQ*>(xg + (int64_t)vr * DI + c0 + c4);
    }
    if constexpr (CM) {
#pragma unroll
      for (int it = 0; it < kPQ; ++it)
        R.p[it] = *reinterpret_cast<const RawQ*>(((pwin_rows >> it) & 1 ? wg : xpg) + psrc[it] + boff);
      // (the aligned dword holding the element: the rows start at even elements)
#pragma unroll
      for (int m = 0; m < 7; ++m)
        R.q7[m] = *reinterpret_cast<const uint32_t*>(((pwin_rows >> (8 + m)) & 1 ? wg : xpg) + qsrc[m] + boff -
                                                     (pch & 1));
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      // bf16: the aligned dword holding the element (the rows start at even
      // elements), its half picked at delivery
      const TIn* src = wsrc[r] + boff;
      R.win[r] = E == 2 ? *reinterpret_cast<const uint32_t*>(src - (pch & 1)) : raw_bits<TIn>(src);
    }
    const float* cwp = cwb + (int64_t)boff * W;
#pragma unroll
    for (int t = 0; t < 4; ++t) R.cw[t] = cwp[t < W ? W - 1 - t : 0];
    R.cb = (a.prm.conv_b ? cbb + boff : cwp)[0];
  };
  auto deliver = [&](int blk, PRegs& R) {
    const int ptid = opaque_tid();
    const int par = blk & 1;
    TIn* xw = s_xw(par);
    TIn* xr = xw + 3 * kTtRows;
#pragma unroll
    for (int it = 0; it < kXQ; ++it) {
      const int qi = ptid + it * kTtThreads;
      const int v = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
      if (qi < KT * (kTtRows / 4)) *reinterpret_cast<RawQ*>(xr + v * kTtRows + c4) = R.x[it];
    }
    if constexpr (CM) {
      // the weighted conv outputs W[q][c] = exp(P_last - P_q) dt_q x~_q[c] of
      // this thread's channel at positions 4 pg .. 4 pg + 3 (zero past the
      // path; a delivery past the last block writes a buffer nobody reads)
      {
        const int pg = ptid >> 6, wb = blk < NBLK ? blk : NBLK - 1;
        float xv[7];
#pragma unroll
        for (int m = 0; m < 7; ++m) xv[m] = __uint_as_float(((R.q7[m] >> (16 * (pch & 1))) & 0xFFFFu) << 16);
        float* wq = s_wq(par) + pch * kWqStride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 4 * pg + i;
          float z = fmaf(R.cw[0], xv[i + 3], a.prm.conv_b ? R.cb : 0.0f);
#pragma unroll
          for (int t = 1; t < 4; ++t)
            if (t < W) z = fmaf(R.cw[t], xv[i + 3 - t], z);
          const float xt = d.silu ? silu_fast(z) : z;
          wq[q] = q < clen ? s_wt[wb * kTtMaxT + q] * xt : 0.0f;
        }
      }
      TIn* pr = s_pr(par);
#pragma unroll
      for (int it = 0; it < kPQ; ++it) {
        const int qi = ptid + it * kTtThreads;
        const int rr = qi / (kTtRows / 4), c4 = (qi % (kTtRows / 4)) * 4;
        if ((rr >= 3 && rr < 3 + clen) || (rr < 3 && rr >= 4 - W))
          *reinterpret_cast<RawQ*>(pr + rr * kTtRows + c4) = R.p[it];
      }
    }
    if (ptid < kTtRows) {
      uint32_t win[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) win[r] = E == 2 ? (R.win[r] >> (16 * (ptid & 1))) & 0xFFFFu : R.win[r];
#pragma unroll
      for (int r = 0; r < 3; ++r)
        if (r < W - 1) xw[(4 - W + r) * kTtRows + ptid] = from_bits<TIn>(win[r]);
#pragma unroll
      for (int r = 0; r < 3; ++r)
        if (r < 4 - W) xw[r * kTtRows + ptid] = from_bits<TIn>(0u);
#pragma unroll
      for (int t = 0; t < 4; ++t) s_cw(par)[t * kTtRows + ptid] = t < W ? R.cw[t] : 0.0f;
      s_cb(par)[ptid] = a.prm.conv_b ? R.cb : 0.0f;
      if constexpr (CM) {  // the committed window leaves with its block
        // buffer stores: rows past W - 1 and the blocks past the last (the
        // loop delivers one) fall outside the range and are dropped, so that
        // every phase issues the same memory operations
        const uint32_t c = cw0 + blk * kTtRows + ptid;
#pragma unroll
        for (int r = 0; r < 3; ++r)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)win[r], wo_rsrc,
                                                blk < NBLK ? (int)(((uint32_t)r * CH + c) * 2u) : kOutOfRange, 0, 0);
      }
    }
  };
  if (producer) {  // blocks 0 and 1 in flight through the rest of the prologue
    prefetch(0, prb);
    prefetch(1, pra);  // (NBLK >= 8)
  }
  // the commit: the path's B rows, gathered before the path is validated
  // (a failed commit applies none of them), held until the C rows are dead
  constexpr int kBPT = CM ? (KT * kChunks + kWsThreads - 1) / kWsThreads : 1;
  u32x4 rbp[kBPT];
  if constexpr (CM) {
    const int len_raw = s_misc[3];
    const int lg = len_raw < 0 ? 0 : (len_raw > T ? T : len_raw);
    {  // the path's dt_raw per block head (lane = path position; an invalid
       // path is discarded with the commit)
      const TIn* dtpg = reinterpret_cast<const TIn*>(a.dt_prev) + unit * T * (int64_t)H;
      const int vp = lane < lg ? s_path[lane] : 0;
      const int vs = (vp >= 0 && vp < T) ? vp : 0;
#pragma unroll
      for (int i = 0; i < kHB; ++i) {
        const int bw = wave + kWsWaves * i;
        const int h = (cw0 + (bw < NBLK ? bw : 0) * kTtRows) / P;
        hdtp[i] = raw_bits<TIn>(dtpg + (int64_t)vs * H + h);
      }
    }
    const unsigned char* Bpg =
        reinterpret_cast<const unsigned char*>(a.B_prev) + ((unit * T) * G + g) * (int64_t)N * E;
#pragma unroll
    for (int it = 0; it < kBPT; ++it) {
      const int ci = tid + it * kWsThreads, q = ci / kChunks, ch = ci % kChunks;
      rbp[it] = u32x4{0u, 0u, 0u, 0u};
      if (q < lg) {
        const int v = s_path[q];
        const int vs = (v >= 0 && v < T) ? v : 0;
        rbp[it] = *reinterpret_cast<const u32x4*>(Bpg + (int64_t)vs * G * N * E + ch * 16);
      }
    }
    if (wave == 1) {
      // the committed tree and the path, by ballot
      bool bad_p = false, bad_path = false;
      if (lane < T) {
        const int p = s_pparent[lane];
        bad_p = lane == 0 ? p != -1 : (p < -1 || p >= lane || p < s_pparent[lane - 1]);
      }
      if (lane < lg) {
        const int v = s_path[lane];
        bad_path = v < 0 || v >= T || s_pparent[v] != (lane == 0 ? -1 : s_path[lane - 1]);
      }
      const bool prev_ok = __ballot(bad_p) == 0;
      const bool path_ok = len_raw >= 0 && len_raw <= T && __ballot(bad_path) == 0;
      const int st = !prev_ok ? SSM_TREE_E_TREE : (!path_ok ? SSM_TREE_E_PATH : SSM_TREE_OK);
      if (lane == 0) {
        s_misc[1] = st == SSM_TREE_OK ? len_raw : 0;  // 0: state and window pass through unchanged
        if (blockIdx.x == 0 && l == 0 && a.commit_status) a.commit_status[b] = st;
      }
    }
  }
  if (wave == 0) {
    // validation by ballot, root-path sets and conv tap rows, as in
    // verify_tt_kernel
    bool bad = false;
    if (lane < T) {
      const int p = s_parent[lane];
      bad = lane == 0 ? p != -1 : (p < -1 || p >= lane || p < s_parent[lane - 1]);
    }
    const bool ok = __ballot(bad) == 0;
    uint64_t m = 0;
    int packed = 0;
    if (lane < T) {
      int u = lane, a1 = -1, a2 = -1, a3 = -1, depth = 0;
      for (int s = 0; s < kTtMaxT && u >= 0; ++s) {
        m |= 1ull << u;
        ++depth;
        const int p = s_parent[u];
        u = (p >= 0 && p < u) ? p : -1;
        a1 = s == 0 ? u : a1;
        a2 = s == 1 ? u : a2;
        a3 = s == 2 ? u : a3;
      }
#pragma unroll
      for (int jj = 1; jj < 4; ++jj) {
        const int an = jj == 1 ? a1 : (jj == 2 ? a2 : a3);
        const int code = an >= 0 ? an + 3 : 2 - (jj - depth);
        if (jj < W) packed |= code << (8 * (jj - 1));
      }
    }
    s_anc[lane] = m;
    s_cidx[lane] = packed;
    if (lane == 0) {
      s_misc[0] = ok ? 1 : 0;
      if (blockIdx.x == 0 && l == 0 && a.verify_status) a.verify_status[b] = ok ? SSM_TREE_OK : SSM_TREE_E_TREE;
    }
  }
  // C_v . B_u over the lower-triangular tile pairs (eight waves)
  for (int pi = wave; pi < TT * (TT + 1) / 2; pi += kWsWaves) {
    const int ti = pair_ti(pi), tj = pair_tj(pi);
    f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
    const TIn* brow = reinterpret_cast<const TIn*>(s_B + (16 * tj + j) * rs) + 4 * k;
    const TIn* crow = reinterpret_cast<const TIn*>(s_C + (16 * ti + j) * rs) + 4 * k;
    if constexpr (E == 2) {
#pragma unroll
      for (int m = 0; m < (NG + 1) / 2; ++m) {
        const u32x2 b0 = *reinterpret_cast<const u32x2*>(brow + 32 * m);
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(crow + 32 * m);
        u32x2 b1 = u32x2{0u, 0u}, c1 = b1;
        if (2 * m + 1 < NG) {
          b1 = *reinterpret_cast<const u32x2*>(brow + 32 * m + 16);
          c1 = *reinterpret_cast<const u32x2*>(crow + 32 * m + 16);
        }
        cb = mfma32(u32x4{b0.x, b0.y, b1.x, b1.y}, u32x4{c0.x, c0.y, c1.x, c1.y}, cb);
      }
    } else {
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) {
        const f32x4 bq = load4<TIn>(brow + 16 * gg);
        const f32x4 cq = load4<TIn>(crow + 16 * gg);
        cb = mfma4(bq.x, cq.x, cb);
        cb = mfma4(bq.y, cq.y, cb);
        cb = mfma4(bq.z, cq.z, cb);
        cb = mfma4(bq.w, cq.w, cb);
      }
    }
    *reinterpret_cast<f32x4*>(s_cbt + (16 * pi + j) * kPairStride + 4 * k) = cb;
  }
  __syncthreads();  // the B rows are dead: their space holds the conv outputs
  const bool tree_ok = s_misc[0] != 0;
  if (CM && s_misc[1] != clen) {  // the commit failed: nothing is applied
    clen = s_misc[1];
    resolve_sources();
    if (producer) {
      prefetch(0, prb);
      prefetch(1, pra);
    }
  }

  // ---- each block's head: dt, S (fp64) and exp(S), wave = block, lane =
  // node, from the registers loaded at entry ----
  auto raw_f32 = [](uint32_t r) { return E == 2 ? __uint_as_float(r << 16) : __uint_as_float(r); };
#pragma unroll
  for (int i = 0; i < kHB; ++i) {
    const int bw = wave + kWsWaves * i;
    if (bw >= NBLK) break;
    const int v = lane;
    float dtv = 0.0f;
    if (v < T) dtv = softplus_hw(raw_f32(hdt[i]) + hbias[i]);
    int up = v < T ? s_parent[v] : -1;
    up = (up >= 0 && up < v) ? up : -1;
    const double s2 = root_path_sum((double)(dtv * hA[i]), up, v) * 1.4426950408889634;
    s_dt[bw * kTtMaxT + v] = dtv;
    s_S2[bw * kTtMaxT + v] = s2;
    s_Ah[bw * kTtMaxT + v] = __builtin_amdgcn_exp2f((float)s2);
    if (v == 0) s_D[bw] = hD[i];
    if constexpr (CM) {
      // the accepted path in closed form (lane = path position q):
      //   h_new = exp(P_last) h + sum_q exp(P_last - P_q) dt_q x~_q B_q,
      // P_q = sum of dt * A over positions 0..q, in fp64 (zero steps past
      // the path's length leave P_last in lane 63)
      const int len = s_misc[1];
      float dtq = 0.0f;
      if (v < len) dtq = softplus_hw(raw_f32(hdtp[i]) + hbias[i]);
      double pq = (double)(dtq * hA[i]);
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(pq, off);
        if (v >= off) pq += o;
      }
      const double plast = __shfl(pq, kWave - 1);
      s_wt[bw * kTtMaxT + v] =
          v < len ? __builtin_amdgcn_exp2f((float)((plast - pq) * 1.4426950408889634)) * dtq : 0.0f;
      if (v == 0) s_at[bw] = __builtin_amdgcn_exp2f((float)(plast * 1.4426950408889634));
    }
  }

  // block 0 delivered (with the commit after the barrier below: its
  // weighted path conv reads the head data of other waves)
  if (!CM && producer) {
    deliver(0, prb);
    prefetch(2, prb);
  }
  // consumers with bf16 inputs and d_state <= 128: the C operands of every
  // node tile and column group pair stay in registers for all the
  // workgroup's blocks (wider states read them from LDS per block)
  constexpr bool kCReg = E == 2 && NG <= 8;
  constexpr int kCM = kCReg ? (NG + 1) / 2 : 1;
  u32x4 creg[kCReg ? TT : 1][kCM];
  if constexpr (kCReg) {
    if (!producer) {
      const int ln = opaque_tid() & (kWave - 1), jj = ln & 15, kk = ln >> 4;
#pragma unroll
      for (int ti = 0; ti < TT; ++ti)
#pragma unroll
        for (int m = 0; m < kCM; ++m) {
          const TIn* crow = reinterpret_cast<const TIn*>(s_C + (16 * ti + jj) * rs) + 32 * m + 4 * kk;
          const u32x2 c0q = *reinterpret_cast<const u32x2*>(crow);
          const u32x2 c1q = 2 * m + 1 < NG ? *reinterpret_cast<const u32x2*>(crow + 16) : u32x2{0u, 0u};
          creg[ti][m] = u32x4{c0q.x, c0q.y, c1q.x, c1q.y};
        }
    }
  }
  f32x4 accp[TT];  // consumers: the previous block's C . h0
#pragma unroll
  for (int ti = 0; ti < TT; ++ti) accp[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  if constexpr (CM) {
    if (producer) {
      deliver(0, prb);
      prefetch(2, prb);
    }
    // the C rows are dead: the path's B rows take their place, as
    // [position q][column j][group gg] (NG bf16 per (q, j)), so that the
    // lane that brings B_q[16 gg + j] for every gg reads them at once
    uint16_t* s_bt = reinterpret_cast<uint16_t*>(s_C);
#pragma unroll
    for (int it = 0; it < kBPT; ++it) {
      const int ci = tid + it * kWsThreads, q = ci / kChunks, ch = ci % kChunks;
      if (q < KT) {  // chunk ch holds columns 8 ch .. 8 ch + 7
        const u32x4 w = rbp[it];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = e < 2 ? w.x : (e < 4 ? w.y : (e < 6 ? w.z : w.w));
          s_bt[(q * 16 + (ch & 1) * 8 + e) * NG + (ch >> 1)] = (uint16_t)(word >> (16 * (e & 1)));
        }
      }
    }
    __syncthreads();
  }

  // whether block ph - 1's conv outputs (set by the producers in phase ph - 1,
  // read by the consumers in phase ph) hold a non-finite value
  bool xt_nonfinite = false;
  // Each role runs its own loop of NBLK + 1 phases, one barrier each (the
  // role is uniform per wave): in one shared loop the registers the
  // consumers load for the next block had to survive the producers' branch
  // as well, the allocator gave the loads other registers, and the copy at
  // the end of every phase waited for them.
  if (producer) {
    // phase ph (< NBLK) delivers block ph + 1 from the set R and refills R
    // with block ph + 3 (the last block again near the end, and a delivery
    // past the last block: every phase issues the same memory operations);
    // the two sets alternate by phase
    auto pphase = [&](int ph, PRegs& R) {
      uint32_t nf_any = 0;  // (as in verify_tt_kernel)
      {
        const int par = ph & 1;
        // ---- conv of block ph (lane = channel, wave = node quads) ----
        {
          const int ptid = opaque_tid();
          const int cl = ptid & (kWave - 1);
          const TIn* xw = s_xw(par);
          const TIn* xr = xw + 3 * kTtRows;
          float wt[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) wt[t] = s_cw(par)[t * kTtRows + cl];
          const float cbv = s_cb(par)[cl];
          u32x4 codes4[TT];
#pragma unroll
          for (int it = 0; it < TT; ++it)
            codes4[it] = *reinterpret_cast<const u32x4*>(s_cidx + 4 * (rw + kTtWaves * it));
          float xs[TT][4][4];
#pragma unroll
          for (int it = 0; it < TT; ++it) {
            const int q = rw + kTtWaves * it;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t codes = __builtin_amdgcn_readfirstlane(codes4[it][r]);
              xs[it][r][0] = load_in(xr, (4 * q + r) * kTtRows + cl);
#pragma unroll
              for (int t = 1; t < 4; ++t)
                xs[it][r][t] = load_in(xw, ((codes >> (8 * (t - 1))) & 255) * kTtRows + cl);
            }
          }
          float* xt = s_xt(par);
#pragma unroll
          for (int it = 0; it < TT; ++it) {
            const int q = rw + kTtWaves * it;
            f32x4 xq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float z = fmaf(wt[0], xs[it][r][0], cbv);
#pragma unroll
              for (int t = 1; t < 4; ++t) z = fmaf(wt[t], xs[it][r][t], z);
              xq[r] = z;
            }
            if (d.silu) {
#pragma unroll
              for (int r = 0; r < 4; ++r) xq[r] = silu_fast(xq[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) xq[r] = 4 * q + r < T ? xq[r] : 0.0f;
            const uint32_t nfb = nonfinite_quad(xq);
            s_nf(par)[cl * (kTtMaxT / 4) + q] = (uint8_t)nfb;
            nf_any |= nfb;
            // (the swizzled [channel][node] layout of verify_tt_kernel's conv outputs)
            *reinterpret_cast<f32x4*>(xt + cl * kTtMaxT + 4 * (q ^ (cl & 15))) = xq;
          }
        }
        // ---- M of block ph ----
        {
          const int ptid = opaque_tid();
          const int r = (ptid >> 2) & 15, cq = ptid & 3;
          const double* S2w = s_S2 + ph * kTtMaxT;
          const float* dtw = s_dt + ph * kTtMaxT;
          const float Dh0 = s_D[ph];
          float* mm = s_m(par);
          switch (rw) {
            case 0: m_form_slot<TT, 0>(mm, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
            case 1: m_form_slot<TT, 1>(mm, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
            case 2: m_form_slot<TT, 2>(mm, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
            default: m_form_slot<TT, 3>(mm, s_cbt, s_anc, S2w, dtw, Dh0, r, cq); break;
          }
        }
      }
      deliver(ph + 1, R);
      prefetch(ph + 3 < NBLK ? ph + 3 : NBLK - 1, R);
      if (nf_any) s_nff[ph] = 1;  // (a plain flag: the reduction of __syncthreads_or
      __syncthreads();             // put its temporaries on registers with loads in flight)
    };
    for (int ph = 0; ph < NBLK; ph += 2) {  // (NBLK even)
      pphase(ph, pra);
      pphase(ph + 1, prb);
    }
    __syncthreads();  // phase NBLK: the consumers' last path terms
  } else {
    // ---- the commit and C . h0 of block ph (its state arrived a phase ago) ----
    auto cstate = [&](int ph, f32x4 (&acc)[TT]) {
#pragma unroll
      for (int ti = 0; ti < TT; ++ti) acc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        const int ln = opaque_tid() & (kWave - 1), jj = ln & 15, kk = ln >> 4;
        const int c0 = cw0 + ph * kTtRows;
        // the next block's state, loaded unconditionally (the last block
        // reloads its own: a conditional load would leave the old value
        // live beside the new one and cost a copy that waits for the load)
        const int nb = ph + 1 < NBLK ? kTtRows : 0;
        const TS* nsin =
            reinterpret_cast<const TS*>(a.state_in) + (unit * DI + c0 + nb + rw * 16 + jj) * (int64_t)N + 4 * kk;
        if constexpr (CM) {
          // ---- the commit of block ph's channels, then the state leaves ----
          // h_new^T = exp(P_last) h^T + Bp^T W on the matrix cores, four path
          // positions per product: lane j + 16 k brings B_q[16 gg + j] and
          // W[q][channel j] for q = s4 + k, and its state quads are the
          // accumulator rows (columns 16 gg + 4 k .. + 3 of channel j)
          const int ch = rw * 16 + jj;
          if (clen > 0) {
            const int par = ph & 1;
            const TIn* pr = s_pr(par);
            const float at = s_at[ph];
            float cwv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) cwv[t] = s_cw(par)[t * kTtRows + ch];
            const float cbv = s_cb(par)[ch];
            f32x4 hc[NG];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) hc[gg] = SQ::to_f32(hq[gg]) * at;
            const unsigned char* bt = s_C + jj * 2 * NG;  // this lane's column of the path's B rows
#pragma unroll 2
            for (int s4 = 0; s4 < clen; s4 += 4) {
              const int q = s4 + kk;  // positions past the path read stale rows, selected away
              uint32_t bw[(NG + 1) / 2];  // B_q[16 gg + j] for every gg (zero past the path)
              const unsigned char* bq = bt + q * 32 * NG;
              if constexpr (NG == 8) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(bq);
                bw[0] = v.x; bw[1] = v.y; bw[2] = v.z; bw[3] = v.w;
              } else if constexpr (NG == 4) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(bq);
                bw[0] = v.x; bw[1] = v.y;
              } else if constexpr (NG == 2) {
                bw[0] = *reinterpret_cast<const uint32_t*>(bq);
              } else {
                bw[0] = *reinterpret_cast<const uint16_t*>(bq);
              }
              float wv;
              if (s4 < kWqPos) {  // formed by the producers
                wv = s_wq(par)[ch * kWqStride + q];
              } else {
                float z = fmaf(cwv[0], load_in(pr, (3 + q) * kTtRows + ch), cbv);
#pragma unroll
                for (int t = 1; t < 4; ++t)
                  if (t < W) z = fmaf(cwv[t], load_in(pr, (3 + q - t) * kTtRows + ch), z);
                const float xt = d.silu ? silu_fast(z) : z;
                wv = q < clen ? s_wt[ph * kTtMaxT + q] * xt : 0.0f;
              }
#pragma unroll
              for (int gg = 0; gg < NG; ++gg) {
                const uint32_t w2 = bw[gg >> 1];
                const float bv = __uint_as_float((gg & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
                hc[gg] = mfma4(bv, wv, hc[gg]);
              }
            }
            // the committed state as stored (a bfloat16 state is rounded):
            // the next tree is verified from exactly what was written
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) hq[gg] = SQ::from_f32(hc[gg]);
          }
          TS* so = reinterpret_cast<TS*>(a.state_out) + (unit * DI + c0 + ch) * (int64_t)N + 4 * kk;
#pragma unroll
          for (int gg = 0; gg < NG; ++gg) SQ::store(so + 16 * gg, hq[gg]);
        }
        if constexpr (E == 2) {
#pragma unroll
          for (int m = 0; m < (NG + 1) / 2; ++m) {
            const bool two = 2 * m + 1 < NG;
            u32x4 h0, h1, h2;
            if constexpr (sizeof(TS) == 2) {
              const u32x2 lo2 = hq[2 * m], hi2 = two ? hq[2 * m + 1] : u32x2{0u, 0u};
              h0 = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
            } else {
              split3(hq[2 * m], two ? hq[2 * m + 1] : f32x4{0.f, 0.f, 0.f, 0.f}, h0, h1, h2);
            }
#pragma unroll
            for (int ti = 0; ti < TT; ++ti) {
              u32x4 ca;
              if constexpr (kCReg) {
                ca = creg[ti][m];
              } else {
                const TIn* crow = reinterpret_cast<const TIn*>(s_C + (16 * ti + jj) * rs) + 32 * m + 4 * kk;
                const u32x2 c0q = *reinterpret_cast<const u32x2*>(crow);
                const u32x2 c1q = two ? *reinterpret_cast<const u32x2*>(crow + 16) : u32x2{0u, 0u};
                ca = u32x4{c0q.x, c0q.y, c1q.x, c1q.y};
              }
              if constexpr (sizeof(TS) != 2) {
                acc[ti] = mfma32(ca, h2, acc[ti]);
                acc[ti] = mfma32(ca, h1, acc[ti]);
              }
              acc[ti] = mfma32(ca, h0, acc[ti]);
            }
            hq[2 * m] = SQ::load(nsin + 32 * m);
            if (two) hq[2 * m + 1] = SQ::load(nsin + 32 * m + 16);
            asm volatile("" ::: "memory");
          }
        } else {
#pragma unroll
          for (int gg = 0; gg < NG; ++gg) {
            const f32x4 h = SQ::to_f32(hq[gg]);
#pragma unroll
            for (int ti = 0; ti < TT; ++ti) {
              const f32x4 cq =
                  load4<TIn>(reinterpret_cast<const TIn*>(s_C + (16 * ti + jj) * rs) + 16 * gg + 4 * kk);
              acc[ti] = mfma4(cq.x, h.x, acc[ti]);
              acc[ti] = mfma4(cq.y, h.y, acc[ti]);
              acc[ti] = mfma4(cq.z, h.z, acc[ti]);
              acc[ti] = mfma4(cq.w, h.w, acc[ti]);
            }
            hq[gg] = SQ::load(nsin + 16 * gg);
            asm volatile("" ::: "memory");
          }
        }
      }
    };
    // ---- path terms and y of block pb ----
    auto cpath = [&](int pb) {
      {
        const int par = pb & 1;
        const int ln = opaque_tid() & (kWave - 1), jj = ln & 15, kk = ln >> 4;
        const int c0 = cw0 + pb * kTtRows;
        const int row = rw * 16 + jj;
        const float* Ahh = s_Ah + pb * kTtMaxT;
        const float* xt = s_xt(par);
        const float* mm = s_m(par);
        float* yrow = a.y + unit * T * (int64_t)DI + c0 + row;
        const uint32_t yoff = (uint32_t)(c0 + row) * 4u;  // bytes into the unit's y rows
        // column tile outermost: one x~ quad per tj serves every node tile
        // ti >= tj, and the TT accumulators are independent product chains
        f32x4 y[TT];
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) y[ti] = *reinterpret_cast<const f32x4*>(Ahh + 16 * ti + 4 * kk) * accp[ti];
#pragma unroll
        for (int tj = 0; tj < TT; ++tj) {
          const f32x4 xq = *reinterpret_cast<const f32x4*>(xt + row * kTtMaxT + 4 * ((4 * tj + kk) ^ (row & 15)));
#pragma unroll
          for (int ti = tj; ti < TT; ++ti) {
            const f32x4 mop = *reinterpret_cast<const f32x4*>(mm + (16 * pair_of(ti, tj) + jj) * kPairStride + 4 * kk);
            y[ti] = mfma4(mop.x, xq.x, y[ti]);
            y[ti] = mfma4(mop.y, xq.y, y[ti]);
            y[ti] = mfma4(mop.z, xq.z, y[ti]);
            y[ti] = mfma4(mop.w, xq.w, y[ti]);
          }
          asm volatile("" ::: "memory");  // one column tile's operands at a time
        }
        // lane (c + 16 k) holds nodes 16 ti + 4 k + r of channel row: a 4 x 4
        // transpose within each lane quad (node r <-> channel c % 4) gives
        // lane (4 m + s + 16 k) channels 4 m .. 4 m + 3 of node 16 ti + 4 k + s,
        // one 16-byte store per node tile instead of four 4-byte ones
        const int s = jj & 3;
        const uint32_t yoff4 = (uint32_t)(c0 + rw * 16 + (jj & ~3)) * 4u;
#pragma unroll
        for (int ti = 0; ti < TT; ++ti) {
          const f32x4 tq = quad_transpose(y[ti], jj);
          const int v = 16 * ti + 4 * kk + s;
          const u32x4 bits = tree_ok ? __builtin_bit_cast(u32x4, tq) : u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u,
                                                                               0x7FC00000u};
          __builtin_amdgcn_raw_buffer_store_b128(bits, y_rsrc, v < T ? (int)((uint32_t)v * DI * 4u + yoff4) : kOutOfRange,
                                                 0, 0);
        }
        if (xt_nonfinite) {  // (rare) y_v not finite where v's root path holds a non-finite x~_u
          const uint64_t nfm = nonfinite_nodes(s_nf(par), row);
          for (int v = 4 * kk; v < T; v = (v & 3) == 3 ? v + 13 : v + 1)  // this lane's nodes 16 ti + 4 k + r
            if (s_anc[v] & nfm) yrow[(int64_t)v * DI] = __builtin_nanf("");
          // (these stores stay out of the count the next phase's waits assume)
          __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
      }
    };
    // phase 0: block 0's state part; phases 1 .. NBLK - 1: block ph's state
    // part and block ph - 1's path terms; phase NBLK: the last path terms
    // (every loop phase issues the same memory operations)
    f32x4 acc[TT];
    cstate(0, acc);
    // as many (dropped) stores as a phase's path terms issue: the loop's
    // waits for the state count them
#pragma unroll
    for (int i = 0; i < TT; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, y_rsrc, kOutOfRange - 64 * i, 0, 0);
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) accp[ti] = acc[ti];
    __syncthreads();
    xt_nonfinite = s_nff[0] != 0;  // block ph's conv outputs, whose path terms come next
    for (int ph = 1; ph < NBLK; ++ph) {
      cstate(ph, acc);
      cpath(ph - 1);
#pragma unroll
      for (int ti = 0; ti < TT; ++ti) accp[ti] = acc[ti];
      __syncthreads();
      xt_nonfinite = s_nff[ph] != 0;
    }
    cpath(NBLK - 1);
    __syncthreads();
  }
}

namespace {

template <typename TIn, typename TS, int NG, int TT, bool CM = false>
int launch_ws_t(const CommitVerifyArgs& a, int nblk, hipStream_t s) {
  const size_t lds = (size_t)TtWsLds(16 * NG, (int)sizeof(TIn), TT, CM, nblk).total;
  if (lds > 160 * 1024) return SSM_TREE_E_DIMS;
  if (allow_lds(verify_tt_ws_kernel<TIn, TS, NG, TT, CM>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  dim3 grid(a.d.d_in / (nblk * kTtRows), a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((verify_tt_ws_kernel<TIn, TS, NG, TT, CM>), grid, dim3(kWsThreads), lds, s, a, nblk);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

// a verify's arguments in the round's argument block (nothing committed)
CommitVerifyArgs ws_args(const VerifyArgs& v) {
  CommitVerifyArgs a{};
  a.d = v.d;
  a.prm = v.prm;
  a.parent = v.parent;
  a.x = v.x;
  a.B = v.B;
  a.C = v.C;
  a.dt_raw = v.dt_raw;
  a.z = v.z;
  a.window_in = v.window;
  a.state_in = v.state;
  a.y = v.y;
  a.verify_status = v.seq_status;
  return a;
}

template <typename TIn, typename TS, int NG, int TT, bool OPT = false>
int launch_tt_t(const VerifyArgs& a, hipStream_t s) {
  const size_t lds = (size_t)TtLds(16 * NG, (int)sizeof(TIn), TT, OPT).total;
  if (lds > 160 * 1024) return SSM_TREE_E_DIMS;  // (fp32 inputs with d_state 256) the caller falls back
  if (allow_lds(verify_tt_kernel<TIn, TS, NG, TT, OPT>, lds) != hipSuccess) return SSM_TREE_E_HIP;
  const int blocks = a.d.d_in / a.d.G / kTtRows;  // 64-channel blocks per B/C group
  const int nblk = blocks % 4 == 0 ? 4 : (blocks % 2 == 0 ? 2 : 1);
  dim3 grid(a.d.d_in / (nblk * kTtRows), a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((verify_tt_kernel<TIn, TS, NG, TT, OPT>), grid, dim3(kTtThreads), lds, s, a, nblk);
  return hipGetLastError() == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

// the role-split kernel where each block lies in one head and a workgroup
// can take 8 or 16 blocks (else the per-block kernel)
template <typename TIn, typename TS, int NG, int TT>
int launch_tt_pick(const VerifyArgs& a, hipStream_t s) {
  if constexpr (sizeof(TS) == 4)  // the options: the per-block kernel's instantiation of their own
    if (a.d.xbc || a.z) return launch_tt_t<TIn, TS, NG, TT, true>(a, s);
  const int blocks = a.d.d_in / a.d.G / kTtRows;
  if (a.d.P % kTtRows == 0 && blocks % 8 == 0) {
    // the most blocks per workgroup (the prologue's share of its time
    // shrinks) that divide the group and whose tables fit the LDS
    int nblk = 8;
    for (int c = kWsMaxBlkV; c > 8; c -= 8)
      if (blocks % c == 0 && TtWsLds(16 * NG, (int)sizeof(TIn), TT, false, c).total <= 160 * 1024) {
        nblk = c;
        break;
      }
    const int st = launch_ws_t<TIn, TS, NG, TT>(ws_args(a), nblk, s);
    if (st != SSM_TREE_E_DIMS) return st;  // E_DIMS: its LDS does not fit, nothing launched
  }
  return launch_tt_t<TIn, TS, NG, TT>(a, s);
}

template <typename TIn, typename TS, int NG>
int launch_tt_g(const VerifyArgs& a, hipStream_t s) {
  const int T = a.d.T;
  if (T <= 32) return launch_tt_pick<TIn, TS, NG, 2>(a, s);
  if (T <= 48) return launch_tt_pick<TIn, TS, NG, 3>(a, s);
  return launch_tt_pick<TIn, TS, NG, 4>(a, s);
}

template <typename TIn, typename TS>
int launch_tt_in(const VerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_tt_g<TIn, TS, 1>(a, s);
    case 32: return launch_tt_g<TIn, TS, 2>(a, s);
    case 64: return launch_tt_g<TIn, TS, 4>(a, s);
    case 128: return launch_tt_g<TIn, TS, 8>(a, s);
    case 256: return launch_tt_g<TIn, TS, 16>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

// the round (commit of the accepted path, then verify of the next tree) in
// the role-split kernel
template <typename TS, int NG>
int launch_tt_round_g(const CommitVerifyArgs& a, hipStream_t s) {
  const int blocks = a.d.d_in / a.d.G / kTtRows;
  // the most blocks per workgroup (an even count dividing the group) whose
  // tables fit the LDS next to the commit's buffers
  const int TTs = a.d.T <= 32 ? 2 : (a.d.T <= 48 ? 3 : 4);
  int nblk = 8;
  for (int c = kWsMaxBlk; c > 8; c -= 2)
    if (blocks % c == 0 && TtWsLds(16 * NG, 2, TTs, true, c).total <= 160 * 1024) {
      nblk = c;
      break;
    }
  const int T = a.d.T;
  if (T <= 32) return launch_ws_t<bf16_t, TS, NG, 2, true>(a, nblk, s);
  if (T <= 48) return launch_ws_t<bf16_t, TS, NG, 3, true>(a, nblk, s);
  return launch_ws_t<bf16_t, TS, NG, 4, true>(a, nblk, s);
}

template <typename TS>
int launch_tt_round_in(const CommitVerifyArgs& a, hipStream_t s) {
  switch (a.d.N) {
    case 16: return launch_tt_round_g<TS, 1>(a, s);
    case 32: return launch_tt_round_g<TS, 2>(a, s);
    case 64: return launch_tt_round_g<TS, 4>(a, s);
    case 128: return launch_tt_round_g<TS, 8>(a, s);
    default: return SSM_TREE_E_DIMS;
  }
}

}  // namespace

// whether the round of trees of 17..64 nodes runs as one launch: bf16
// inputs, d_state <= 128, every 64-channel block inside one head, B/C
// groups of a multiple of 8 blocks, none of the options (their rounds run
// as commit then verify)
bool tt_round_applies(const Dims& d, bool bf16, bool gate) {
  return bf16 && d.T > 16 && d.T <= kTtMaxT && !d.fifo && !d.xbc && !gate && d.N <= 128 && d.P % kTtRows == 0 &&
         (d.d_in / d.G) % (8 * kTtRows) == 0;
}

int launch_tt_round(const CommitVerifyArgs& a, hipStream_t s) {
  return a.d.sbf16 ? launch_tt_round_in<bf16_t>(a, s) : launch_tt_round_in<float>(a, s);
}

// trees of 17..64 nodes, heads a multiple of 16 channels, 64-channel blocks
bool tt_verify_applies(const Dims& d) {
  return d.T > 16 && d.T <= kTtMaxT && d.P % 16 == 0 && (d.d_in / d.G) % kTtRows == 0;
}

// whether the kernel's LDS fits the shape (it does except for fp32 inputs
// with d_state 256); opt: the options' instantiation
bool tt_verify_fits(const Dims& d, bool bf16, bool opt) {
  const int TT = (d.T + 15) / 16;
  return TtLds(d.N, bf16 ? 2 : 4, TT < 2 ? 2 : TT, opt).total <= 160 * 1024;
}

int launch_verify_tt(const VerifyArgs& a, bool bf16, hipStream_t s) {
  if (a.d.sbf16) return bf16 ? launch_tt_in<bf16_t, bf16_t>(a, s) : launch_tt_in<float, bf16_t>(a, s);
  return bf16 ? launch_tt_in<bf16_t, float>(a, s) : launch_tt_in<float, float>(a, s);
}

}  // namespace ssmt
