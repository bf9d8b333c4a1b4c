// commit.hip - ssm_tree_commit kernel for gfx950.
//
// SpecMamba page sec. 3.1: after verification the root state is advanced
// along the accepted path by recomputing the recurrence from the stored
// per-token dt, B and x (no per-node state is kept between verify and
// commit).  For path nodes u_0 .. u_{m-1}:
//   h <- dA_{u_k} h + (dt_{u_k} x~_{u_k}) B_{u_k}^T     k = 0 .. m-1
// and the conv window becomes the last W-1 rows of (old window, x_{u_0..}),
// copied bit for bit.
//
// The state update is elementwise, so the kernel is a coalesced HBM stream:
// a workgroup owns 64 channels (rows) of one (layer, sequence); its threads
// issue all their 16-byte state loads first, prepare the per-path scalars,
// the conv outputs and the fp32 B rows in LDS, then update and store.
// Each state load or store instruction of a wave covers 1 KiB of whole
// 128-byte lines, and the state is touched once, so both go non-temporal
// (streamed past the caches): 1.08 -> 1.00 ms on the 2.7B batch-16
// workload.  (The MFMA-layout kernels touch half a line per instruction;
// there the non-temporal hint measured slower.)
#include <type_traits>

#include "common.h"

namespace ssmt {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCommitRows = 64;
constexpr int kCommitThreads = 256;
constexpr int kCommitChunk = 16;  // path nodes staged in LDS at a time
static_assert(kCommitChunk * kCommitRows % kCommitThreads == 0, "x staging trip count");

// d_state up to 128 fits 5 waves per SIMD (<= 96 VGPRs) without spills;
// the 256 form holds twice the state and keeps the compiler's choice
template <typename TIn, typename TS, int QPT>
__global__ void __launch_bounds__(kCommitThreads) __attribute__((amdgpu_waves_per_eu(QPT <= 8 ? 5 : 1)))
commit_kernel(CommitArgs a, int HWMAX) {
  typedef StateQuad<TS> SQ;
  const Dims d = a.d;
  // d_state is N = 16 QPT (64 rows of N, 4 per quad, over 256 threads)
  constexpr int N = 16 * QPT, qpr = N / 4;  // qpr: float4 quads per row
  const int T = d.T, P = d.P, H = d.H, W = d.W, DI = d.d_in;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  const int c0 = blockIdx.x * kCommitRows;
  const int g = c0 / (DI / d.G);
  const int h_lo = c0 / P;

  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* s_parent = reinterpret_cast<int32_t*>(smem);
  int32_t* s_path = s_parent + kMaxNodes;
  int32_t* s_misc = s_path + kMaxNodes;
  float* s_dA = reinterpret_cast<float*>(s_misc + 4);      // [T][HWMAX]
  float* s_dtv = s_dA + kMaxNodes * HWMAX;                 // [T][HWMAX] dt
  float* s_dtx = s_dtv + kMaxNodes * HWMAX;                // [chunk][64] raw x of the path nodes
  float2* s_ax = reinterpret_cast<float2*>(s_dtx + kCommitChunk * kCommitRows);  // [chunk][64] (dA, dt x~) per row
  float* s_B = reinterpret_cast<float*>(s_ax + kCommitChunk * kCommitRows);     // [chunk][N]

  // ---- issue the state loads first (QPT quads per thread) ----
  // A bf16 state moves in 16-byte accesses: access it2 of a thread is the 8
  // consecutive elements 8 (tid + 256 it2) .., i.e. quads 2 it2 and 2 it2 + 1;
  // otherwise quad it is the 4 elements 4 (tid + 256 it) ..
  constexpr bool kWide = sizeof(TS) == 2 && QPT % 2 == 0;
  typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
  const TS* sin = reinterpret_cast<const TS*>(a.state_in) + (unit * DI + c0) * (int64_t)N;
  typename SQ::Raw hq[QPT];
  if constexpr (kWide) {
#pragma unroll
    for (int it2 = 0; it2 < QPT / 2; ++it2) {
      const int qo = threadIdx.x + it2 * kCommitThreads;
      const u32x4c w = __builtin_nontemporal_load(reinterpret_cast<const u32x4c*>(sin + 8 * qo));
      hq[2 * it2] = typename SQ::Raw{w.x, w.y};
      hq[2 * it2 + 1] = typename SQ::Raw{w.z, w.w};
    }
  } else {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      const int qi = threadIdx.x + it * kCommitThreads;
      hq[it] = SQ::load_nt(sin + 4 * qi);
    }
  }

  // ---- validate tree and path ----
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    s_parent[i] = a.parent[(int64_t)b * T + i];
    s_path[i] = a.path[(int64_t)b * T + i];
  }
  __syncthreads();
  const bool tree_ok = tree_is_valid(s_parent, T);
  // the path, one link per thread: path[0] is a root-level node and each
  // later entry a child of the one before
  const int plen = a.path_len[b];
  int bad = 0;
  if (tree_ok && plen >= 0 && plen <= T) {
    for (int k = threadIdx.x; k < plen; k += blockDim.x) {
      const int v = s_path[k];
      bad |= (v < 0 || v >= T || s_parent[v] != (k == 0 ? -1 : s_path[k - 1]));
    }
  }
  const bool path_bad = __syncthreads_or(bad) != 0 || plen < 0 || plen > T;
  const int st = !tree_ok ? SSM_TREE_E_TREE : (path_bad ? SSM_TREE_E_PATH : SSM_TREE_OK);
  if (threadIdx.x == 0 && blockIdx.x == 0 && l == 0 && a.seq_status) a.seq_status[b] = st;
  if (st != SSM_TREE_OK) return;  // outputs of a failed sequence stay unwritten
  const int len = plen;

  // ---- per-path scalars, conv outputs, B rows ----
  const int HW = (c0 + kCommitRows - 1) / P - h_lo + 1;
  const TIn* dtr = reinterpret_cast<const TIn*>(a.dt_raw) + unit * T * H;
  for (int i = threadIdx.x; i < len * HW; i += blockDim.x) {
    const int k = i / HW, hh = i % HW, h = h_lo + hh;
    const float z = load_in(dtr, (int64_t)s_path[k] * H + h) + a.prm.dt_bias[(int64_t)l * H + h];
    const float dt = softplus_f32(z);
    s_dA[k * HWMAX + hh] = expf(dt * a.prm.A[(int64_t)l * H + h]);
    s_dtv[k * HWMAX + hh] = dt;
  }
  const int CH = d.CH;  // conv channels = window row length
  const TIn* xin = reinterpret_cast<const TIn*>(a.x) + unit * T * DI;
  const TIn* Bg = reinterpret_cast<const TIn*>(a.B) + (unit * T * d.G + g) * (int64_t)N;
  const TIn* win_in = reinterpret_cast<const TIn*>(a.window_in) + unit * (W - 1) * (int64_t)CH;

  // the conv threads (one per channel) carry their weights, the sliding
  // window of raw inputs and the new window rows across the path's chunks
  const bool conv_thr = threadIdx.x < kCommitRows;
  const int cc = c0 + (conv_thr ? threadIdx.x : 0), hhc = cc / P - h_lo;
  // wj[jj] weighs conv input jj (0 = the token itself, jj = the jj-th previous token)
  float wj[4] = {0.f, 0.f, 0.f, 0.f}, cbc = 0.f, hist[3] = {0.f, 0.f, 0.f};  // hist[0] = newest
  TIn nw[3];
  if (conv_thr) {
    const float* cw = a.prm.conv_w + ((int64_t)l * CH + cc) * W;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wj[jj] = (jj < W) ? cw[W - 1 - jj] : 0.0f;
    cbc = a.prm.conv_b ? a.prm.conv_b[(int64_t)l * CH + cc] : 0.0f;
#pragma unroll
    for (int r = 0; r < 3; ++r) hist[r] = (r < W - 1) ? load_in(win_in, (int64_t)(W - 2 - r) * CH + cc) : 0.0f;
    // new window row r (oldest first) is element len + r of the sequence
    // (old window rows, x of the path nodes); every source is read before
    // any write, so that an in-place window is safe
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      if (r < W - 1) {
        const int e = len + r;
        nw[r] = (e < W - 1) ? win_in[(int64_t)e * CH + cc] : xin[(int64_t)s_path[e - (W - 1)] * DI + cc];
      }
    }
  }

  // the state in fp32 registers for the whole path
  f32x4 h[QPT];
#pragma unroll
  for (int it = 0; it < QPT; ++it) h[it] = SQ::to_f32(hq[it]);

  // ---- the path in chunks of kCommitChunk nodes (LDS holds one chunk) ----
  for (int k0 = 0; k0 < len; k0 += kCommitChunk) {
    const int kn = len - k0 < kCommitChunk ? len - k0 : kCommitChunk;
    if (k0 > 0) __syncthreads();  // the previous chunk's rows are consumed
    // the chunk's raw x of the workgroup's channels and (no xBC conv) its
    // B rows, in quads of 4 inputs: fixed trip counts and clamped
    // addresses, so that every load of a thread is in flight before the
    // first LDS write.  x: 16 nodes x 16 quads = one quad per thread.
    {
      typedef StateQuad<TIn> IQ;
      constexpr int kQx = kCommitRows / 4, kQb = N / 4;  // quads per x row, per B row
      constexpr int kBr = (kCommitChunk * kQb + kCommitThreads - 1) / kCommitThreads;
      static_assert(kCommitChunk * kQx == kCommitThreads, "one x quad per thread");
      const int kx = min((int)threadIdx.x / kQx, kn - 1);
      const typename IQ::Raw xr = IQ::load(xin + (int64_t)s_path[k0 + kx] * DI + c0 + (threadIdx.x % kQx) * 4);
      typename IQ::Raw br[kBr];
      if (!d.xbc) {
#pragma unroll
        for (int r = 0; r < kBr; ++r) {
          const int q = min((int)threadIdx.x + r * kCommitThreads, kCommitChunk * kQb - 1);
          const int kk = min(q / kQb, kn - 1);
          br[r] = IQ::load(Bg + (int64_t)s_path[k0 + kk] * d.G * N + (q % kQb) * 4);
        }
      }
      if ((int)threadIdx.x < kn * kQx)
        *reinterpret_cast<f32x4*>(s_dtx + threadIdx.x * 4) = IQ::to_f32(xr);
      if (!d.xbc) {
#pragma unroll
        for (int r = 0; r < kBr; ++r) {
          const int q = threadIdx.x + r * kCommitThreads;
          if (q < kn * kQb) *reinterpret_cast<f32x4*>(s_B + q * 4) = IQ::to_f32(br[r]);
        }
      }
    }
    if (d.xbc) {
      for (int i = threadIdx.x; i < kn * N; i += blockDim.x) {
        // the xBC conv of B channel (g, n) at path node k: its taps read the
        // sequence (old window rows, then the path nodes) backwards from k
        const int kk = i / N, k = k0 + kk, n = i % N;
        const int ch = DI + g * N + n;
        const float* cw = a.prm.conv_w + ((int64_t)l * CH + ch) * W;
        float acc = a.prm.conv_b ? a.prm.conv_b[(int64_t)l * CH + ch] : 0.0f;
        for (int j = 0; j < W; ++j) {
          const int e = k + W - 1 - j;
          const float in = e < W - 1 ? load_in(win_in, (int64_t)e * CH + ch)
                                     : load_in(Bg + (int64_t)s_path[e - (W - 1)] * d.G * N, n);
          acc = fmaf(cw[W - 1 - j], in, acc);
        }
        s_B[kk * N + n] = d.silu ? silu_fast(acc) : acc;
      }
    }
    __syncthreads();  // the chunk's x rows and B rows are in LDS
    if (conv_thr) {
#pragma unroll 1
      for (int kk = 0; kk < kn; ++kk) {
        const float xv = s_dtx[kk * kCommitRows + threadIdx.x];
        float z = fmaf(wj[0], xv, cbc);
#pragma unroll
        for (int jj = 1; jj < 4; ++jj)
          if (jj < W) z = fmaf(wj[jj], hist[jj - 1], z);
        const float xt = d.silu ? silu_fast(z) : z;
        s_ax[kk * kCommitRows + threadIdx.x] =
            make_float2(s_dA[(k0 + kk) * HWMAX + hhc], s_dtv[(k0 + kk) * HWMAX + hhc] * xt);
        hist[2] = hist[1];
        hist[1] = hist[0];
        hist[0] = xv;
      }
    }
    __syncthreads();  // (dA, dt x~) of the chunk
    // ---- state update along the chunk ----
    // every access of a thread shares its B columns (N / 4 and N / 8 divide
    // 256), so one B read per node serves all of them
    if constexpr (kWide) {
      constexpr int opr = N / 8;  // 8-element accesses per row
#pragma unroll 1
      for (int kk = 0; kk < kn; ++kk) {
        const f32x4 bq0 = *reinterpret_cast<const f32x4*>(s_B + kk * N + (threadIdx.x % opr) * 8);
        const f32x4 bq1 = *reinterpret_cast<const f32x4*>(s_B + kk * N + (threadIdx.x % opr) * 8 + 4);
#pragma unroll
        for (int it2 = 0; it2 < QPT / 2; ++it2) {
          const int row = (threadIdx.x + it2 * kCommitThreads) / opr;
          const float2 ax = s_ax[kk * kCommitRows + row];
          f32x4& h0 = h[2 * it2];
          f32x4& h1 = h[2 * it2 + 1];
          h0 *= ax.x;
          h1 *= ax.x;
          h0.x = fmaf(ax.y, bq0.x, h0.x);
          h0.y = fmaf(ax.y, bq0.y, h0.y);
          h0.z = fmaf(ax.y, bq0.z, h0.z);
          h0.w = fmaf(ax.y, bq0.w, h0.w);
          h1.x = fmaf(ax.y, bq1.x, h1.x);
          h1.y = fmaf(ax.y, bq1.y, h1.y);
          h1.z = fmaf(ax.y, bq1.z, h1.z);
          h1.w = fmaf(ax.y, bq1.w, h1.w);
        }
      }
    } else {
      // quad it of a thread is row tid / qpr + it * (256 / qpr), columns
      // 4 (tid % qpr) .. +3: qpr = N / 4 divides 256, so every quad of a
      // thread shares its B columns and one B read per node serves them all
#pragma unroll 1
      for (int kk = 0; kk < kn; ++kk) {
        const f32x4 bq = *reinterpret_cast<const f32x4*>(s_B + kk * N + (threadIdx.x % qpr) * 4);
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
          const int row = (threadIdx.x + it * kCommitThreads) / qpr;
          const float2 ax = s_ax[kk * kCommitRows + row];
          // scale in place, then one fused multiply-add: both steps write
          // the state's own registers (no copy of the state per node)
          h[it] *= ax.x;
          h[it].x = fmaf(ax.y, bq.x, h[it].x);
          h[it].y = fmaf(ax.y, bq.y, h[it].y);
          h[it].z = fmaf(ax.y, bq.z, h[it].z);
          h[it].w = fmaf(ax.y, bq.w, h[it].w);
        }
      }
    }
  }
  if (conv_thr && W > 1) {
    TIn* win_out = reinterpret_cast<TIn*>(a.window_out) + unit * (W - 1) * (int64_t)CH;
#pragma unroll
    for (int r = 0; r < 3; ++r)
      if (r < W - 1) win_out[(int64_t)r * CH + cc] = nw[r];
  }
  TS* sout = reinterpret_cast<TS*>(a.state_out) + (unit * DI + c0) * (int64_t)N;
  if constexpr (kWide) {
#pragma unroll
    for (int it2 = 0; it2 < QPT / 2; ++it2) {
      const int qo = threadIdx.x + it2 * kCommitThreads;
      const typename SQ::Raw r0 = SQ::from_f32(h[2 * it2]), r1 = SQ::from_f32(h[2 * it2 + 1]);
      __builtin_nontemporal_store(u32x4c{r0.x, r0.y, r1.x, r1.y}, reinterpret_cast<u32x4c*>(sout + 8 * qo));
    }
  } else {
#pragma unroll
    for (int it = 0; it < QPT; ++it) {
      const int qi = threadIdx.x + it * kCommitThreads;
      SQ::store_nt(sout + 4 * qi, SQ::from_f32(h[it]));
    }
  }
}

// The B and C rows of the conv window after a commit with the xBC conv:
// row r = element len + r of (old window rows, raw B and C of each path
// node), copied bit for bit.  Every workgroup of a (layer, sequence) reads
// the old B and C rows, so they are rewritten only here, in a launch of
// its own after those readers.  A thread owns one channel and reads all of
// its old rows before writing any, so the update is safe in place.  A
// sequence whose commit fails keeps its rows (pass_through: they are
// copied to the output, as the fused round requires).
template <typename TIn>
__global__ void __launch_bounds__(kCommitThreads) commit_window_bc_kernel(WindowBcArgs a) {
  const Dims d = a.d;
  const int T = d.T, W = d.W, DI = d.d_in, CH = d.CH, GN = d.G * d.N;
  const int b = blockIdx.y, l = blockIdx.z;
  const int64_t unit = (int64_t)l * d.Bsz + b;
  __shared__ int32_t s_parent[kMaxNodes], s_path[kMaxNodes], s_len;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    s_parent[i] = a.parent[(int64_t)b * T + i];
    s_path[i] = a.path[(int64_t)b * T + i];
  }
  __syncthreads();
  const bool tree_ok = tree_is_valid(s_parent, T);
  if (threadIdx.x == 0) {
    int len = a.path_len[b];
    bool ok = tree_ok && len >= 0 && len <= T;
    for (int k = 0; ok && k < len; ++k) {
      const int v = s_path[k];
      ok = v >= 0 && v < T && s_parent[v] == (k == 0 ? -1 : s_path[k - 1]);
    }
    s_len = ok ? len : -1;
  }
  __syncthreads();
  int len = s_len;
  if (len < 0) {
    if (!a.pass_through) return;
    len = 0;
  }
  const int ch = blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. 2 G N: B channels, then C channels
  if (ch >= 2 * GN) return;
  // raw bits of the input type: the rows are copied, never converted
  typedef typename std::conditional<sizeof(TIn) == 2, uint16_t, uint32_t>::type R;
  const R* win_in = reinterpret_cast<const R*>(a.window_in) + unit * (W - 1) * (int64_t)CH + DI + ch;
  R* win_out = reinterpret_cast<R*>(a.window_out) + unit * (W - 1) * (int64_t)CH + DI + ch;
  const R* src = reinterpret_cast<const R*>(ch < GN ? a.B : a.C) + unit * T * (int64_t)GN + (ch < GN ? ch : ch - GN);
  R o0 = 0, o1 = 0, o2 = 0;  // old rows 0..W-2 (no dynamic indexing: that would go to scratch memory)
  if (W > 1) o0 = win_in[0];
  if (W > 2) o1 = win_in[(int64_t)CH];
  if (W > 3) o2 = win_in[(int64_t)2 * CH];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    if (r < W - 1) {
      const int e = len + r;
      win_out[(int64_t)r * CH] =
          e < W - 1 ? (e == 0 ? o0 : (e == 1 ? o1 : o2)) : src[(int64_t)s_path[e - (W - 1)] * GN];
    }
  }
}

template <typename TIn>
static hipError_t launch_wbc(const WindowBcArgs& a, hipStream_t s) {
  dim3 grid((2 * a.d.G * a.d.N + kCommitThreads - 1) / kCommitThreads, a.d.Bsz, a.d.L);
  hipLaunchKernelGGL((commit_window_bc_kernel<TIn>), grid, dim3(kCommitThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_window_bc(const WindowBcArgs& a, bool bf16, hipStream_t s) {
  if (a.d.W < 2 || !a.d.xbc) return hipSuccess;
  return bf16 ? launch_wbc<bf16_t>(a, s) : launch_wbc<float>(a, s);
}

// SSM_TREE_CONV_XBC: the commit kernel convolves the path's B rows; the
// window's B and C rows follow in commit_window_bc_kernel.
bool commit_options_supported(const Dims&) { return true; }

template <typename TIn, typename TS, int QPT>
static hipError_t launch_c(const CommitArgs& a, hipStream_t s) {
  const int HWMAX = ((kCommitRows + a.d.P - 1) / a.d.P + 1 + 3) & ~3;
  const size_t lds = sizeof(int32_t) * (2 * kMaxNodes + 4) +
                     sizeof(float) * ((size_t)2 * kMaxNodes * HWMAX + 3 * kCommitChunk * kCommitRows +
                                      (size_t)(a.d.T < kCommitChunk ? a.d.T : kCommitChunk) * a.d.N);
  dim3 grid(a.d.d_in / kCommitRows, a.d.Bsz, a.d.L);
  hipError_t e = allow_lds(commit_kernel<TIn, TS, QPT>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((commit_kernel<TIn, TS, QPT>), grid, dim3(kCommitThreads), lds, s, a, HWMAX);
  return hipGetLastError();
}

template <typename TIn, typename TS>
static hipError_t launch_cin(const CommitArgs& a, hipStream_t s) {
  // quads per thread = 64 rows * N / 4 / 256 threads = N / 16
  switch (a.d.N) {
    case 16: return launch_c<TIn, TS, 1>(a, s);
    case 32: return launch_c<TIn, TS, 2>(a, s);
    case 64: return launch_c<TIn, TS, 4>(a, s);
    case 128: return launch_c<TIn, TS, 8>(a, s);
    case 256: return launch_c<TIn, TS, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t s) {
  hipError_t e = bf16 ? (a.d.sbf16 ? launch_cin<bf16_t, bf16_t>(a, s) : launch_cin<bf16_t, float>(a, s))
                      : (a.d.sbf16 ? launch_cin<float, bf16_t>(a, s) : launch_cin<float, float>(a, s));
  if (e != hipSuccess || !a.d.xbc) return e;
  WindowBcArgs w{a.d, a.parent, a.path, a.path_len, a.B, a.C, a.window_in, a.window_out, 0};
  return launch_window_bc(w, bf16, s);
}

}  // namespace ssmt
