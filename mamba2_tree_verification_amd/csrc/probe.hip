// probe.hip - HBM ceiling probes for the measurement harness.
//
// Built into libssm_tree_probe.so, apart from libssm_tree.so: it is not
// part of the verification ABI.  Each probe streams a buffer laid out like
// the root SSM state (rows of 128 float32 = 512 bytes, one row per channel)
// in the tiles and access patterns the state kernels use, so that its
// achieved bandwidth is the practical ceiling those kernels are measured
// against:
//
//   kind   0 read only            (a verify's state stream)
//          1 copy, src -> dst     (a commit or fused round: state read and
//                                  written once)
//          2 read, plus one 512-byte row written per 8 rows read (the
//                                  ratio of y to state bytes in a 16-node
//                                  verify)
//   layout 0 coalesced: in each 16-byte access instruction a wave covers
//            two whole rows (1 KiB of whole 128-byte lines)
//          1 matrix-core operand layout: wave w of a tile owns rows
//            16 w .. 16 w + 15, lane j + 16 k reads columns 16 gg + 4 k ..
//            + 3 of row j for gg = 0 .. 7 (half a line per row per
//            instruction; two consecutive instructions complete the lines)
//   nt     bit 0: non-temporal loads; bit 1: non-temporal stores
//   grid   0: one workgroup of 256 threads per 64-row tile; otherwise that
//          many workgroups, each walking tiles blockIdx.x, + grid, ... with
//          the next tile's loads issued before the current one is used.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;                 // rows per tile
constexpr int kCols = 128;                // floats per row
constexpr int kThreads = 256;
constexpr int kQ = kRows * kCols / 4 / kThreads;  // 16-byte quads per thread per tile (8)

template <int LAYOUT>
__device__ __forceinline__ int64_t quad_offset(int tid, int it) {
  if constexpr (LAYOUT == 0) {
    return (int64_t)(tid + it * kThreads) * 4;  // float offset inside the tile
  } else {
    const int lane = tid & 63, w = tid >> 6, j = lane & 15, k = lane >> 4;
    return (int64_t)(16 * w + j) * kCols + 16 * it + 4 * k;
  }
}

template <bool NT>
__device__ __forceinline__ u32x4 ld(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st(float* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}

template <int KIND, int LAYOUT, int NT>
__device__ __forceinline__ void consume(const u32x4 (&r)[kQ], float* dst_tile, int tid, uint32_t& acc) {
  constexpr bool kNtSt = (NT & 2) != 0;
  if constexpr (KIND == 1) {
#pragma unroll
    for (int it = 0; it < kQ; ++it) st<kNtSt>(dst_tile + quad_offset<LAYOUT>(tid, it), r[it]);
  } else {
#pragma unroll
    for (int it = 0; it < kQ; ++it) acc ^= r[it].x ^ r[it].y ^ r[it].z ^ r[it].w;
    if constexpr (KIND == 2) {
      // one row in eight: 8 rows of a 64-row tile, one quad per thread
      const u32x4 v = u32x4{acc, acc + 1u, acc + 2u, acc + 3u};
      st<kNtSt>(dst_tile + (int64_t)tid * 4, v);
    }
  }
}

template <int KIND, int LAYOUT, int NT>
__global__ void __launch_bounds__(kThreads) probe_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         int64_t tiles, int persistent, uint32_t* sink) {
  constexpr bool kNtLd = (NT & 1) != 0;
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  // kind 2 writes 8 rows per tile: tile t lands at dst + t * 8 rows
  const int64_t dst_tile_floats = KIND == 1 ? (int64_t)kRows * kCols : (int64_t)8 * kCols;
  if (!persistent) {
    const int64_t t = blockIdx.x;
    if (t >= tiles) return;
    u32x4 r[kQ];
    const float* s = src + t * kRows * kCols;
#pragma unroll
    for (int it = 0; it < kQ; ++it) r[it] = ld<kNtLd>(s + quad_offset<LAYOUT>(tid, it));
    consume<KIND, LAYOUT, NT>(r, dst + t * dst_tile_floats, tid, acc);
  } else {
    int64_t t = blockIdx.x;
    const int64_t stride = gridDim.x;
    if (t >= tiles) return;
    u32x4 cur[kQ], nxt[kQ];
    const float* s = src + t * kRows * kCols;
#pragma unroll
    for (int it = 0; it < kQ; ++it) cur[it] = ld<kNtLd>(s + quad_offset<LAYOUT>(tid, it));
    for (; t < tiles; t += stride) {
      const int64_t tn = t + stride < tiles ? t + stride : t;  // the last tile reloads itself
      const float* sn = src + tn * kRows * kCols;
#pragma unroll
      for (int it = 0; it < kQ; ++it) nxt[it] = ld<kNtLd>(sn + quad_offset<LAYOUT>(tid, it));
      consume<KIND, LAYOUT, NT>(cur, dst + t * dst_tile_floats, tid, acc);
#pragma unroll
      for (int it = 0; it < kQ; ++it) cur[it] = nxt[it];
    }
  }
  if (acc == 0x9E3779B9u) sink[tid] = acc;  // keeps the reads of kinds 0 and 2 alive
}

template <int KIND, int LAYOUT, int NT>
hipError_t launch(const float* src, float* dst, int64_t tiles, int grid, uint32_t* sink, hipStream_t s) {
  const int64_t g = grid > 0 ? grid : tiles;
  hipLaunchKernelGGL((probe_kernel<KIND, LAYOUT, NT>), dim3((unsigned)g), dim3(kThreads), 0, s, src, dst, tiles,
                     grid > 0 ? 1 : 0, sink);
  return hipGetLastError();
}

template <int KIND, int LAYOUT>
hipError_t by_nt(int nt, const float* src, float* dst, int64_t tiles, int grid, uint32_t* sink, hipStream_t s) {
  switch (nt) {
    case 0: return launch<KIND, LAYOUT, 0>(src, dst, tiles, grid, sink, s);
    case 1: return launch<KIND, LAYOUT, 1>(src, dst, tiles, grid, sink, s);
    case 2: return launch<KIND, LAYOUT, 2>(src, dst, tiles, grid, sink, s);
    default: return launch<KIND, LAYOUT, 3>(src, dst, tiles, grid, sink, s);
  }
}

template <int KIND>
hipError_t by_layout(int layout, int nt, const float* src, float* dst, int64_t tiles, int grid, uint32_t* sink,
                     hipStream_t s) {
  return layout == 0 ? by_nt<KIND, 0>(nt, src, dst, tiles, grid, sink, s) : by_nt<KIND, 1>(nt, src, dst, tiles, grid, sink, s);
}

}  // namespace

extern "C" {

// Bytes of `dst` a probe writes for `tiles` tiles of 64 rows x 512 bytes.
int64_t ssm_probe_dst_bytes(int kind, int64_t tiles) {
  return kind == 1 ? tiles * kRows * kCols * 4 : kind == 2 ? tiles * 8 * kCols * 4 : 0;
}

// Stream `tiles` tiles of src (tiles x 32 KiB, 16-byte aligned device
// memory).  dst holds ssm_probe_dst_bytes(kind, tiles) bytes (unused for
// kind 0); sink is 256 uint32 of device memory.  Returns 0, -3 for
// arguments out of range, -6 for a failed launch.
int ssm_probe_stream(int kind, int layout, int nt, int grid, const float* src, float* dst, int64_t tiles,
                     uint32_t* sink, void* hip_stream) {
  if (kind < 0 || kind > 2 || layout < 0 || layout > 1 || nt < 0 || nt > 3 || tiles <= 0 || tiles > (int64_t)1 << 31 || grid < 0 ||
      !src || !sink || (kind != 0 && !dst))
    return -3;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  hipError_t e;
  switch (kind) {
    case 0: e = by_layout<0>(layout, nt, src, dst, tiles, grid, sink, s); break;
    case 1: e = by_layout<1>(layout, nt, src, dst, tiles, grid, sink, s); break;
    default: e = by_layout<2>(layout, nt, src, dst, tiles, grid, sink, s); break;
  }
  return e == hipSuccess ? 0 : -6;
}

}  // extern "C"
