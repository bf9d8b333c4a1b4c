// common.h - device helpers and launch argument blocks shared by the HIP
// kernels of libssm_tree.so (gfx950 only; wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_tree.h"

namespace ssmt {

constexpr int kWave = 64;
constexpr int kMaxNodes = 64;

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);

template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) {
  return p[i];
}

template <>
__device__ __forceinline__ float load_in<bf16_t>(const bf16_t* p, int64_t i) {
  return bf16_bits_to_float(p[i].bits);
}

// ---------------------------------------------------------------------------
// root-state elements: float32, or bfloat16 with SSM_TREE_STATE_BF16
// (arithmetic is float32 either way; a bfloat16 state is rounded on store)
// ---------------------------------------------------------------------------

typedef float sf32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int su32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two fp32 values rounded to bf16 (first in the low half): the hardware
// conversion v_cvt_pk_bf16_f32, round to nearest even, with subnormals kept
// (the kernels run with fp32 denormals preserved); values past the largest
// finite bf16 become infinite and NaN stays a quiet NaN
__device__ __forceinline__ uint32_t bf16_round_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// four consecutive state elements: Raw is what memory holds
template <typename TS>
struct StateQuad;
template <>
struct StateQuad<float> {
  typedef sf32x4 Raw;
  static __device__ __forceinline__ Raw load(const float* p) { return *reinterpret_cast<const sf32x4*>(p); }
  static __device__ __forceinline__ Raw load_nt(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const sf32x4*>(p));
  }
  static __device__ __forceinline__ sf32x4 to_f32(Raw r) { return r; }
  static __device__ __forceinline__ Raw from_f32(sf32x4 v) { return v; }
  static __device__ __forceinline__ void store(float* p, Raw r) { *reinterpret_cast<sf32x4*>(p) = r; }
  static __device__ __forceinline__ void store_nt(float* p, Raw r) {
    __builtin_nontemporal_store(r, reinterpret_cast<sf32x4*>(p));
  }
};
template <>
struct StateQuad<bf16_t> {
  typedef su32x2 Raw;
  static __device__ __forceinline__ Raw load(const bf16_t* p) { return *reinterpret_cast<const su32x2*>(p); }
  static __device__ __forceinline__ Raw load_nt(const bf16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const su32x2*>(p));
  }
  static __device__ __forceinline__ sf32x4 to_f32(Raw r) {
    return sf32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                  __uint_as_float(r.y & 0xFFFF0000u)};
  }
  static __device__ __forceinline__ Raw from_f32(sf32x4 v) {
    return su32x2{bf16_round_pair(v.x, v.y), bf16_round_pair(v.z, v.w)};
  }
  static __device__ __forceinline__ void store(bf16_t* p, Raw r) { *reinterpret_cast<su32x2*>(p) = r; }
  static __device__ __forceinline__ void store_nt(bf16_t* p, Raw r) {
    __builtin_nontemporal_store(r, reinterpret_cast<su32x2*>(p));
  }
};

// softplus with the large-argument cut-over used by Mamba2 (z for z > 20)
__device__ __forceinline__ float softplus_f32(float z) { return z > 20.0f ? z : log1pf(expf(z)); }

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// silu with the hardware exp2 and reciprocal (about 1 ulp each): z large and
// negative gives exp2 = inf and a zero reciprocal, so the result is -0
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// ---------------------------------------------------------------------------
// launch argument blocks (passed by value)
// ---------------------------------------------------------------------------

struct Dims {
  int32_t L, Bsz, T, H, P, N, G, W, silu;
  int32_t d_in;  // H * P
  int32_t fifo;  // verify by the explicit FIFO walk
  int32_t xbc;   // the conv runs over x, B and C
  int32_t CH;    // conv channels (window row length): d_in, or d_in + 2 G N with xbc
  int32_t sbf16; // the root state is stored as bfloat16
};

struct Params {
  const float* A;
  const float* D;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;
};

struct VerifyArgs {
  Dims d;
  Params prm;
  const int32_t* parent;
  const void* x;
  const void* B;
  const void* C;
  const void* dt_raw;
  const void* z;  // gate input, or null
  const void* window;
  const void* state;  // float32, or bfloat16 with sbf16
  float* y;
  int32_t* seq_status;
};

struct CommitArgs {
  Dims d;
  Params prm;
  const int32_t* parent;
  const int32_t* path;
  const int32_t* path_len;
  const void* x;
  const void* B;
  const void* C;  // read only with xbc
  const void* dt_raw;
  const void* window_in;
  const void* state_in;  // float32, or bfloat16 with sbf16
  void* window_out;
  void* state_out;
  int32_t* seq_status;
};

// the B and C rows of the conv window after a commit with the xBC conv
struct WindowBcArgs {
  Dims d;
  const int32_t* parent;
  const int32_t* path;
  const int32_t* path_len;
  const void* B;  // raw B and C of the committed tree's nodes
  const void* C;
  const void* window_in;
  void* window_out;
  int32_t pass_through;  // a failed commit copies its old rows (else leaves them unwritten)
};

// commit of the previous tree's accepted path fused with verify of the next tree
struct CommitVerifyArgs {
  Dims d;
  Params prm;
  const int32_t* parent_prev;
  const int32_t* path;
  const int32_t* path_len;
  const void* x_prev;
  const void* B_prev;
  const void* C_prev;  // read only with xbc
  const void* dt_prev;
  const void* window_in;
  const void* state_in;  // float32, or bfloat16 with sbf16
  void* window_out;
  void* state_out;
  const int32_t* parent;
  const void* x;
  const void* B;
  const void* C;
  const void* dt_raw;
  const void* z;  // gate input, or null
  float* y;
  int32_t* commit_status;
  int32_t* verify_status;
  // SSM_TREE_CONV_XBC on trees of up to 16 nodes: the convolved B and C rows,
  // [L][Bsz][G] blocks of [T][2N] (next tree, B then C) and [T][N] (the
  // accepted path's B), float32, written by bc_conv_kernel ahead of the round
  float* bcw;
};

// Allow a kernel more than the default 64 KiB of dynamic LDS (gfx950 has
// 160 KiB per CU).
template <typename K>
inline hipError_t allow_lds(K* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

// ---------------------------------------------------------------------------
// tree bookkeeping in LDS (one workgroup, T <= 64)
// ---------------------------------------------------------------------------

// BFS labelling check: parent[0] = -1, -1 <= parent[i] < i, non-decreasing.
// Every thread of the workgroup must call it (it contains a barrier).
__device__ __forceinline__ bool tree_is_valid(const int32_t* s_parent, int T) {
  int bad = 0;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    const int p = s_parent[i];
    if (i == 0)
      bad |= (p != -1);
    else
      bad |= (p < -1) | (p >= i) | (p < s_parent[i - 1]);
  }
  return __syncthreads_or(bad) == 0;
}

// Code of conv input j (1 = parent) of node v: node index, or -(1 + r) for
// row r of the committed window (row W-2 newest).
__device__ __forceinline__ int conv_input_code(const int32_t* s_parent, int v, int j, int W) {
  int u = v;
  int k = 0;
  while (k < j && u >= 0) {
    u = s_parent[u];
    ++k;
  }
  if (u >= 0) return u;
  return -(1 + (W - 2) - (j - k));
}

// Per node: depth and the root path (top first) as uint8 node ids,
// path row stride kMaxNodes.  Threads split the nodes.
__device__ __forceinline__ void build_paths(const int32_t* s_parent, int T, int32_t* s_depth, uint8_t* s_path) {
  for (int v = threadIdx.x; v < T; v += blockDim.x) {
    int d = 0;
    for (int u = v; u >= 0; u = s_parent[u]) ++d;
    s_depth[v] = d;
    int k = d - 1;
    for (int u = v; u >= 0; u = s_parent[u]) s_path[v * kMaxNodes + (k--)] = (uint8_t)u;
  }
}

}  // namespace ssmt
