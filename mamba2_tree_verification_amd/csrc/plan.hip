// plan.hip - the tree plan (SpecMamba page sec. 3.2: breadth-first
// flattening and the FIFO of live states) exported for exact comparison,
// plus the status-only kernel used when a call has no nodes.
#include "common.h"

namespace ssmt {

// one workgroup per sequence
__global__ void __launch_bounds__(64) plan_kernel(const int32_t* parent, int T, int W, int32_t* out) {
  __shared__ int32_t s_parent[kMaxNodes];
  __shared__ int32_t s_depth[kMaxNodes];
  __shared__ uint8_t s_path[kMaxNodes * kMaxNodes];
  const int b = blockIdx.x;
  int32_t* o = out + (int64_t)b * (SSM_TREE_PLAN_HEADER + T * SSM_TREE_PLAN_STRIDE);
  for (int i = threadIdx.x; i < T; i += blockDim.x) s_parent[i] = parent[(int64_t)b * T + i];
  __syncthreads();
  const bool valid = tree_is_valid(s_parent, T);
  for (int i = threadIdx.x; i < SSM_TREE_PLAN_HEADER + T * SSM_TREE_PLAN_STRIDE; i += blockDim.x) o[i] = 0;
  __syncthreads();
  if (!valid) {
    if (threadIdx.x == 0) o[0] = SSM_TREE_E_TREE;
    return;
  }
  build_paths(s_parent, T, s_depth, s_path);
  __syncthreads();
  for (int v = threadIdx.x; v < T; v += blockDim.x) {
    int32_t* r = o + SSM_TREE_PLAN_HEADER + v * SSM_TREE_PLAN_STRIDE;
    // children are the contiguous range of indices whose parent is v
    int first = -1, cnt = 0;
    for (int i = v + 1; i < T; ++i)
      if (s_parent[i] == v) {
        if (first < 0) first = i;
        ++cnt;
      }
    r[0] = s_depth[v];
    r[1] = s_parent[v];
    r[2] = first;
    r[3] = cnt;
    for (int j = 1; j <= 3; ++j) r[4 + j] = (j < W) ? conv_input_code(s_parent, v, j, W) : SSM_TREE_PLAN_UNUSED;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    // FIFO ranks in BFS order and the occupancy of a queue that holds the
    // internal nodes pushed (when their parent is expanded) and not yet
    // popped (when they are expanded themselves).
    int rank = 0, maxd = 0, live = 0, peak = 0;
    for (int v = 0; v < T; ++v) {
      int32_t* r = o + SSM_TREE_PLAN_HEADER + v * SSM_TREE_PLAN_STRIDE;
      r[4] = r[3] > 0 ? rank++ : -1;
      if (r[0] > maxd) maxd = r[0];
    }
    for (int p = -1; p < T; ++p) {
      if (p >= 0) {
        if (o[SSM_TREE_PLAN_HEADER + p * SSM_TREE_PLAN_STRIDE + 3] == 0) continue;
        --live;
      }
      for (int i = p + 1; i < T; ++i)
        if (s_parent[i] == p && o[SSM_TREE_PLAN_HEADER + i * SSM_TREE_PLAN_STRIDE + 3] > 0) {
          ++live;
          if (live > peak) peak = live;
        }
    }
    o[0] = SSM_TREE_OK;
    o[1] = peak;
    o[2] = maxd;
    o[3] = rank;
  }
}

__global__ void status_kernel(int32_t* seq_status, int Bsz, int value) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < Bsz) seq_status[i] = value;
}

hipError_t launch_plan(const int32_t* parent, int Bsz, int T, int W, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(Bsz), dim3(64), 0, s, parent, T, W, out);
  return hipGetLastError();
}

hipError_t launch_status(int32_t* seq_status, int Bsz, int value, hipStream_t s) {
  hipLaunchKernelGGL(status_kernel, dim3((Bsz + 255) / 256), dim3(256), 0, s, seq_status, Bsz, value);
  return hipGetLastError();
}

}  // namespace ssmt
