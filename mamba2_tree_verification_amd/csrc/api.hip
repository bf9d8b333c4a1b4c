// api.hip - the extern "C" entry points of libssm_tree.so: argument
// checks on the host, then kernel launches on the caller's stream.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "common.h"

namespace ssmt {
int launch_verify(const VerifyArgs& a, bool bf16, hipStream_t s);  // status code
hipError_t launch_commit(const CommitArgs& a, bool bf16, hipStream_t s);
bool commit_verify_fused_applies(const Dims& d);
// SSM_TREE_CONV_XBC, the gate and SSM_TREE_STATE_BF16
bool verify_options_supported(const Dims& d, bool gate, bool bf16);
bool commit_options_supported(const Dims& d);
bool commit_verify_options_supported(const Dims& d, bool gate);
int launch_commit_verify(const CommitVerifyArgs& a, bool bf16, hipStream_t s);
size_t bc_workspace_bytes(const Dims& d);
bool tt_round_applies(const Dims& d, bool bf16, bool gate);
int launch_tt_round(const CommitVerifyArgs& a, hipStream_t s);
hipError_t launch_plan(const int32_t* parent, int Bsz, int T, int W, int32_t* out, hipStream_t s);
hipError_t launch_status(int32_t* seq_status, int Bsz, int value, hipStream_t s);
}  // namespace ssmt

using namespace ssmt;

namespace {

// the one-launch round for trees of 17-64 nodes (0 in a build that times
// the two-call form against it)
#ifndef SSMT_TT_ROUND
#define SSMT_TT_ROUND 1
#endif
constexpr bool kTtRound = SSMT_TT_ROUND != 0;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The convolved B and C rows of the xBC conv (trees of up to 16 nodes) live
// in a workspace taken in stream order from a memory pool of the library's
// own, one per device: it is allocated on the caller's stream before the
// kernels and released after them, so calls on different streams never
// share one, and the pool keeps its memory for the next call instead of
// returning it to the device at each synchronisation.
constexpr int kMaxDevices = 64;

hipMemPool_t workspace_pool(hipStream_t s) {
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  static std::mutex m;
  static hipMemPool_t pools[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(m);
  if (!pools[dev]) {
    hipMemPoolProps p;
    memset(&p, 0, sizeof(p));
    p.allocType = hipMemAllocationTypePinned;
    p.location.type = hipMemLocationTypeDevice;
    p.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &p) != hipSuccess) return nullptr;
    uint64_t keep = UINT64_MAX;
    if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
      hipMemPoolDestroy(pool);
      return nullptr;
    }
    pools[dev] = pool;
  }
  return pools[dev];
}

// The allocation-free round (ssm_tree_commit_verify_noalloc) keeps the xBC
// workspace in this fixed device array instead: one copy per device, held
// until the process ends and shared by every such call on that device.
// Nothing in it needs clearing: a round writes every value it reads first.
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) static float scratch[kScratchBytes / sizeof(float)];

// scratch's device address on the stream's device, looked up once per device
// with that device current (the host-side name is not a device address)
float* scratch_address(hipStream_t s) {
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  static std::mutex m;
  static float* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(m);
  if (!addr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (e != hipSuccess || !p) return nullptr;
    addr[dev] = static_cast<float*>(p);
  }
  return addr[dev];
}

// the fused round's kernels, with the xBC conv's workspace when it needs one
// (noalloc: the fixed array, never an allocation)
int run_fused(CommitVerifyArgs& a, bool bf16, hipStream_t s, bool noalloc = false) {
  const size_t bytes = bc_workspace_bytes(a.d);
  if (!bytes) return launch_commit_verify(a, bf16, s);
  if (noalloc) {
    if (bytes > kScratchBytes) return SSM_TREE_E_SCRATCH;
    float* p = scratch_address(s);
    if (!p) return SSM_TREE_E_HIP;
    a.bcw = p;
    return launch_commit_verify(a, bf16, s);
  }
  hipMemPool_t pool = workspace_pool(s);
  void* ws = nullptr;
  if (!pool || hipMallocFromPoolAsync(&ws, bytes, pool, s) != hipSuccess) return SSM_TREE_E_HIP;
  a.bcw = static_cast<float*>(ws);
  const int st = launch_commit_verify(a, bf16, s);
  // released in stream order, after the kernels that read it
  if (hipFreeAsync(ws, s) != hipSuccess && st == SSM_TREE_OK) return SSM_TREE_E_HIP;
  return st;
}

int check_dims(const ssm_tree_dims* dm, Dims* out) {
  if (!dm) return SSM_TREE_E_NULL;
  const ssm_tree_dims& d = *dm;
  if (d.in_dtype != SSM_TREE_F32 && d.in_dtype != SSM_TREE_BF16) return SSM_TREE_E_DTYPE;
  if (d.flags & ~(SSM_TREE_CONV_SILU | SSM_TREE_VERIFY_FIFO | SSM_TREE_CONV_XBC | SSM_TREE_STATE_BF16))
    return SSM_TREE_E_FLAGS;
  if (d.n_layers < 0 || d.batch < 0 || d.n_nodes < 0 || d.n_nodes > kMaxNodes) return SSM_TREE_E_DIMS;
  if (d.nheads < 1 || d.headdim < 1 || d.ngroups < 1 || d.nheads % d.ngroups) return SSM_TREE_E_DIMS;
  if (d.conv_width < 1 || d.conv_width > 4) return SSM_TREE_E_DIMS;
  if (d.d_state != 16 && d.d_state != 32 && d.d_state != 64 && d.d_state != 128 && d.d_state != 256)
    return SSM_TREE_E_DIMS;
  const int64_t di = (int64_t)d.nheads * d.headdim;
  if (di % kWave || di > (1 << 20) || (di / d.ngroups) % kWave) return SSM_TREE_E_DIMS;
  const int64_t units = (int64_t)d.n_layers * d.batch;
  if (d.batch > 65535 || d.n_layers > 65535 || units * di * d.d_state > ((int64_t)1 << 40)) return SSM_TREE_E_DIMS;
  const int xbc = (d.flags & SSM_TREE_CONV_XBC) ? 1 : 0;
  *out = Dims{d.n_layers, d.batch, d.n_nodes, d.nheads, d.headdim, d.d_state, d.ngroups, d.conv_width,
              (d.flags & SSM_TREE_CONV_SILU) ? 1 : 0, (int32_t)di, (d.flags & SSM_TREE_VERIFY_FIFO) ? 1 : 0, xbc,
              (int32_t)(di + (xbc ? 2 * (int64_t)d.ngroups * d.d_state : 0)),
              (d.flags & SSM_TREE_STATE_BF16) ? 1 : 0};
  return SSM_TREE_OK;
}

int check_params(const ssm_tree_params* p) {
  if (!p || !p->A || !p->D || !p->dt_bias || !p->conv_w) return SSM_TREE_E_NULL;
  if (misaligned(p->A) || misaligned(p->D) || misaligned(p->dt_bias) || misaligned(p->conv_w) ||
      (p->conv_b && misaligned(p->conv_b)))
    return SSM_TREE_E_ALIGN;
  return SSM_TREE_OK;
}

}  // namespace

extern "C" {

int ssm_tree_abi_version(void) { return SSM_TREE_ABI_VERSION; }

const char* ssm_tree_status_string(int status) {
  switch (status) {
    case SSM_TREE_OK: return "ok";
    case SSM_TREE_E_NULL: return "a required pointer is NULL";
    case SSM_TREE_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SSM_TREE_E_DIMS: return "unsupported or inconsistent dimensions";
    case SSM_TREE_E_DTYPE: return "unknown input dtype";
    case SSM_TREE_E_ALIAS: return "an output overlaps an input";
    case SSM_TREE_E_HIP: return "HIP kernel launch failed";
    case SSM_TREE_E_FLAGS: return "unknown flag bits";
    case SSM_TREE_E_SCRATCH: return "the call needs more scratch memory than the allocation-free entry point holds";
    case SSM_TREE_E_TREE: return "parent[] is not a BFS-ordered tree";
    case SSM_TREE_E_PATH: return "path is not a root-to-node path of the tree";
    default: return "unknown status";
  }
}

int ssm_tree_verify(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent,
                    const void* x, const void* B, const void* C, const void* dt_raw, const void* z,
                    const void* conv_window, const void* state, float* y, int32_t* seq_status, void* hip_stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  if (d.L == 0 || d.Bsz == 0) return SSM_TREE_OK;
  if (d.T == 0) {
    if (seq_status) return launch_status(seq_status, d.Bsz, SSM_TREE_OK, s) == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
    return SSM_TREE_OK;
  }
  if (!verify_options_supported(d, z != nullptr, dims->in_dtype == SSM_TREE_BF16)) return SSM_TREE_E_DIMS;
  if ((st = check_params(params))) return st;
  if (!parent || !x || !B || !C || !dt_raw || !state || !y || (d.W > 1 && !conv_window)) return SSM_TREE_E_NULL;
  const void* ptrs[] = {parent, x, B, C, dt_raw, z, state, y, seq_status, d.W > 1 ? conv_window : nullptr};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return SSM_TREE_E_ALIGN;
  const int64_t e = dims->in_dtype == SSM_TREE_BF16 ? 2 : 4, es = d.sbf16 ? 2 : 4;
  const int64_t U = (int64_t)d.L * d.Bsz, T = d.T, DI = d.d_in, CH = d.CH;
  const Range ry = range_of(y, U * T * DI * 4);
  const Range ins[] = {range_of(parent, (int64_t)d.Bsz * T * 4), range_of(x, U * T * DI * e),
                       range_of(B, U * T * d.G * d.N * e), range_of(C, U * T * d.G * d.N * e),
                       range_of(dt_raw, U * T * d.H * e), range_of(z, z ? U * T * DI * e : 0),
                       range_of(state, U * DI * d.N * es),
                       range_of(conv_window, d.W > 1 ? U * (d.W - 1) * CH * e : 0),
                       range_of(params->A, d.L * (int64_t)d.H * 4), range_of(params->D, d.L * (int64_t)d.H * 4),
                       range_of(params->dt_bias, d.L * (int64_t)d.H * 4),
                       range_of(params->conv_w, d.L * CH * d.W * 4),
                       range_of(params->conv_b, params->conv_b ? d.L * CH * 4 : 0)};
  for (const Range& r : ins)
    if (overlaps(ry, r)) return SSM_TREE_E_ALIAS;
  if (seq_status) {
    const Range rs = range_of(seq_status, (int64_t)d.Bsz * 4);
    if (overlaps(rs, ry)) return SSM_TREE_E_ALIAS;
    for (const Range& r : ins)
      if (overlaps(rs, r)) return SSM_TREE_E_ALIAS;
  }
  if ((d.xbc || z) && commit_verify_fused_applies(d)) {
    // the options on trees of 1-16 nodes run on the fused round's kernel
    // with nothing to commit: no path length, no state or window output
    CommitVerifyArgs a;
    memset(&a, 0, sizeof(a));
    a.d = d;
    a.prm = Params{params->A, params->D, params->dt_bias, params->conv_w, params->conv_b};
    a.parent_prev = parent;  // read but unused: the commit is empty
    a.path = parent;
    a.x_prev = x;
    a.B_prev = B;
    a.C_prev = C;
    a.dt_prev = dt_raw;
    a.window_in = conv_window;
    a.state_in = state;
    a.parent = parent;
    a.x = x;
    a.B = B;
    a.C = C;
    a.dt_raw = dt_raw;
    a.z = z;
    a.y = y;
    a.verify_status = seq_status;
    return run_fused(a, dims->in_dtype == SSM_TREE_BF16, s);
  }
  VerifyArgs a;
  a.d = d;
  a.prm = Params{params->A, params->D, params->dt_bias, params->conv_w, params->conv_b};
  a.parent = parent;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt_raw = dt_raw;
  a.z = z;
  a.window = conv_window;
  a.state = state;
  a.y = y;
  a.seq_status = seq_status;
  return launch_verify(a, dims->in_dtype == SSM_TREE_BF16, s);
}

int ssm_tree_commit(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent,
                    const int32_t* path, const int32_t* path_len, const void* x, const void* B, const void* C,
                    const void* dt_raw, const void* conv_window_in, const void* state_in, void* conv_window_out,
                    void* state_out, int32_t* seq_status, void* hip_stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  if (d.L == 0 || d.Bsz == 0) return SSM_TREE_OK;
  if (!commit_options_supported(d)) return SSM_TREE_E_DIMS;
  if ((st = check_params(params))) return st;
  if (!path_len || !state_in || !state_out) return SSM_TREE_E_NULL;
  if (d.T > 0 && (!parent || !path || !x || !B || !dt_raw || (d.xbc && !C))) return SSM_TREE_E_NULL;
  if (d.W > 1 && (!conv_window_in || !conv_window_out)) return SSM_TREE_E_NULL;
  const void* Cx = d.xbc ? C : nullptr;  // C is read only with the xBC conv
  const void* ptrs[] = {parent, path, path_len, x, B, Cx, dt_raw, state_in, state_out, seq_status,
                        d.W > 1 ? conv_window_in : nullptr, d.W > 1 ? conv_window_out : nullptr};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return SSM_TREE_E_ALIGN;
  const int64_t e = dims->in_dtype == SSM_TREE_BF16 ? 2 : 4, es = d.sbf16 ? 2 : 4;
  const int64_t U = (int64_t)d.L * d.Bsz, T = d.T, DI = d.d_in, CH = d.CH;
  const int64_t wbytes = d.W > 1 ? U * (d.W - 1) * CH * e : 0;
  const Range rso = range_of(state_out, U * DI * d.N * es), rsi = range_of(state_in, U * DI * d.N * es);
  const Range rwo = range_of(conv_window_out, wbytes), rwi = range_of(conv_window_in, wbytes);
  const Range others[] = {range_of(parent, (int64_t)d.Bsz * T * 4), range_of(path, (int64_t)d.Bsz * T * 4),
                          range_of(path_len, (int64_t)d.Bsz * 4), range_of(x, U * T * DI * e),
                          range_of(B, U * T * d.G * d.N * e), range_of(Cx, Cx ? U * T * d.G * d.N * e : 0),
                          range_of(dt_raw, U * T * d.H * e),
                          range_of(params->A, d.L * (int64_t)d.H * 4), range_of(params->D, d.L * (int64_t)d.H * 4),
                          range_of(params->dt_bias, d.L * (int64_t)d.H * 4),
                          range_of(params->conv_w, d.L * CH * d.W * 4),
                          range_of(params->conv_b, params->conv_b ? d.L * CH * 4 : 0)};
  // outputs: exact in-place allowed, any other overlap rejected
  if (state_out != state_in && overlaps(rso, rsi)) return SSM_TREE_E_ALIAS;
  if (d.W > 1 && conv_window_out != conv_window_in && overlaps(rwo, rwi)) return SSM_TREE_E_ALIAS;
  if (overlaps(rso, rwo) || overlaps(rso, rwi) || overlaps(rwo, rsi)) return SSM_TREE_E_ALIAS;
  for (const Range& r : others)
    if (overlaps(rso, r) || overlaps(rwo, r)) return SSM_TREE_E_ALIAS;
  if (seq_status) {
    const Range rs = range_of(seq_status, (int64_t)d.Bsz * 4);
    if (overlaps(rs, rso) || overlaps(rs, rwo) || overlaps(rs, rsi) || overlaps(rs, rwi)) return SSM_TREE_E_ALIAS;
    for (const Range& r : others)
      if (overlaps(rs, r)) return SSM_TREE_E_ALIAS;
  }
  CommitArgs a;
  a.d = d;
  a.prm = Params{params->A, params->D, params->dt_bias, params->conv_w, params->conv_b};
  a.parent = parent;
  a.path = path;
  a.path_len = path_len;
  a.x = x;
  a.B = B;
  a.C = Cx;
  a.dt_raw = dt_raw;
  a.window_in = conv_window_in;
  a.state_in = state_in;
  a.window_out = conv_window_out;
  a.state_out = state_out;
  a.seq_status = seq_status;
  return launch_commit(a, dims->in_dtype == SSM_TREE_BF16, s) == hipSuccess ? SSM_TREE_OK : SSM_TREE_E_HIP;
}

static int commit_verify_impl(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent_prev,
                              const int32_t* path, const int32_t* path_len, const void* x_prev, const void* B_prev,
                              const void* C_prev, const void* dt_raw_prev, const void* conv_window_in,
                              const void* state_in, void* conv_window_out, void* state_out, const int32_t* parent,
                              const void* x, const void* B, const void* C, const void* dt_raw, const void* z,
                              float* y, int32_t* commit_status, int32_t* verify_status, void* hip_stream,
                              bool noalloc) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st) return st;
  if (d.L == 0 || d.Bsz == 0) return SSM_TREE_OK;
  const bool fused = !d.fifo && commit_verify_fused_applies(d);
  // the options (xBC conv, gate, bfloat16 state) must be supported by
  // whichever kernels run, checked before anything is enqueued
  if ((d.xbc || z || d.sbf16) && d.T > 0 &&
      !(fused ? commit_verify_options_supported(d, z != nullptr)
              : commit_options_supported(d) &&
                    verify_options_supported(d, z != nullptr, dims->in_dtype == SSM_TREE_BF16)))
    return SSM_TREE_E_DIMS;
  if ((st = check_params(params))) return st;
  if (!path_len || !state_in || !state_out) return SSM_TREE_E_NULL;
  if (d.T > 0 && (!parent_prev || !path || !x_prev || !B_prev || !dt_raw_prev || !parent || !x || !B || !C ||
                  !dt_raw || !y || (d.xbc && !C_prev)))
    return SSM_TREE_E_NULL;
  if (d.W > 1 && (!conv_window_in || !conv_window_out)) return SSM_TREE_E_NULL;
  const void* Cp = d.xbc ? C_prev : nullptr;  // read only with the xBC conv
  const void* ptrs[] = {parent_prev, path, path_len, x_prev, B_prev, Cp, dt_raw_prev, state_in, state_out, parent,
                        x, B, C, dt_raw, z, y, commit_status, verify_status,
                        d.W > 1 ? conv_window_in : nullptr, d.W > 1 ? conv_window_out : nullptr};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return SSM_TREE_E_ALIGN;
  const int64_t e = dims->in_dtype == SSM_TREE_BF16 ? 2 : 4, es = d.sbf16 ? 2 : 4;
  const int64_t U = (int64_t)d.L * d.Bsz, T = d.T, DI = d.d_in, CH = d.CH;
  const int64_t wbytes = d.W > 1 ? U * (d.W - 1) * CH * e : 0;
  const int64_t bcb = U * T * d.G * d.N * e;
  const Range rso = range_of(state_out, U * DI * d.N * es), rsi = range_of(state_in, U * DI * d.N * es);
  const Range rwo = range_of(conv_window_out, wbytes), rwi = range_of(conv_window_in, wbytes);
  const Range ry = range_of(y, U * T * DI * 4);
  const Range rcs = range_of(commit_status, commit_status ? (int64_t)d.Bsz * 4 : 0);
  const Range rvs = range_of(verify_status, verify_status ? (int64_t)d.Bsz * 4 : 0);
  const Range ins[] = {range_of(parent_prev, (int64_t)d.Bsz * T * 4), range_of(path, (int64_t)d.Bsz * T * 4),
                       range_of(path_len, (int64_t)d.Bsz * 4), range_of(x_prev, U * T * DI * e),
                       range_of(B_prev, bcb), range_of(Cp, Cp ? bcb : 0), range_of(dt_raw_prev, U * T * d.H * e),
                       range_of(parent, (int64_t)d.Bsz * T * 4), range_of(x, U * T * DI * e), range_of(B, bcb),
                       range_of(C, bcb), range_of(dt_raw, U * T * d.H * e), range_of(z, z ? U * T * DI * e : 0),
                       range_of(params->A, d.L * (int64_t)d.H * 4), range_of(params->D, d.L * (int64_t)d.H * 4),
                       range_of(params->dt_bias, d.L * (int64_t)d.H * 4),
                       range_of(params->conv_w, d.L * CH * d.W * 4),
                       range_of(params->conv_b, params->conv_b ? d.L * CH * 4 : 0)};
  // outputs: state and window may equal their inputs exactly; nothing else may overlap
  if (state_out != state_in && overlaps(rso, rsi)) return SSM_TREE_E_ALIAS;
  if (d.W > 1 && conv_window_out != conv_window_in && overlaps(rwo, rwi)) return SSM_TREE_E_ALIAS;
  const Range outs[] = {rso, rwo, ry, rcs, rvs};
  for (int i = 0; i < 5; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return SSM_TREE_E_ALIAS;
    for (int k = i + 1; k < 5; ++k)
      if (overlaps(outs[i], outs[k])) return SSM_TREE_E_ALIAS;
    if (i >= 1 && overlaps(outs[i], rsi)) return SSM_TREE_E_ALIAS;
    if (i != 1 && overlaps(outs[i], rwi)) return SSM_TREE_E_ALIAS;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool bf16 = dims->in_dtype == SSM_TREE_BF16;
  CommitVerifyArgs a;
  memset(&a, 0, sizeof(a));
  a.d = d;
  a.prm = Params{params->A, params->D, params->dt_bias, params->conv_w, params->conv_b};
  a.parent_prev = parent_prev;
  a.path = path;
  a.path_len = path_len;
  a.x_prev = x_prev;
  a.B_prev = B_prev;
  a.C_prev = Cp;
  a.dt_prev = dt_raw_prev;
  a.window_in = conv_window_in;
  a.state_in = state_in;
  a.window_out = conv_window_out;
  a.state_out = state_out;
  a.parent = parent;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt_raw = dt_raw;
  a.z = z;
  a.y = y;
  a.commit_status = commit_status;
  a.verify_status = verify_status;
  if (fused) return run_fused(a, bf16, s, noalloc);
  // (no other path of the round uses scratch memory: the two calls below
  // never reach the xBC workspace, which only the fused shapes take)
  // trees of 17-64 nodes: one launch where the role-split verify applies
  // (E_DIMS from it: nothing was launched)
  if (kTtRound && tt_round_applies(d, bf16, z != nullptr)) {
    st = launch_tt_round(a, s);
    if (st != SSM_TREE_E_DIMS) return st;
  }
  // The two calls in turn, on the same stream.  The outputs first receive
  // the inputs and the commit then runs in place on them, so that a
  // sequence whose commit fails carries its old state and window into the
  // verify, as the fused kernels do.
  if (state_out != state_in &&
      hipMemcpyAsync(state_out, state_in, rso.hi - rso.lo, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SSM_TREE_E_HIP;
  if (wbytes && conv_window_out != conv_window_in &&
      hipMemcpyAsync(conv_window_out, conv_window_in, wbytes, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SSM_TREE_E_HIP;
  st = ssm_tree_commit(dims, params, parent_prev, path, path_len, x_prev, B_prev, Cp, dt_raw_prev, conv_window_out,
                       state_out, conv_window_out, state_out, commit_status, hip_stream);
  if (st) return st;
  return ssm_tree_verify(dims, params, parent, x, B, C, dt_raw, z, conv_window_out, state_out, y, verify_status,
                         hip_stream);
}

int ssm_tree_commit_verify(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent_prev,
                           const int32_t* path, const int32_t* path_len, const void* x_prev, const void* B_prev,
                           const void* C_prev, const void* dt_raw_prev, const void* conv_window_in,
                           const void* state_in, void* conv_window_out, void* state_out, const int32_t* parent,
                           const void* x, const void* B, const void* C, const void* dt_raw, const void* z,
                           float* y, int32_t* commit_status, int32_t* verify_status, void* hip_stream) {
  return commit_verify_impl(dims, params, parent_prev, path, path_len, x_prev, B_prev, C_prev, dt_raw_prev,
                            conv_window_in, state_in, conv_window_out, state_out, parent, x, B, C, dt_raw, z, y,
                            commit_status, verify_status, hip_stream, false);
}

int ssm_tree_commit_verify_noalloc(const ssm_tree_dims* dims, const ssm_tree_params* params,
                                   const int32_t* parent_prev, const int32_t* path, const int32_t* path_len,
                                   const void* x_prev, const void* B_prev, const void* C_prev,
                                   const void* dt_raw_prev, const void* conv_window_in, const void* state_in,
                                   void* conv_window_out, void* state_out, const int32_t* parent, const void* x,
                                   const void* B, const void* C, const void* dt_raw, const void* z, float* y,
                                   int32_t* commit_status, int32_t* verify_status, void* hip_stream) {
  return commit_verify_impl(dims, params, parent_prev, path, path_len, x_prev, B_prev, C_prev, dt_raw_prev,
                            conv_window_in, state_in, conv_window_out, state_out, parent, x, B, C, dt_raw, z, y,
                            commit_status, verify_status, hip_stream, true);
}

int ssm_tree_plan(const ssm_tree_dims* dims, const int32_t* parent, int32_t* plan_out, void* hip_stream) {
  if (!dims) return SSM_TREE_E_NULL;
  if (dims->batch < 0 || dims->n_nodes < 0 || dims->n_nodes > kMaxNodes || dims->conv_width < 1 ||
      dims->conv_width > 4 || dims->batch > 65535)
    return SSM_TREE_E_DIMS;
  if (dims->batch == 0) return SSM_TREE_OK;
  if (!plan_out || (dims->n_nodes > 0 && !parent)) return SSM_TREE_E_NULL;
  if (misaligned(plan_out) || (parent && misaligned(parent))) return SSM_TREE_E_ALIGN;
  const int64_t nb = (int64_t)dims->batch * (SSM_TREE_PLAN_HEADER + dims->n_nodes * SSM_TREE_PLAN_STRIDE) * 4;
  if (parent && overlaps(range_of(plan_out, nb), range_of(parent, (int64_t)dims->batch * dims->n_nodes * 4)))
    return SSM_TREE_E_ALIAS;
  return launch_plan(parent, dims->batch, dims->n_nodes, dims->conv_width, plan_out,
                     reinterpret_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? SSM_TREE_OK
             : SSM_TREE_E_HIP;
}

}  // extern "C"
