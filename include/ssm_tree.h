/*
 * ssm_tree.h - C ABI of libssm_tree.so: verifying a speculative draft-token
 * tree through Mamba2 selective-SSM layers on AMD Instinct MI355X (gfx950).
 *
 * The operation (from the pages that describe the method):
 *   SpecMamba page, "FPGA加速Mamba推理：SpecMamba方案与优化实践"
 *   (jsqmd.com/news/939380):
 *     sec. 2.1  rejecting draft tokens needs the hidden state of the last
 *               accepted token, and keeping every intermediate state is too
 *               costly;
 *     sec. 3.1  draft side stores only the per-token Delta, A, B, X; the
 *               target recomputes only the affected path;
 *     sec. 3.2  the candidate tree is flattened breadth-first and verified
 *               with a FIFO of live states, each child state formed from its
 *               parent's, a state released once its children are done;
 *     sec. 5.2  trees of branching 2-3, depth 4-5, 12-16 predicted tokens.
 *   LightMamba part of "FPGA accelerator part 2"
 *   (pinghaoyang.com.cn/aigc/posts/fpga-accelerator-part-2/), "why Mamba is
 *   hard to accelerate": in_proj yields X, B, C, Delta, Z; X passes conv1d,
 *   the SSM keeps h_t and emits Y; the recurrence fragments read
 *   h_t = Abar (.) h_{t-1} + Bbar (.) X_t.
 *
 * Per (layer l, sequence b, node v, head h, headdim row p, state index n),
 * with g = h / (H / G) and c = h * P + p (shown for the default conv over
 * x; SSM_TREE_CONV_XBC convolves B and C the same way, and a gate input z
 * multiplies y by silu(z)):
 *   dt_v[h]  = softplus(dt_raw_v[h] + dt_bias[h])   (softplus(z) = z, z > 20)
 *   dA_v[h]  = exp(dt_v[h] * A[h])
 *   x~_v[c]  = act(conv_b[c] + sum_{j<W} conv_w[c][W-1-j] * u_j[c])
 *              u_0 = x_v, u_j = x of the j-th ancestor of v, continuing into
 *              the conv window newest row first once past the tree root;
 *              act = identity, or SiLU with SSM_TREE_CONV_SILU
 *   h_v      = dA_v[h] * h_parent(v) + (dt_v[h] * x~_v[c]) * B_v[g][n]
 *              (h_parent = root state for parent -1)
 *   y_v[c]   = sum_n C_v[g][n] * h_v[h][p][n] + D[h] * x~_v[c]
 *
 * Memory: every tensor argument is a DEVICE pointer to contiguous row-major
 * data, 16-byte aligned, allocated and owned by the caller.  The library
 * allocates nothing, keeps no mutable global state and is reentrant; it
 * enqueues work on `hip_stream` (a hipStream_t, NULL = default stream) and
 * returns without synchronising.  Structs are read on the host during the
 * call only.
 *
 * Errors: the return value is SSM_TREE_OK or a negative code for problems
 * detectable on the host (nothing is enqueued then).  Problems that depend
 * on device data (an invalid parent[] or path) are reported per sequence in
 * seq_status[b] once the stream reaches the work; other sequences are
 * processed normally.
 */
#ifndef SSM_TREE_H
#define SSM_TREE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_TREE_ABI_VERSION 4

/* input element types for x, B, C, dt_raw and the conv window */
#define SSM_TREE_F32 0
#define SSM_TREE_BF16 1

/* dims.flags */
#define SSM_TREE_CONV_SILU 1 /* SiLU after the conv (Mamba2 checkpoints use it; the pages name no activation) */
/* The causal conv runs over x, B and C (the Mamba2 convention: in_proj's
 * xBC passes conv1d as a whole) instead of over x only.  The conv window,
 * conv_w and conv_b then span CH = H*P + 2*G*N channels in the order x,
 * B [G][N], C [G][N]; the SSM uses the convolved B and C.  Supported by
 * ssm_tree_verify and ssm_tree_commit_verify for trees of 1 to 64 nodes
 * with a headdim that is a multiple of 16 and, past 16 nodes, (H*P/G) a
 * multiple of 64 and the float32-staged B and C rows within the LDS (bf16
 * inputs: d_state up to 128 at 64 nodes, 256 up to 32 nodes; fp32 inputs:
 * up to 64 at 64 nodes, 128 up to 48 nodes, 256 up to 32 nodes); not with
 * SSM_TREE_VERIFY_FIFO; and by
 * ssm_tree_commit for every supported shape.  Other combinations return
 * SSM_TREE_E_DIMS before anything is enqueued.
 * On trees of 1 to 16 nodes ssm_tree_verify and ssm_tree_commit_verify
 * first convolve each sequence's B and C rows once, into a workspace of
 * L*Bsz*G*(T*3*N + 256) float32 values that the library takes in stream order
 * from a memory pool of its own on the stream's device and releases, in
 * stream order, after the kernels that read it (SSM_TREE_E_HIP if that
 * allocation fails). */
#define SSM_TREE_CONV_XBC 4
/* ssm_tree_verify computes every child state explicitly, walking the tree
 * breadth-first with a FIFO of live states (SpecMamba page sec. 3.2), instead
 * of the default root projection.  Same outputs up to fp32 rounding; slower.
 * Ignored by ssm_tree_commit. */
#define SSM_TREE_VERIFY_FIFO 2
/* The root state (state, state_in, state_out) is stored as bfloat16 instead
 * of float32, halving its bytes, which dominate the traffic (SpecMamba page
 * sec. 3.1 lists mixed precision among its memory optimisations; the
 * format is a reading).  Arithmetic stays float32; a committed state is
 * rounded to the nearest bfloat16, ties to even, when stored, and the
 * fused round verifies the next tree from that stored value.  Supported by
 * ssm_tree_commit for every shape; by ssm_tree_verify for trees of 1 to 64
 * nodes with a headdim that is a multiple of 16 (and, past 16 nodes,
 * (H*P/G) a multiple of 64; not fp32 inputs with d_state 256 past 16
 * nodes); by ssm_tree_commit_verify where both its calls are; never with
 * SSM_TREE_VERIFY_FIFO, SSM_TREE_CONV_XBC or the gate.  Other combinations
 * return SSM_TREE_E_DIMS before anything is enqueued. */
#define SSM_TREE_STATE_BF16 8

/* return / status codes */
#define SSM_TREE_OK 0
#define SSM_TREE_E_NULL (-1)   /* a required pointer is NULL */
#define SSM_TREE_E_ALIGN (-2)  /* a tensor pointer is not 16-byte aligned */
#define SSM_TREE_E_DIMS (-3)   /* unsupported or inconsistent dimensions */
#define SSM_TREE_E_DTYPE (-4)  /* unknown in_dtype */
#define SSM_TREE_E_ALIAS (-5)  /* an output overlaps an input (other than an allowed exact in-place) */
#define SSM_TREE_E_HIP (-6)    /* a HIP launch failed */
#define SSM_TREE_E_FLAGS (-7)  /* unknown bits in dims.flags */
#define SSM_TREE_E_SCRATCH (-8) /* ssm_tree_commit_verify_noalloc: the call needs more than its fixed scratch */
#define SSM_TREE_E_TREE (-10)  /* seq_status: parent[] is not a BFS labelling */
#define SSM_TREE_E_PATH (-11)  /* seq_status: path is not a root-to-node path of the tree */

/* Dimensions.  Supported: 0 <= n_nodes <= 64; d_state in {16,32,64,128,256};
 * 1 <= conv_width <= 4; nheads % ngroups == 0; nheads*headdim a multiple of
 * 64 and (nheads*headdim/ngroups) a multiple of 64. */
typedef struct ssm_tree_dims {
  int32_t n_layers;   /* L   : independent layer instances in this call */
  int32_t batch;      /* Bsz : sequences, each with its own tree */
  int32_t n_nodes;    /* T   : nodes per tree */
  int32_t nheads;     /* H */
  int32_t headdim;    /* P */
  int32_t d_state;    /* N */
  int32_t ngroups;    /* G : B and C are shared by H/G consecutive heads */
  int32_t conv_width; /* W */
  int32_t in_dtype;   /* SSM_TREE_F32 or SSM_TREE_BF16 */
  int32_t flags;      /* 0 or SSM_TREE_CONV_SILU | SSM_TREE_VERIFY_FIFO | SSM_TREE_CONV_XBC | SSM_TREE_STATE_BF16 */
} ssm_tree_dims;

/* Per-layer parameters, float32 device pointers. */
typedef struct ssm_tree_params {
  const float* A;       /* [L][H]        decay rate per head (negative in Mamba2) */
  const float* D;       /* [L][H]        skip weight per head */
  const float* dt_bias; /* [L][H] */
  const float* conv_w;  /* [L][CH][W]    depthwise conv weights, tap W-1 = current token;
                           CH = H*P, or H*P + 2*G*N with SSM_TREE_CONV_XBC */
  const float* conv_b;  /* [L][CH]       or NULL for no conv bias */
} ssm_tree_params;

/*
 * ssm_tree_verify: every node's output y for every layer and sequence.
 *
 * parent      [Bsz][T] int32.  BFS labelling: parent[0] = -1,
 *             -1 <= parent[i] < i, parent[] non-decreasing (children of a
 *             node are a contiguous index range).  -1 = child of the root
 *             state.  Shared by all layers.
 * x           [L][Bsz][T][H*P]   in_dtype   per-node conv input
 * B, C        [L][Bsz][T][G][N]  in_dtype
 * dt_raw      [L][Bsz][T][H]     in_dtype   step size before bias/softplus
 * z           [L][Bsz][T][H*P]   in_dtype   gate input, or NULL for no gate:
 *             y = (C . h + D x~) * silu(z) ([LM] "why Mamba is hard to
 *             accelerate": Y is multiplied elementwise with Z).  Supported
 *             with the same shapes as SSM_TREE_CONV_XBC.
 * conv_window [L][Bsz][W-1][CH]  in_dtype   raw conv inputs (x, and B and C
 *             with SSM_TREE_CONV_XBC) of the last W-1 committed tokens,
 *             oldest row first (may be NULL when W == 1)
 * state       [L][Bsz][H][P][N]  float32, or bfloat16 with SSM_TREE_STATE_BF16:
 *             root SSM state (read only)
 * y           [L][Bsz][T][H][P]  float32    out; must not overlap any input
 * seq_status  [Bsz] int32 out, or NULL.  SSM_TREE_OK or SSM_TREE_E_TREE;
 *             a sequence with an invalid tree gets NaN in all its y.
 *
 * Child states are never written to memory: the root state is read once.
 */
int ssm_tree_verify(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent,
                    const void* x, const void* B, const void* C, const void* dt_raw, const void* z,
                    const void* conv_window, const void* state, float* y, int32_t* seq_status, void* hip_stream);

/*
 * ssm_tree_commit: advance the root state and conv window along the
 * accepted path (SpecMamba page sec. 3.1: recompute the accepted path from
 * the stored per-token dt, B and x instead of storing per-node states).
 *
 * path        [Bsz][T] int32: path[b][0..len) = root-level node, its child,
 *             ... (entries past len are ignored)
 * path_len    [Bsz] int32, 0 <= len <= T (0 = keep state and window)
 * x, B, dt_raw, conv_window_in, state_in: as for ssm_tree_verify
 * C           as for ssm_tree_verify; read only with SSM_TREE_CONV_XBC (for
 *             the window) and may be NULL otherwise
 * conv_window_out [L][Bsz][W-1][CH] in_dtype: last W-1 rows of
 *             (old window, raw conv inputs of each path node), copied bit
 *             for bit
 * state_out   [L][Bsz][H][P][N] float32 (bfloat16 with SSM_TREE_STATE_BF16,
 *             rounded to nearest even): state of the last path node
 * Outputs may equal the matching input exactly (in place); any other
 * overlap is SSM_TREE_E_ALIAS.
 * seq_status  [Bsz] or NULL: SSM_TREE_OK, SSM_TREE_E_TREE or SSM_TREE_E_PATH;
 *             a failed sequence's outputs are left unwritten.
 */
int ssm_tree_commit(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent,
                    const int32_t* path, const int32_t* path_len, const void* x, const void* B, const void* C,
                    const void* dt_raw, const void* conv_window_in, const void* state_in, void* conv_window_out,
                    void* state_out, int32_t* seq_status, void* hip_stream);

/*
 * ssm_tree_commit_verify: ssm_tree_commit of the previous tree's accepted
 * path followed by ssm_tree_verify of the next tree from the committed state
 * and window, in one pass over the root state (it is read and written once
 * instead of being read by verify and read and written by commit).
 *
 * parent_prev, path, path_len, x_prev, B_prev, C_prev, dt_raw_prev: the
 *             previous tree and its accepted path, as for ssm_tree_commit
 *             (C_prev read only with SSM_TREE_CONV_XBC, may be NULL otherwise)
 * conv_window_in, state_in -> conv_window_out, state_out: as for
 *             ssm_tree_commit (exact in-place allowed)
 * parent, x, B, C, dt_raw, z: the next tree, as for ssm_tree_verify (same
 *             dims: T nodes; z NULL for no gate)
 * y           [L][Bsz][T][H*P] float32 out: the next tree's outputs
 * commit_status [Bsz] or NULL: as ssm_tree_commit's seq_status.  A sequence
 *             whose commit fails gets its state_in and conv_window_in copied
 *             unchanged to state_out and conv_window_out, and its next tree
 *             is verified from them.
 * verify_status [Bsz] or NULL: as ssm_tree_verify's seq_status (next tree).
 * Outputs equal ssm_tree_commit followed by ssm_tree_verify up to fp32
 * rounding.  One launch: trees of 1 to 16 nodes with a headdim that is a
 * multiple of 16; trees of 17 to 64 nodes with bf16 inputs, d_state <= 128,
 * a headdim that is a multiple of 64, (H*P/G) a multiple of 512 and neither
 * SSM_TREE_CONV_XBC nor a gate (the accepted path is then committed in
 * closed form, exp of fp64 prefix sums of dt*A weighting each path token:
 * equal to the sequential replay up to fp32 rounding).  Other shapes, and
 * dims.flags with SSM_TREE_VERIFY_FIFO, copy state and window to the
 * outputs (unless in place), run ssm_tree_commit in place on them and then
 * ssm_tree_verify.
 * Host-side errors as for the two calls; every output range is checked
 * against every input range before anything is enqueued.
 */
int ssm_tree_commit_verify(const ssm_tree_dims* dims, const ssm_tree_params* params, const int32_t* parent_prev,
                           const int32_t* path, const int32_t* path_len, const void* x_prev, const void* B_prev,
                           const void* C_prev, const void* dt_raw_prev, const void* conv_window_in,
                           const void* state_in, void* conv_window_out, void* state_out, const int32_t* parent,
                           const void* x, const void* B, const void* C, const void* dt_raw, const void* z,
                           float* y, int32_t* commit_status, int32_t* verify_status, void* hip_stream);

/*
 * ssm_tree_commit_verify_noalloc: ssm_tree_commit_verify for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, outputs, status
 * codes and kernels; it calls no allocating routine.
 * The one scratch buffer a round uses, the convolved B and C rows of
 * SSM_TREE_CONV_XBC on trees of 1 to 16 nodes (L*Bsz*G*(T*3*N + 256)
 * float32 values), is here a fixed device array of 32 MiB that the library holds on
 * each device it runs on until the process ends, instead of the stream-
 * ordered pool allocation ssm_tree_commit_verify makes.  A call that needs
 * more returns SSM_TREE_E_SCRATCH before anything is enqueued.  Every call
 * on one device shares that array, which keeps the last call's contents
 * (nothing needs clearing: a round writes each value it reads first), so
 * calls that overlap on one device (other streams, other threads) race:
 * the caller serialises them.  Calls that need no scratch (no
 * SSM_TREE_CONV_XBC, or more than 16 nodes) behave exactly as
 * ssm_tree_commit_verify.
 */
int ssm_tree_commit_verify_noalloc(const ssm_tree_dims* dims, const ssm_tree_params* params,
                                   const int32_t* parent_prev, const int32_t* path, const int32_t* path_len,
                                   const void* x_prev, const void* B_prev, const void* C_prev,
                                   const void* dt_raw_prev, const void* conv_window_in, const void* state_in,
                                   void* conv_window_out, void* state_out, const int32_t* parent, const void* x,
                                   const void* B, const void* C, const void* dt_raw, const void* z, float* y,
                                   int32_t* commit_status, int32_t* verify_status, void* hip_stream);

/*
 * ssm_tree_plan: the tree plan the kernels derive from parent[] (SpecMamba
 * page sec. 3.2: breadth-first flattening, FIFO of live states), exported
 * so that its integer bookkeeping can be compared exactly.
 *
 * plan_out [Bsz][SSM_TREE_PLAN_HEADER + T * SSM_TREE_PLAN_STRIDE] int32:
 *   header: status, peak FIFO occupancy (internal nodes pushed and not yet
 *           popped), maximum depth, number of internal nodes;
 *   per node: depth (root-level = 1), parent, first child (-1 if none),
 *           child count, FIFO rank (order among internal nodes, -1 for a
 *           leaf), conv inputs for taps 1..3 (node index, or -(1 + r) for
 *           window row r, SSM_TREE_PLAN_UNUSED beyond W-1).
 * An invalid tree yields the status and zeros elsewhere.  Only dims.batch,
 * n_nodes and conv_width are read.
 */
#define SSM_TREE_PLAN_HEADER 4
#define SSM_TREE_PLAN_STRIDE 8
#define SSM_TREE_PLAN_UNUSED (-32768)
int ssm_tree_plan(const ssm_tree_dims* dims, const int32_t* parent, int32_t* plan_out, void* hip_stream);

/* Static text for a status code (never NULL). */
const char* ssm_tree_status_string(int status);

/* SSM_TREE_ABI_VERSION of the loaded library. */
int ssm_tree_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SSM_TREE_H */
