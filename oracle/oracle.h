/*
 * oracle.h - plain float64 CPU oracle for tree verification through
 * Mamba2 selective-SSM layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be used by
 * the product path.
 *
 * Sources (the web pages this method is described on):
 *   [SM]  "FPGA加速Mamba推理：SpecMamba方案与优化实践" (jsqmd.com/news/939380)
 *         sec. 2.1 hidden-state backtracking, sec. 3.1 memory-aware hybrid
 *         backtracking, sec. 3.2 FIFO-based tree verification (its
 *         FIFO_tree_verification pseudocode), sec. 5.2 tree parameters.
 *   [LM]  LightMamba part of "FPGA accelerator part 2"
 *         (pinghaoyang.com.cn/aigc/posts/fpga-accelerator-part-2/),
 *         "why Mamba is hard to accelerate" (Mamba block: in_proj makes
 *         X, B, C, Delta, Z; X passes conv1d, then the SSM keeps h_t and
 *         emits Y) and the rotation paragraph whose inline fragments give
 *         the recurrence h_t = Abar (.) h_{t-1} + Bbar (.) X_t.
 *
 * Readings where the pages are silent (each listed in the design notes):
 * conv over x only (over x, B and C with the xbc option, the Mamba2
 * convention), identity activation unless the SiLU flag is set, taps
 * in causal-conv1d order (weight W-1 multiplies the current token), the
 * SSM consumes the post-conv x, dt = softplus(dt_raw + dt_bias) with
 * softplus(z) = z for z > 20, dA = exp(dt * A), group of head h is
 * h / (H / G), parent -1 means "child of the root state".  The optional gate
 * multiplies y by silu(z) ([LM] "why Mamba is hard to accelerate": Y is
 * multiplied elementwise with Z).
 *
 * Layouts (row-major, one (layer, sequence) unit), with CH = H*P conv
 * channels, or H*P + 2*G*N with xbc (channel order: x, then B as [G][N],
 * then C as [G][N]):
 *   x [T][H*P], B and C [T][G][N], dt_raw [T][H], z [T][H*P] or NULL,
 *   window [W-1][CH] (raw inputs of the last W-1 tokens, oldest row first),
 *   state [H][P][N], y [T][H][P];
 *   A, D, dt_bias [H]; conv_w [CH][W]; conv_b [CH] or NULL.
 */
#ifndef SSM_ORACLE_H
#define SSM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_E_ARG (-3)
#define ORACLE_E_TREE (-10)
#define ORACLE_E_PATH (-11)

/* per-node plan record: depth, parent, first_child, n_children, fifo_rank,
 * then conv ancestor codes for taps 1..3 (node index >= 0, window row r as
 * -(1 + r), unused tap -32768) */
#define ORACLE_PLAN_STRIDE 8
#define ORACLE_PLAN_UNUSED (-32768)

typedef struct {
  int32_t T, H, P, N, G, W, silu, xbc;
} oracle_dims;

typedef struct {
  const double *x, *B, *C, *dt_raw, *window, *state;
  const double *A, *D, *dt_bias, *conv_w, *conv_b;
  const double* z; /* gate input [T][H*P], or NULL for no gate */
} oracle_unit;

int oracle_validate_tree(const int32_t* parent, int32_t T);
int oracle_validate_path(const int32_t* parent, int32_t T, const int32_t* path, int32_t len);
int oracle_plan(const int32_t* parent, int32_t T, int32_t W, int32_t* plan, int32_t* peak_fifo,
                int32_t* max_depth, int32_t* n_internal);
int oracle_verify(const oracle_dims* d, const int32_t* parent, const oracle_unit* u, double* y,
                  int32_t* peak_fifo);
int oracle_commit(const oracle_dims* d, const int32_t* parent, const int32_t* path, int32_t len,
                  const oracle_unit* u, double* state_out, double* window_out);
int oracle_scan(const oracle_dims* d, int32_t S, const oracle_unit* u, double* y, double* state_out,
                double* window_out);

/* Storage of a committed root state in bfloat16 ([SM] names mixed precision
 * among its memory optimisations; the format is a reading).  Each value is
 * rounded to the bfloat16 grid: 8 significant bits, float32's exponent
 * range with its subnormals (spacing 2^-133 below 2^-126), nearest value,
 * ties to the even significand, infinite beyond the largest finite value
 * (255 * 2^120); zeros, infinities and NaNs pass through.  gap (may be
 * NULL) receives, per value, the distance from x to the nearest rounding
 * boundary (a midpoint between grid values) divided by |x|, or +inf where
 * there is none (zero, inf, NaN). */
void oracle_round_bf16(const double* x, double* out, double* gap, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
