/*
 * oracle.c - plain, slow, float64 CPU oracle (test infrastructure only).
 *
 * Nothing here is blocked, fused or reordered beyond the definition: the
 * tree is walked with a literal FIFO queue of materialised per-node states
 * as in [SM] sec. 3.2, every state is a full [H][P][N] float64 array, and
 * the conv taps are found by following parent links.  See oracle.h for the
 * sources, layouts and readings.
 *
 * ORACLE_MUTANT (compile-time, default 0) plants one deliberate mistake;
 * the test suite builds each mutant separately to show that its pins catch
 * it.  A normal build has ORACLE_MUTANT == 0 and no mutated line.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(k) (ORACLE_MUTANT == (k))

/* softplus with the usual large-argument cut-over ([LM]: Delta is the step
 * size; positivity via softplus is the Mamba2 convention). */
static double softplus(double z) {
  if (MUT(9)) return exp(z);
  return z > 20.0 ? z : log1p(exp(z));
}

static double act(double z, int silu) { return silu ? z / (1.0 + exp(-z)) : z; }

/* [SM] sec. 3.2: the tree is flattened breadth-first.  Valid parent[] arrays
 * are exactly the BFS labellings: parent[0] = -1, -1 <= parent[i] < i, and
 * parent[] non-decreasing (children of one node form a contiguous range that
 * follows the ranges of earlier nodes). */
int oracle_validate_tree(const int32_t* parent, int32_t T) {
  if (T < 0) return ORACLE_E_ARG;
  if (T == 0) return ORACLE_OK;
  if (parent[0] != -1) return ORACLE_E_TREE;
  for (int32_t i = 1; i < T; ++i) {
    if (parent[i] < -1 || parent[i] >= i) return ORACLE_E_TREE;
    if (!MUT(11) && parent[i] < parent[i - 1]) return ORACLE_E_TREE;
  }
  return ORACLE_OK;
}

/* [SM] sec. 3.1: the accepted path runs from a root-level node down parent
 * links; its length is at most the node count. */
int oracle_validate_path(const int32_t* parent, int32_t T, const int32_t* path, int32_t len) {
  int st = oracle_validate_tree(parent, T);
  if (st != ORACLE_OK) return st;
  if (len < 0 || (MUT(20) ? len >= T : len > T)) return ORACLE_E_PATH;
  for (int32_t k = 0; k < len; ++k) {
    int32_t v = path[k];
    if (v < 0 || v >= T) return ORACLE_E_PATH;
    if (MUT(19) && k == 0) continue;
    int32_t want = (k == 0) ? -1 : path[k - 1];
    if (parent[v] != want) return ORACLE_E_PATH;
  }
  return ORACLE_OK;
}

static int32_t node_depth(const int32_t* parent, int32_t v) {
  int32_t d = 0;
  while (v >= 0) {
    ++d;
    v = parent[v];
  }
  return d;
}

/* code of the j-th conv input of node v (j = 1 is its parent): a node index,
 * or -(1 + r) for row r of the committed window (row W-2 is the newest). */
static int32_t anc_code(const int32_t* parent, int32_t v, int32_t j, int32_t W) {
  int32_t u = v;
  int32_t k = 0;
  while (k < j && u >= 0) {
    u = parent[u];
    ++k;
  }
  if (u >= 0) return u;
  /* walked past the tree root after k steps: k - 1 ancestors were tree nodes
   * above v, so the remaining j - (k - 1) - 1 steps go into the window */
  int32_t into = j - k; /* 0 -> newest window row */
  int32_t row = (W - 2) - into;
  if (MUT(8)) row = into;
  return -(1 + row);
}

int oracle_plan(const int32_t* parent, int32_t T, int32_t W, int32_t* plan, int32_t* peak_fifo,
                int32_t* max_depth, int32_t* n_internal) {
  int st = oracle_validate_tree(parent, T);
  if (st != ORACLE_OK) return st;
  if (W < 1 || W > 4) return ORACLE_E_ARG;
  int32_t maxd = 0, nint = 0;
  for (int32_t v = 0; v < T; ++v) {
    int32_t* r = plan + (int64_t)v * ORACLE_PLAN_STRIDE;
    int32_t first = -1, cnt = 0;
    for (int32_t i = 0; i < T; ++i)
      if (parent[i] == v) {
        if (first < 0) first = i;
        ++cnt;
      }
    r[0] = node_depth(parent, v);
    r[1] = parent[v];
    r[2] = first;
    r[3] = cnt;
    r[4] = -1;
    for (int32_t j = 1; j <= 3; ++j) r[4 + j] = (j < W) ? anc_code(parent, v, j, W) : ORACLE_PLAN_UNUSED;
    if (r[0] > maxd) maxd = r[0];
    if (cnt > 0) r[4] = nint++;
  }
  /* FIFO occupancy: internal nodes are pushed in BFS order when their parent
   * is expanded and popped in the same order; count pushed-not-popped. */
  int32_t peak = 0, live = 0;
  for (int32_t pnode = -1; pnode < T; ++pnode) {
    if (pnode >= 0) {
      if (plan[(int64_t)pnode * ORACLE_PLAN_STRIDE + 3] == 0) continue;
      --live; /* pop */
    }
    for (int32_t i = 0; i < T; ++i)
      if (parent[i] == pnode && plan[(int64_t)i * ORACLE_PLAN_STRIDE + 3] > 0) {
        ++live;
        if (live > peak) peak = live;
      }
  }
  if (peak_fifo) *peak_fifo = peak;
  if (max_depth) *max_depth = maxd;
  if (n_internal) *n_internal = nint;
  return ORACLE_OK;
}

/* Conv channels: x only, or x, B and C with the xbc option. */
static int32_t conv_channels(const oracle_dims* d) { return d->H * d->P + (d->xbc ? 2 * d->G * d->N : 0); }

/* Raw (pre-conv) input of conv channel ch at node or token v. */
static double raw_in(const oracle_dims* d, const oracle_unit* u, int32_t v, int32_t ch) {
  const int32_t DI = d->H * d->P, GN = d->G * d->N;
  if (ch < DI) return u->x[(int64_t)v * DI + ch];
  if (ch < DI + GN) return u->B[(int64_t)v * GN + (ch - DI)];
  return u->C[(int64_t)v * GN + (ch - DI - GN)];
}

/* Row of conv weights used for channel ch. */
static int32_t weight_row(const oracle_dims* d, int32_t ch) {
  const int32_t DI = d->H * d->P, GN = d->G * d->N;
  if (MUT(15) && ch >= DI && ch < DI + GN) return ch + GN; /* B convolved with C's weights */
  return ch;
}

/* Causal depthwise conv1d of channel ch at node v over its ancestor path
 * ([LM]: X passes conv1d before the SSM).  Weight W-1 multiplies the node's
 * own input, weight W-1-j its j-th ancestor's (or a window row past the
 * root). */
static double conv_at_node(const oracle_dims* d, const int32_t* parent, const oracle_unit* u, int32_t v,
                           int32_t ch) {
  const int32_t W = d->W, CH = conv_channels(d), wr = weight_row(d, ch);
  double acc = u->conv_b ? u->conv_b[ch] : 0.0;
  for (int32_t j = 0; j < W; ++j) {
    double in;
    if (j == 0) {
      in = raw_in(d, u, v, ch);
    } else {
      int32_t code = anc_code(parent, v, j, W);
      in = code >= 0 ? raw_in(d, u, code, ch) : u->window[(int64_t)(-1 - code) * CH + ch];
    }
    int32_t tap = MUT(3) ? j : (W - 1 - j);
    acc += u->conv_w[(int64_t)wr * W + tap] * in;
  }
  return act(acc, d->silu);
}

/* Output gate: y * silu(z). */
static double gate(double z) { return MUT(16) ? 1.0 / (1.0 + exp(-z)) : z / (1.0 + exp(-z)); }

typedef struct {
  int32_t node;
  double* h; /* [H][P][N] */
} fifo_entry;

/* [SM] sec. 3.2 FIFO_tree_verification, read so that every child is pushed
 * once (after its state is formed) and a node's state is released once all
 * its children are done.  Each child's state is formed from its parent's:
 *   h_c = exp(dt_c A) h_parent + (dt_c x~_c) outer B_c      ([LM] recurrence)
 *   y_c = C_c . h_c + D x~_c                                 ([LM]: SSM emits Y)
 */
int oracle_verify(const oracle_dims* d, const int32_t* parent, const oracle_unit* u, double* y,
                  int32_t* peak_fifo) {
  const int32_t T = d->T, H = d->H, P = d->P, N = d->N, G = d->G, DI = H * P;
  if (T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || d->W < 1 || d->W > 4)
    return ORACLE_E_ARG;
  int st = oracle_validate_tree(parent, T);
  if (peak_fifo) *peak_fifo = 0;
  if (st != ORACLE_OK) {
    for (int64_t i = 0; i < (int64_t)T * DI; ++i) y[i] = NAN;
    return st;
  }
  if (T == 0) return ORACLE_OK;
  const int64_t SZ = (int64_t)H * P * N;
  const int32_t hpg = H / G;

  /* per-node step sizes and the conv outputs, recomputed from raw inputs */
  const int32_t GN = G * N;
  double* dt = (double*)malloc(sizeof(double) * (size_t)T * H);
  double* xt = (double*)malloc(sizeof(double) * (size_t)T * DI);
  double* bt = d->xbc ? (double*)malloc(sizeof(double) * (size_t)T * GN) : NULL;
  double* ct = d->xbc ? (double*)malloc(sizeof(double) * (size_t)T * GN) : NULL;
  for (int32_t v = 0; v < T; ++v) {
    for (int32_t h = 0; h < H; ++h) {
      double z = u->dt_raw[(int64_t)v * H + h] + (MUT(7) ? 0.0 : u->dt_bias[h]);
      dt[(int64_t)v * H + h] = softplus(z);
    }
    for (int32_t c = 0; c < DI; ++c) xt[(int64_t)v * DI + c] = conv_at_node(d, parent, u, v, c);
    if (d->xbc) {
      for (int32_t i = 0; i < GN; ++i) {
        bt[(int64_t)v * GN + i] = conv_at_node(d, parent, u, v, DI + i);
        ct[(int64_t)v * GN + i] = conv_at_node(d, parent, u, v, DI + GN + i);
      }
    }
  }
  const double* Bsrc = d->xbc ? bt : u->B; /* the B and C the recurrence sees */
  const double* Csrc = d->xbc ? ct : u->C;

  fifo_entry* q = (fifo_entry*)malloc(sizeof(fifo_entry) * (size_t)(T + 1));
  int32_t head = 0, tail = 0, peak = 0;
  q[tail++] = (fifo_entry){-1, (double*)u->state}; /* root state, not owned */

  while (head < tail) {
    fifo_entry cur = q[head++];
    for (int32_t c = 0; c < T; ++c) {
      if (parent[c] != cur.node) continue;
      double* hc = (double*)malloc(sizeof(double) * (size_t)SZ);
      int32_t par_x = (cur.node >= 0) ? cur.node : c;
      for (int32_t h = 0; h < H; ++h) {
        const int32_t g = MUT(14) ? (h % G) : (h / hpg);
        const double dtc = dt[(int64_t)c * H + h];
        const double dA = exp((MUT(2) ? -1.0 : 1.0) * dtc * u->A[h]);
        const double* Bc = (MUT(6) ? Csrc : Bsrc) + ((int64_t)c * G + g) * N;
        const double* Cc = (MUT(6) ? Bsrc : Csrc) + ((int64_t)c * G + g) * N;
        for (int32_t p = 0; p < P; ++p) {
          const int32_t ch = h * P + p;
          const double xin = xt[(int64_t)(MUT(4) ? par_x : c) * DI + ch];
          const double coef = dtc * xin;
          const double* hp = cur.h + ((int64_t)h * P + p) * N;
          double* hn = hc + ((int64_t)h * P + p) * N;
          double acc = 0.0;
          for (int32_t n = 0; n < N; ++n) {
            hn[n] = dA * hp[n] + coef * Bc[n];
            acc += Cc[n] * (MUT(5) ? hp[n] : hn[n]);
          }
          y[(int64_t)c * DI + ch] = acc + (MUT(1) ? 0.0 : u->D[h] * xt[(int64_t)c * DI + ch]);
          if (u->z) y[(int64_t)c * DI + ch] *= gate(u->z[(int64_t)c * DI + ch]);
        }
      }
      int has_children = 0;
      for (int32_t i = c + 1; i < T; ++i)
        if (parent[i] == c) {
          has_children = 1;
          break;
        }
      if (has_children) {
        q[tail++] = (fifo_entry){c, hc};
        if (tail - head > peak) peak = tail - head;
      } else {
        free(hc);
      }
    }
    if (cur.node >= 0) free(cur.h); /* release after all children are done */
  }
  if (peak_fifo) *peak_fifo = peak;
  free(q);
  free(ct);
  free(bt);
  free(xt);
  free(dt);
  return ORACLE_OK;
}

/* [SM] sec. 3.1: the accepted path is committed by recomputing the root
 * state along it from the stored per-token dt_raw, B and x (no per-node
 * state is kept).  The window gains each path token's raw conv inputs
 * (x, and B and C with xbc), oldest row dropped; it is a copy of input
 * values. */
int oracle_commit(const oracle_dims* d, const int32_t* parent, const int32_t* path, int32_t len,
                  const oracle_unit* u, double* state_out, double* window_out) {
  const int32_t T = d->T, H = d->H, P = d->P, N = d->N, G = d->G, W = d->W, DI = H * P;
  if (T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || W < 1 || W > 4) return ORACLE_E_ARG;
  int st = oracle_validate_path(parent, T, path, len);
  if (st != ORACLE_OK) return st;
  const int32_t CH = conv_channels(d), GN = G * N;
  const int64_t SZ = (int64_t)H * P * N;
  const int32_t hpg = H / G;
  double* h = (double*)malloc(sizeof(double) * (size_t)SZ);
  double* win = (double*)malloc(sizeof(double) * (size_t)(W > 1 ? W - 1 : 1) * CH);
  double* cv = (double*)malloc(sizeof(double) * (size_t)CH); /* conv outputs of every channel */
  memcpy(h, u->state, sizeof(double) * (size_t)SZ);
  if (W > 1) memcpy(win, u->window, sizeof(double) * (size_t)(W - 1) * CH);
  for (int32_t k = 0; k < len; ++k) {
    const int32_t v = path[k];
    for (int32_t ch = 0; ch < CH; ++ch) {
      const int32_t wr = weight_row(d, ch);
      double acc = u->conv_b ? u->conv_b[ch] : 0.0;
      acc += u->conv_w[(int64_t)wr * W + (W - 1)] * raw_in(d, u, v, ch);
      for (int32_t j = 1; j < W; ++j) acc += u->conv_w[(int64_t)wr * W + (W - 1 - j)] * win[(int64_t)(W - 1 - j) * CH + ch];
      cv[ch] = act(acc, d->silu);
    }
    for (int32_t hh = 0; hh < H; ++hh) {
      const int32_t g = hh / hpg;
      const double dtv = softplus(u->dt_raw[(int64_t)v * H + hh] + u->dt_bias[hh]);
      const double dA = exp(dtv * u->A[hh]);
      const double* Bv = d->xbc ? cv + DI + (int64_t)g * N : u->B + ((int64_t)v * G + g) * N;
      for (int32_t p = 0; p < P; ++p) {
        const double coef = dtv * cv[hh * P + p];
        double* hr = h + ((int64_t)hh * P + p) * N;
        for (int32_t n = 0; n < N; ++n) {
          hr[n] = dA * hr[n] + coef * Bv[n];
          if (MUT(13)) hr[n] *= dA;
        }
      }
    }
    if (W > 1) {
      for (int32_t r = 0; r + 1 < W - 1; ++r) memcpy(win + (int64_t)r * CH, win + (int64_t)(r + 1) * CH, sizeof(double) * CH);
      if (!MUT(10))
        for (int32_t ch = 0; ch < (MUT(17) ? DI : CH); ++ch) win[(int64_t)(W - 2) * CH + ch] = raw_in(d, u, v, ch);
    }
  }
  (void)GN;
  memcpy(state_out, h, sizeof(double) * (size_t)SZ);
  if (W > 1) memcpy(window_out, win, sizeof(double) * (size_t)(W - 1) * CH);
  free(cv);
  free(win);
  free(h);
  return ORACLE_OK;
}

/* Textbook sequential Mamba2 SSM over a plain token sequence of length S
 * (no tree): the causal conv runs over the concatenation (window rows,
 * then the tokens' raw inputs) by index, and the recurrence is applied
 * token by token.  x, B, C, dt_raw, z are indexed by token.  Used as the
 * independent special case a chain tree must reduce to. */
int oracle_scan(const oracle_dims* d, int32_t S, const oracle_unit* u, double* y, double* state_out,
                double* window_out) {
  const int32_t H = d->H, P = d->P, N = d->N, G = d->G, W = d->W, DI = H * P;
  if (S < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || W < 1 || W > 4) return ORACLE_E_ARG;
  const int32_t GN = G * N, CH = DI + (d->xbc ? 2 * GN : 0);
  const int64_t SZ = (int64_t)H * P * N;
  const int32_t hpg = H / G;
  const int32_t L = (W - 1) + S; /* concatenated sequence length */
  double* seq = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * CH);
  if (W > 1) memcpy(seq, u->window, sizeof(double) * (size_t)(W - 1) * CH);
  for (int32_t t = 0; t < S; ++t) {
    double* row = seq + (int64_t)(W - 1 + t) * CH;
    memcpy(row, u->x + (int64_t)t * DI, sizeof(double) * DI);
    if (d->xbc) {
      memcpy(row + DI, u->B + (int64_t)t * GN, sizeof(double) * GN);
      memcpy(row + DI + GN, u->C + (int64_t)t * GN, sizeof(double) * GN);
    }
  }
  double* h = (double*)malloc(sizeof(double) * (size_t)SZ);
  double* bc = (double*)malloc(sizeof(double) * (size_t)(2 * GN)); /* this token's B and C as the SSM sees them */
  memcpy(h, u->state, sizeof(double) * (size_t)SZ);
  for (int32_t t = 0; t < S; ++t) {
    for (int32_t i = 0; i < 2 * GN; ++i) {
      if (!d->xbc) {
        bc[i] = i < GN ? u->B[(int64_t)t * GN + i] : u->C[(int64_t)t * GN + i - GN];
        continue;
      }
      const int32_t c = DI + i;
      double cv = u->conv_b ? u->conv_b[c] : 0.0;
      for (int32_t k = 0; k < W; ++k) cv += u->conv_w[(int64_t)c * W + k] * seq[(int64_t)(t + k) * CH + c];
      bc[i] = d->silu ? cv / (1.0 + exp(-cv)) : cv;
    }
    for (int32_t hh = 0; hh < H; ++hh) {
      const int32_t g = hh / hpg;
      const double z = u->dt_raw[(int64_t)t * H + hh] + u->dt_bias[hh];
      const double dtv = z > 20.0 ? z : log(1.0 + exp(z));
      const double dA = exp(dtv * u->A[hh]);
      for (int32_t p = 0; p < P; ++p) {
        const int32_t c = hh * P + p;
        double cv = u->conv_b ? u->conv_b[c] : 0.0;
        for (int32_t k = 0; k < W; ++k) cv += u->conv_w[(int64_t)c * W + k] * seq[(int64_t)(t + k) * CH + c];
        if (d->silu) cv = cv / (1.0 + exp(-cv));
        double* hr = h + ((int64_t)hh * P + p) * N;
        double acc = 0.0;
        for (int32_t n = 0; n < N; ++n) {
          hr[n] = dA * hr[n] + dtv * cv * bc[g * N + n];
          acc += bc[GN + g * N + n] * hr[n];
        }
        double out = acc + u->D[hh] * cv;
        if (u->z) {
          const double zz = u->z[(int64_t)t * DI + c];
          out *= zz / (1.0 + exp(-zz));
        }
        y[(int64_t)t * DI + c] = out;
      }
    }
  }
  if (state_out) memcpy(state_out, h, sizeof(double) * (size_t)SZ);
  if (window_out && W > 1) memcpy(window_out, seq + (int64_t)S * CH, sizeof(double) * (size_t)(W - 1) * CH);
  free(bc);
  free(h);
  free(seq);
  return ORACLE_OK;
}

/* One value to the bfloat16 grid (see oracle.h).  The grid spacing of x's
 * binade is q = 2^(e - 8) for |x| in [2^(e-1), 2^e) with e - 1 >= -126, and
 * 2^-133 below; x / q is exact in float64, and its integer part k and
 * fraction decide the rounding. */
static double round_bf16_one(double x, double* gap) {
  if (x == 0.0 || isnan(x) || isinf(x)) {
    if (gap) *gap = INFINITY;
    return x;
  }
  const double a = fabs(x);
  int e;
  frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
  const int qe = (e - 1 >= -126) ? e - 8 : -133;
  const double q = ldexp(1.0, qe);
  const double r = a / q;
  const double k = floor(r), f = r - k;
  double kr;
  if (f > 0.5)
    kr = k + 1.0;
  else if (f < 0.5)
    kr = k;
  else /* a tie: the even significand (k even) */
    kr = (MUT(18) ? 1.0 : (fmod(k, 2.0) == 0.0 ? 0.0 : 1.0)) + k;
  double v = kr * q;
  if (v > 255.0 * ldexp(1.0, 120)) v = INFINITY;
  if (gap) {
    /* the nearest boundary is k + 1/2, or, at the bottom of a binade whose
     * lower neighbour is twice as fine, the midpoint k - 1/4 below it */
    double g = fabs(f - 0.5);
    if (k == 128.0 && e - 1 > -126 && f + 0.25 < g) g = f + 0.25;
    *gap = g * q / a;
  }
  return x < 0 ? -v : v;
}

void oracle_round_bf16(const double* x, double* out, double* gap, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16_one(x[i], gap ? gap + i : NULL);
}
