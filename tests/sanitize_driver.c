/*
 * sanitize_driver.c - runs the host C of this repository (the float64
 * oracle and the seeded input generator) under AddressSanitizer and
 * UndefinedBehaviorSanitizer, built with gcc on the CPU by
 * tests/test_sanitizers.py.  It exercises every entry point on random
 * forests, chains and stars of 0..64 nodes, on valid and invalid trees and
 * paths (out-of-range ids, broken links, over-long lengths), all widths and
 * the options, and the generator's single- and multi-threaded fills.  The
 * sanitizers abort on an out-of-bounds access, a leak or undefined
 * behaviour; the driver itself only checks statuses it can predict.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.h"

int tg_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset, int dist, double a,
                double b, int nthreads);
int tg_fill_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset, int dist, double a,
                 double b, int nthreads);
void tg_raw_bits(uint64_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t offset);
uint16_t tg_f32_to_bf16(float f);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 11);
}
static double rndu(void) { return (rnd() + 0.5) / 2097152.0 / 1024.0 - 1.0; }

static double* vec(int64_t n, double scale) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) p[i] = scale * rndu();
  return p;
}

/* a BFS labelling: 0 = random forest, 1 = chain, 2 = star */
static void tree(int32_t* parent, int T, int kind) {
  for (int i = 0; i < T; ++i) {
    if (i == 0) parent[i] = -1;
    else if (kind == 1) parent[i] = i - 1;
    else if (kind == 2) parent[i] = 0;
    else {
      int lo = parent[i - 1];
      parent[i] = lo + (int)(rnd() % (uint32_t)(i - lo));
    }
  }
}

static int run_unit(int T, int H, int P, int N, int G, int W, int silu, int xbc, int gate, int kind) {
  oracle_dims d = {T, H, P, N, G, W, silu, xbc};
  const int64_t di = (int64_t)H * P, ch = di + (xbc ? 2 * (int64_t)G * N : 0);
  double *x = vec((int64_t)T * di, 1.0), *B = vec((int64_t)T * G * N, 1.0), *C = vec((int64_t)T * G * N, 1.0);
  double *dt = vec((int64_t)T * H, 2.0), *win = vec((W - 1) * ch, 1.0), *st = vec(di * N, 0.5);
  double *A = vec(H, 1.0), *D = vec(H, 1.0), *bias = vec(H, 1.0), *cw = vec(ch * W, 0.5), *cb = vec(ch, 0.5);
  double* z = gate ? vec((int64_t)T * di, 2.0) : NULL;
  for (int h = 0; h < H; ++h) A[h] = -1.0 - fabs(A[h]) * 15.0;
  oracle_unit u = {x, B, C, dt, win, st, A, D, bias, cw, (kind & 1) ? cb : NULL, z};
  int32_t* parent = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* path = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T + 2));
  double* y = (double*)malloc(sizeof(double) * (size_t)((int64_t)T * di + 1));
  double* so = (double*)malloc(sizeof(double) * (size_t)(di * N));
  double* wo = (double*)malloc(sizeof(double) * (size_t)((W - 1) * ch + 1));
  int32_t* plan = (int32_t*)malloc(sizeof(int32_t) * (size_t)((T > 0 ? T : 1) * ORACLE_PLAN_STRIDE));
  int bad = 0;
  tree(parent, T, kind % 3);
  int32_t peak = 0, maxd = 0, nint = 0;
  if (oracle_validate_tree(parent, T) != ORACLE_OK) bad |= 1;
  if (oracle_plan(parent, T, W, plan, &peak, &maxd, &nint) != ORACLE_OK) bad |= 2;
  if (oracle_verify(&d, parent, &u, y, &peak) != ORACLE_OK) bad |= 4;
  /* a root path of a random node, then broken variants */
  int len = 0;
  if (T > 0) {
    int v = (int)(rnd() % (uint32_t)T), tmp[64];
    for (int w = v; w >= 0; w = parent[w]) tmp[len++] = w;
    for (int k = 0; k < len; ++k) path[k] = tmp[len - 1 - k];
  }
  if (oracle_commit(&d, parent, path, len, &u, so, wo) != ORACLE_OK) bad |= 8;
  if (oracle_scan(&d, T, &u, y, so, wo) != ORACLE_OK) bad |= 16;
  if (T > 0) {
    path[0] = T;  /* out of range */
    if (oracle_commit(&d, parent, path, 1, &u, so, wo) != ORACLE_E_PATH) bad |= 32;
    path[0] = -5;
    if (oracle_validate_path(parent, T, path, 1) != ORACLE_E_PATH) bad |= 64;
    for (int k = 0; k < T + 1; ++k) path[k] = k;  /* one entry too many */
    if (oracle_validate_path(parent, T, path, T + 1) != ORACLE_E_PATH) bad |= 128;
  }
  if (T > 1) {
    parent[1] = 5 + T;  /* invalid tree */
    if (oracle_verify(&d, parent, &u, y, &peak) != ORACLE_E_TREE) bad |= 256;
    if (oracle_plan(parent, T, W, plan, &peak, &maxd, &nint) != ORACLE_E_TREE) bad |= 512;
  }
  free(x); free(B); free(C); free(dt); free(win); free(st); free(A); free(D); free(bias); free(cw); free(cb);
  free(z); free(parent); free(path); free(y); free(so); free(wo); free(plan);
  return bad;
}

int main(void) {
  int fails = 0;
  static const int shapes[][6] = {{4, 16, 16, 1, 4, 0}, {2, 16, 32, 2, 3, 1}, {3, 8, 16, 3, 1, 0}, {4, 16, 64, 2, 2, 1}};
  for (int s = 0; s < 4; ++s)
    for (int T = 0; T <= 64; T += (T < 10 ? 1 : 9))
      for (int kind = 0; kind < 6; ++kind) {
        const int* p = shapes[s];
        const int r = run_unit(T, p[0], p[1], p[2], p[3], p[4], p[5], (kind + s) & 1, kind == 4, kind);
        if (r) {
          fprintf(stderr, "shape %d T %d kind %d: status mask %d\n", s, T, kind, r);
          ++fails;
        }
      }
  /* bf16 storage rounding over special and random values */
  double xs[64], out[64], gap[64];
  for (int i = 0; i < 64; ++i) xs[i] = ldexp(rndu(), (int)(rnd() % 300) - 150);
  xs[0] = 0.0; xs[1] = -0.0; xs[2] = INFINITY; xs[3] = -INFINITY; xs[4] = NAN; xs[5] = 3.4e38; xs[6] = 1e-45;
  oracle_round_bf16(xs, out, gap, 64);
  oracle_round_bf16(xs, out, NULL, 64);
  /* the generator: single- and multi-threaded fills, offsets, raw bits */
  const int64_t n = 200000;
  float* f = (float*)malloc(sizeof(float) * (size_t)n);
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)n);
  uint64_t* r = (uint64_t*)malloc(sizeof(uint64_t) * 1000);
  for (int dist = 0; dist < 3; ++dist) {
    tg_fill_f32(f, n, 0x55D00000ull, 3, 17, dist, 0.0, 1.0, 1);
    tg_fill_f32(f, n, 0x55D00000ull, 3, 17, dist, 0.0, 1.0, 8);
    tg_fill_bf16(h, n, 0x55D00003ull, 5, 0, dist, -4.0, -2.0, 8);
    tg_fill_bf16(h, 7, 0x55D00003ull, 5, 1 << 20, dist, -4.0, -2.0, 8);
  }
  tg_raw_bits(r, 1000, 1, 2, 3);
  if (tg_f32_to_bf16(1.0f) != 0x3F80) ++fails;
  free(f); free(h); free(r);
  printf("sanitize driver: %d failing cases\n", fails);
  return fails ? 1 : 0;
}
