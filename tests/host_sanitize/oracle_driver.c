/* Host sanitizer driver for the oracle: oracle.c is compiled into this file's
 * translation unit with AddressSanitizer and UndefinedBehaviorSanitizer (no
 * OpenMP: the pragmas are ignored), and every entry point runs on small
 * seeded inputs that reach its edge cases -- first groups with missing
 * slots, incomplete groups, nothing visible, k above the visible count,
 * padded and out-of-range top-k entries, ring and linear windows, windows
 * longer than the context, a -inf sink, fp32, bf16 and fp64 element types.
 * A memory or undefined-behaviour error aborts the process; the values are
 * checked by the pins, not here (only finiteness where it must hold). */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) { /* splitmix64 -> [-1, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}

/* n values of element type dt, freshly allocated (exact sizes, so ASan sees
 * any read past the end) */
static void* alloc_vals(int dt, size_t n) {
  void* p = malloc(n * esize(dt) + (n == 0));
  for (size_t i = 0; i < n; ++i) {
    double v = rnd();
    if (dt == ORC_F64) ((double*)p)[i] = v;
    else if (dt == ORC_F32) ((float*)p)[i] = (float)v;
    else {
      float f = (float)v;
      uint32_t u;
      memcpy(&u, &f, 4);
      ((uint16_t*)p)[i] = (uint16_t)(u >> 16);
    }
  }
  return p;
}

static int check_finite(const double* x, size_t n, const char* what) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) {
      fprintf(stderr, "%s: non-finite value at %zu\n", what, i);
      return 1;
    }
  return 0;
}

static int run_compress(int dt, int B, int L, int d, int rope, int ratio, int overlap, int N_cap, long p0_base) {
  int m = overlap ? 2 : 1;
  void* kv = alloc_vals(dt, (size_t)B * L * m * d);
  void* sc = alloc_vals(dt, (size_t)B * L * m * d);
  double* gamma = (double*)malloc(sizeof(double) * d);
  for (int i = 0; i < d; ++i) gamma[i] = 1.0 + 0.1 * rnd();
  double* cache = (double*)calloc((size_t)B * N_cap * d, sizeof(double));
  uint8_t* written = (uint8_t*)calloc((size_t)B * N_cap, 1);
  int32_t* pos0 = (int32_t*)malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) pos0[b] = (int32_t)(p0_base + b * 3);
  long n = orc_compress(kv, sc, dt, gamma, cache, written, pos0, B, L, d, rope, ratio, overlap, N_cap, 1e-6, 10000.0);
  int bad = check_finite(cache, (size_t)B * N_cap * d, "compress");
  double* pooled = (double*)malloc(sizeof(double) * d);
  for (long g = p0_base / ratio - 1; g <= (p0_base + L) / ratio + 1; ++g)
    orc_pool(kv, sc, dt, L, d, ratio, overlap, p0_base, g, pooled); /* -1 for groups outside: fine */
  if (overlap && p0_base == 0) {
    double* c2 = (double*)calloc((size_t)B * N_cap * d, sizeof(double));
    orc_compress_rolling(kv, sc, dt, gamma, c2, B, L, d, rope, ratio, N_cap, 1e-6, 10000.0);
    free(c2);
  }
  free(kv), free(sc), free(gamma), free(cache), free(written), free(pos0), free(pooled);
  printf("compress dt=%d B=%d L=%d d=%d ratio=%d overlap=%d: %ld entries\n", dt, B, L, d, ratio, overlap, n);
  return bad;
}

static int run_index_topk(int dt, int B, int S, int Hi, int di, int N_cap, int ratio, int k, long t0) {
  void* q = alloc_vals(dt, (size_t)B * S * Hi * di);
  void* kc = alloc_vals(dt, (size_t)B * N_cap * di);
  double* w = (double*)malloc(sizeof(double) * B * S * Hi);
  for (int i = 0; i < B * S * Hi; ++i) w[i] = rnd();
  int32_t* q_pos = (int32_t*)malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) q_pos[b] = (int32_t)(t0 + 5 * b);
  double* scores = (double*)malloc(sizeof(double) * B * S * N_cap);
  int32_t* nvis = (int32_t*)malloc(sizeof(int32_t) * B * S);
  orc_index_scores(q, dt, w, kc, dt, q_pos, B, S, Hi, di, N_cap, ratio, 0u, scores, nvis);
  orc_index_scores(q, dt, w, kc, dt, q_pos, B, S, Hi, di, N_cap, ratio, ORC_NO_RELU, scores, nvis);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * B * S * k);
  double* kth = (double*)malloc(sizeof(double) * B * S);
  orc_topk(scores, nvis, B, S, N_cap, k, idx, kth);
  int bad = 0;
  for (int i = 0; i < B * S * k; ++i)
    if (idx[i] < -1 || idx[i] >= N_cap) bad = 1;
  free(q), free(kc), free(w), free(q_pos), free(scores), free(nvis), free(idx), free(kth);
  printf("index+topk dt=%d B=%d S=%d N_cap=%d k=%d t0=%ld\n", dt, B, S, N_cap, k, t0);
  return bad;
}

static int run_attn(int dt, int B, int S, int H, int D, int rope, int N_cap, int k, int W_cap, int window,
                    int linear, int sink_inf, long t0) {
  void* q = alloc_vals(dt, (size_t)B * S * H * D);
  void* cmp = alloc_vals(dt, (size_t)B * N_cap * D);
  void* win = alloc_vals(dt, (size_t)B * W_cap * D);
  double* sink = (double*)malloc(sizeof(double) * H);
  for (int h = 0; h < H; ++h) sink[h] = sink_inf ? -INFINITY : rnd();
  int32_t* q_pos = (int32_t*)malloc(sizeof(int32_t) * B);
  int32_t* wp0 = (int32_t*)malloc(sizeof(int32_t) * B);
  for (int b = 0; b < B; ++b) {
    q_pos[b] = (int32_t)(t0 + 7 * b);
    wp0[b] = q_pos[b] - (W_cap - S);
  }
  int32_t* topk = (int32_t*)malloc(sizeof(int32_t) * ((size_t)B * S * k + 1));
  for (int i = 0; i < B * S * k; ++i) {
    double r = rnd();
    topk[i] = r < -0.8 ? -1 : r > 0.9 ? N_cap + 3 : (int32_t)((r + 1.0) * 0.5 * N_cap); /* padding, out of range */
  }
  double* out = (double*)malloc(sizeof(double) * B * S * H * D);
  double* lse = (double*)malloc(sizeof(double) * B * S * H);
  int32_t* ncand = (int32_t*)malloc(sizeof(int32_t) * B * S);
  int rc1 = orc_attn(q, dt, cmp, dt, topk, k, 4, win, dt, linear ? wp0 : NULL, sink, q_pos, out, lse, ncand, B, S, H,
                     D, rope, N_cap, W_cap, window, 1.0 / sqrt((double)D), 10000.0);
  int bad = rc1 != 0 || check_finite(out, (size_t)B * S * H * D, "attn (sparse)");
  int rc2 = orc_attn(q, dt, cmp, dt, NULL, 0, 4, win, dt, linear ? wp0 : NULL, sink, q_pos, out, lse, ncand, B, S, H,
                     D, rope, N_cap, W_cap, window, 1.0 / sqrt((double)D), 10000.0);
  bad |= rc2 != 0 || check_finite(out, (size_t)B * S * H * D, "attn (dense)");
  free(q), free(cmp), free(win), free(sink), free(q_pos), free(wp0), free(topk), free(out), free(lse), free(ncand);
  printf("attn dt=%d B=%d S=%d H=%d D=%d N_cap=%d k=%d W_cap=%d window=%d linear=%d sink_inf=%d t0=%ld\n", dt, B, S,
         H, D, N_cap, k, W_cap, window, linear, sink_inf, t0);
  return bad;
}

int main(void) {
  int bad = 0;
  double v[8];
  for (int i = 0; i < 8; ++i) v[i] = rnd();
  orc_rope(v, 8, 12345.0, 10000.0, 1);
  orc_rope(v, 8, 12345.0, 10000.0, -1);
  const int dts[3] = {ORC_F32, ORC_BF16, ORC_F64};
  for (int t = 0; t < 3; ++t) {
    int dt = dts[t];
    bad |= run_compress(dt, 2, 8, 64, 16, 4, 1, 16, 0);      /* first groups: entry 0 has no previous group */
    bad |= run_compress(dt, 3, 8, 64, 16, 4, 1, 16, 29);     /* unaligned buffers, incomplete groups */
    bad |= run_compress(dt, 2, 39, 32, 8, 4, 1, 64, 128);    /* a chunk of several entries */
    bad |= run_compress(dt, 2, 300, 16, 4, 128, 0, 8, 70);   /* C128A */
    bad |= run_compress(dt, 1, 8, 64, 16, 4, 1, 2, 4000);    /* entries past N_cap */
    bad |= run_index_topk(dt, 2, 3, 4, 32, 50, 4, 16, 0);    /* nothing visible at t = 0..2 */
    bad |= run_index_topk(dt, 3, 1, 2, 32, 200, 4, 64, 90);  /* visible < k */
    bad |= run_index_topk(dt, 1, 2, 4, 16, 40, 4, 8, 900);   /* visible capped at N_cap */
    bad |= run_attn(dt, 2, 1, 4, 64, 16, 30, 8, 16, 16, 0, 0, 3);      /* window longer than the context */
    bad |= run_attn(dt, 2, 3, 4, 64, 16, 30, 8, 18, 16, 1, 1, 100);    /* linear window, -inf sink */
    bad |= run_attn(dt, 1, 1, 2, 32, 0, 5, 12, 8, 8, 0, 0, 400);       /* k above N_cap, no RoPE */
  }
  if (bad) {
    fprintf(stderr, "oracle driver: a check failed\n");
    return 1;
  }
  printf("oracle driver: ok\n");
  return 0;
}
