/*
 * oracle.c -- plain, slow, fp64 CPU definition of the DeepSeek-V4 compressed
 * attention path (token-level compressors, indexer + top-k, sparse MQA with a
 * learned sink and inverse RoPE).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP kernels against an
 * independent definition.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Sources (page titles as published):
 *   [P1] "DeepSeek-V4-Pro 架构：一个 token 的旅程" (hs-black.github.io)
 *        sections "局部和压缩记忆，共用一次归一化" (shared candidate set, sink),
 *        "输出投影也分组…" (inverse RoPE on o), "压缩是逐通道的 learned pooling"
 *        (per-channel softmax pooling, RMSNorm, RoPE on the tail dims),
 *        "一个通道，逐项算出压缩结果" (missing slots: gate -inf, weight 0),
 *        "压缩条目必须等整组完成后才可见" (visibility rule),
 *        "少读 KV 之前，Indexer 仍要给历史打分" (indexer heads, signed weights).
 *   [P5] "图解DeepSeek V4：详细计算流程解析" (jsqmd.com) sections 2 (window +
 *        compressed channels, <= window+topK reads), 2.1 C4A (overlapping
 *        2*ratio state, pre/cur halves, concat then roll), 2.2 Index,
 *        2.3 (sink, MQA, inverse RoPE), 3 HCA / C128A (non-overlapping).
 *
 * Every floating-point operation is done in double.  Inputs may be given as
 * fp32, bf16 (raw 16-bit patterns) or fp64 and are widened exactly.
 *
 * Readings of points the pages leave open (each is an argument or a fixed
 * convention here, never a hidden constant):
 *   - RoPE rotates interleaved pairs (2i, 2i+1) of the last rope_dim dims by
 *     theta_i = pos * base^(-2i/rope_dim); inverse RoPE rotates by -theta_i.
 *   - A compressed entry g is rotated at position g*ratio (its first token).
 *   - The index score of a (query, entry) pair is sum_h w_h * ReLU(q_h . k);
 *     flag ORC_NO_RELU selects the plain linear form instead.
 *   - Top-k keeps the min(k, visible) largest scores, ties to the lower entry
 *     index, remaining slots padded with -1.
 *   - The window of query position t is positions [max(0, t-window+1), t];
 *     window rows and compressed entries form one candidate set; the same row
 *     serves as key and value.
 *
 * Pins (CPU tests): every function below is checked against closed forms,
 * invariants, library routines, brute force or the worked value printed in
 * [P1], for fp32/fp64 inputs and for bf16 inputs (known bit patterns widen to
 * their IEEE values; bf16-coded inputs give the same results as the same
 * values in fp64), and a mutation run plants mistakes in copies of this file
 * and checks that a pin fails for each.  Parity unpinned: only the
 * model-fidelity constants listed above, which are readings of the pages,
 * not values the pages fix.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2

#define ORC_NO_RELU 1u

/* ---- exact widening of the input element types ------------------------ */
static double ld(const void* p, int dt, size_t i) {
  if (dt == ORC_F64) return ((const double*)p)[i];
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  /* bf16: the 16 high bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t esize(int dt) { return dt == ORC_F64 ? 8 : dt == ORC_F32 ? 4 : 2; }

/* ---- RoPE ([P1] low-rank Q section; pooling section) ------------------ */
/* Rotate x[0..rope_dim) (the tail of a vector) for position pos.
 * sign = +1 applies RoPE, sign = -1 applies the inverse rotation. */
void orc_rope(double* x, int rope_dim, double pos, double base, int sign) {
  for (int i = 0; i < rope_dim / 2; ++i) {
    double theta = pos * pow(base, -2.0 * (double)i / (double)rope_dim);
    double c = cos(sign * theta), s = sin(sign * theta);
    double a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * c - b * s;
    x[2 * i + 1] = a * s + b * c;
  }
}

/* ---- RMSNorm (gamma only, no bias) ------------------------------------ */
static void rms_norm(double* y, int d, const double* gamma, double eps) {
  double ss = 0.0;
  for (int c = 0; c < d; ++c) ss += y[c] * y[c];
  double inv = 1.0 / sqrt(ss / d + eps);
  for (int c = 0; c < d; ++c) y[c] = y[c] * inv * gamma[c];
}

/* ---- pooling of one compressed entry, before normalisation -------------
 * [P1] pooling section: softmax along the token axis, separately for every
 * channel.  [P5] 2.1: with overlap, the 2*ratio slots of entry g are the
 * previous group's tokens read from the first half of the state channels
 * ([0,d)) followed by the group's own tokens read from the second half
 * ([d,2d)).  [P1] worked example: when there is no previous group (g == 0)
 * those slots carry gate -inf and weight 0.  Without overlap (C128A, [P5]
 * 3.1) the slots are the group's own ratio tokens over a d-wide state.
 *
 * kv, sc: state rows of one sequence, [L, m*d] with m = overlap ? 2 : 1;
 * row r holds absolute token pos0 + r.  Returns 0, or -1 if a needed token
 * is outside the buffer. */
int orc_pool(const void* kv, const void* sc, int dt, int L, int d, int ratio, int overlap, long pos0, long g,
             double* pooled) {
  int m = overlap ? 2 : 1;
  int nslot = overlap ? 2 * ratio : ratio;
  double* s = (double*)malloc(sizeof(double) * nslot);
  double* v = (double*)malloc(sizeof(double) * nslot);
  int rc = 0;
  for (int c = 0; c < d && rc == 0; ++c) {
    for (int j = 0; j < nslot; ++j) {
      long tok;
      int ch;
      if (overlap && j < ratio) {
        tok = (g - 1) * ratio + j; /* previous group, first-half channels */
        ch = c;
      } else {
        tok = g * ratio + (overlap ? j - ratio : j); /* own group */
        ch = overlap ? d + c : c;
      }
      if (overlap && j < ratio && g == 0) {
        s[j] = -INFINITY; /* missing slot: gate -inf */
        v[j] = 0.0;
        continue;
      }
      long row = tok - pos0;
      if (row < 0 || row >= L) {
        rc = -1;
        break;
      }
      s[j] = ld(sc, dt, (size_t)row * m * d + ch);
      v[j] = ld(kv, dt, (size_t)row * m * d + ch);
    }
    if (rc) break;
    double mx = -INFINITY;
    for (int j = 0; j < nslot; ++j)
      if (s[j] > mx) mx = s[j];
    double den = 0.0, num = 0.0;
    for (int j = 0; j < nslot; ++j) {
      double e = exp(s[j] - mx); /* exp(-inf) == 0: weight 0 */
      den += e;
      num += e * v[j];
    }
    pooled[c] = num / den;
  }
  free(s);
  free(v);
  return rc;
}

/* ---- compressor: parallel form ----------------------------------------
 * [P1] visibility section: entry g exists once token g*ratio+ratio-1 has
 * arrived; [P1] pooling section: pool, RMSNorm, RoPE on the last rope_dim
 * dims.  Entry g is written iff all tokens it needs lie in the buffer.
 * kv_state, score_state: [B, L, m*d]; pos0: [B] absolute position of row 0;
 * cache: [B, N_cap, d] fp64 (only written rows change); written: [B, N_cap]
 * flags (nullable).  Returns the number of entries written. */
long orc_compress(const void* kv_state, const void* score_state, int dt, const double* gamma, double* cache,
                  uint8_t* written, const int32_t* pos0, int B, int L, int d, int rope_dim, int ratio, int overlap,
                  int N_cap, double eps, double rope_base) {
  int m = overlap ? 2 : 1;
  long count = 0;
  double* y = (double*)malloc(sizeof(double) * d);
  for (int b = 0; b < B; ++b) {
    long p0 = pos0[b];
    for (long g = 0; g < N_cap; ++g) {
      long first = g * ratio, last = g * ratio + ratio - 1;
      if (first < p0 || last > p0 + L - 1) continue;
      if (overlap && g > 0 && (g - 1) * ratio < p0) continue; /* previous group not in buffer */
      const size_t off = (size_t)b * L * m * d;
      if (orc_pool((const char*)kv_state + off * esize(dt), (const char*)score_state + off * esize(dt), dt, L, d,
                   ratio, overlap, p0, g, y) != 0)
        continue;
      rms_norm(y, d, gamma, eps);
      orc_rope(y + (d - rope_dim), rope_dim, (double)(g * ratio), rope_base, +1);
      memcpy(cache + ((size_t)b * N_cap + g) * d, y, sizeof(double) * d);
      if (written) written[(size_t)b * N_cap + g] = 1;
      ++count;
    }
  }
  free(y);
  return count;
}

/* ---- compressor: the rolling-state form of [P5] 2.1, token by token ----
 * State [2*ratio, 2*d]: rows [0,ratio) are "pre", rows [ratio,2*ratio) are
 * "cur".  A new token's projections go to cur row (t mod ratio).  When the
 * group completes, the 2*ratio x d operand is pre's first-half channels
 * stacked over cur's second-half channels, pooled per channel; then cur is
 * copied over pre.  Before the first completion pre holds -inf scores.
 * Sequence b's tokens start at position 0 (pos0 must be 0 here).
 * Entries go to cache [B, N_cap, d] like orc_compress. Returns entries written. */
long orc_compress_rolling(const void* kv_state, const void* score_state, int dt, const double* gamma, double* cache,
                          int B, int L, int d, int rope_dim, int ratio, int N_cap, double eps, double rope_base) {
  long count = 0;
  size_t W = (size_t)2 * d;
  double* kvs = (double*)malloc(sizeof(double) * 2 * ratio * W);
  double* scs = (double*)malloc(sizeof(double) * 2 * ratio * W);
  double* y = (double*)malloc(sizeof(double) * d);
  for (int b = 0; b < B; ++b) {
    for (size_t i = 0; i < 2 * ratio * W; ++i) {
      kvs[i] = 0.0;
      scs[i] = -INFINITY;
    }
    for (long t = 0; t < L; ++t) {
      int slot = ratio + (int)(t % ratio);
      for (size_t c = 0; c < W; ++c) {
        size_t src = ((size_t)b * L + t) * W + c;
        kvs[slot * W + c] = ld(kv_state, dt, src);
        scs[slot * W + c] = ld(score_state, dt, src);
      }
      if ((t + 1) % ratio != 0) continue;
      long g = t / ratio;
      for (int c = 0; c < d; ++c) {
        /* concat([state[:ratio, :d], state[ratio:, d:]]) along the token axis */
        double mx = -INFINITY;
        for (int j = 0; j < 2 * ratio; ++j) {
          size_t idx = (size_t)j * W + (j < ratio ? c : d + c);
          if (scs[idx] > mx) mx = scs[idx];
        }
        double den = 0.0, num = 0.0;
        for (int j = 0; j < 2 * ratio; ++j) {
          size_t idx = (size_t)j * W + (j < ratio ? c : d + c);
          double e = exp(scs[idx] - mx);
          den += e;
          num += e * kvs[idx];
        }
        y[c] = num / den;
      }
      rms_norm(y, d, gamma, eps);
      orc_rope(y + (d - rope_dim), rope_dim, (double)(g * ratio), rope_base, +1);
      if (g < N_cap) {
        memcpy(cache + ((size_t)b * N_cap + g) * d, y, sizeof(double) * d);
        ++count;
      }
      /* roll: cur overwrites pre */
      memcpy(kvs, kvs + (size_t)ratio * W, sizeof(double) * ratio * W);
      memcpy(scs, scs + (size_t)ratio * W, sizeof(double) * ratio * W);
    }
  }
  free(kvs);
  free(scs);
  free(y);
  return count;
}

/* ---- indexer scores ----------------------------------------------------
 * [P1] indexer section: 64 heads over one shared compressed index cache,
 * signed per-head weights w (already scaled).  [P1] visibility: only entries
 * s < (t+1)/ratio exist for query position t.  scores: [B, S, N_cap]; entries
 * at or past the visible count are set to -inf.  nvis: [B, S]. */
void orc_index_scores(const void* q_idx, int qdt, const double* w, const void* idx_cache, int kdt,
                      const int32_t* q_pos, int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags,
                      double* scores, int32_t* nvis) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      long t = (long)q_pos[b] + s;
      long nv = (t + 1) / ratio;
      if (nv > N_cap) nv = N_cap;
      nvis[(size_t)b * S + s] = (int32_t)nv;
      double* out = scores + ((size_t)b * S + s) * N_cap;
      for (long e = 0; e < N_cap; ++e) {
        if (e >= nv) {
          out[e] = -INFINITY;
          continue;
        }
        double acc = 0.0;
        for (int h = 0; h < Hi; ++h) {
          double dot = 0.0;
          for (int c = 0; c < di; ++c)
            dot += ld(q_idx, qdt, (((size_t)b * S + s) * Hi + h) * di + c) *
                   ld(idx_cache, kdt, ((size_t)b * N_cap + e) * di + c);
          double f = (flags & ORC_NO_RELU) ? dot : (dot > 0.0 ? dot : 0.0);
          acc += w[((size_t)b * S + s) * Hi + h] * f;
        }
        out[e] = acc;
      }
    }
}

/* ---- top-k -------------------------------------------------------------
 * [P5] section 2: the index module keeps at most topK compressed entries.
 * Keeps the min(k, nvis) largest scores (ties: lower entry first), in
 * descending score order, then pads with -1.  kth: [B,S] score of the last
 * kept entry (NaN when none), nullable. */
typedef struct {
  double v;
  int32_t i;
} orc_pair;

static int cmp_pair(const void* a, const void* b) {
  const orc_pair* x = (const orc_pair*)a;
  const orc_pair* y = (const orc_pair*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->i > y->i) - (x->i < y->i);
}

void orc_topk(const double* scores, const int32_t* nvis, int B, int S, int N_cap, int k, int32_t* topk_idx,
              double* kth) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      size_t q = (size_t)b * S + s;
      int nv = nvis[q];
      orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * (nv > 0 ? nv : 1));
      for (int e = 0; e < nv; ++e) {
        p[e].v = scores[q * N_cap + e];
        p[e].i = e;
      }
      qsort(p, nv, sizeof(orc_pair), cmp_pair);
      int keep = nv < k ? nv : k;
      for (int j = 0; j < k; ++j) topk_idx[q * k + j] = j < keep ? p[j].i : -1;
      if (kth) kth[q] = keep > 0 ? p[keep - 1].v : NAN;
      free(p);
    }
}

/* ---- attention ---------------------------------------------------------
 * [P1] shared-normalisation section: window entries and selected compressed
 * entries form one candidate set under one softmax; a learned per-head sink
 * adds exp(sink) to the denominator and contributes no value.  [P5] 2.3:
 * every head attends to the same single KV row (MQA); the output is
 * de-rotated.  [P1] output-projection section: o = inverse_RoPE(o).
 *
 * Candidates of query position t:
 *   window rows of positions u in [max(0, t-window+1), t]; with win_pos0 ==
 *   NULL the window buffer is a ring (row u mod W_cap), else row u-win_pos0[b];
 *   compressed entries: if topk_idx != NULL, the entries of topk_idx[b,s,:k]
 *   in [0, N_cap) (padding -1 and indices past the cache select nothing);
 *   otherwise (dense, HCA) every s < (t+1)/ratio.
 * logits l = scale * <q_h, row>;  Z = sum exp(l) + exp(sink_h);
 * o_h = sum exp(l)/Z * row; out = o with its last rope_dim dims rotated by
 * -theta(t).  lse[b,s,h] = log Z (nullable).  ncand[b,s] = candidate count
 * (nullable).  Returns 0, or -1 if a window row is outside the buffer. */
int orc_attn(const void* q, int qdt, const void* cmp_cache, int cdt, const int32_t* topk_idx, int k, int ratio,
             const void* win_kv, int wdt, const int32_t* win_pos0, const double* sink, const int32_t* q_pos,
             double* out, double* lse, int32_t* ncand, int B, int S, int H, int D, int rope_dim, int N_cap,
             int W_cap, int window, double scale, double rope_base) {
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad)
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s) {
      size_t qi = (size_t)b * S + s;
      long t = (long)q_pos[b] + s;
      /* gather the candidate rows as (source, row index) */
      long u0 = t - window + 1;
      if (u0 < 0) u0 = 0;
      long nwin = t - u0 + 1;
      long ncmp = 0;
      long nv = (t + 1) / (ratio > 0 ? ratio : 1);
      if (nv > N_cap) nv = N_cap;
      if (topk_idx) {
        /* a list entry that names no cache row (< 0: padding; >= N_cap)
         * selects nothing */
        for (int j = 0; j < k; ++j)
          if (topk_idx[qi * k + j] >= 0 && topk_idx[qi * k + j] < N_cap) ++ncmp;
      } else {
        ncmp = nv;
      }
      long n = nwin + ncmp;
      if (ncand) ncand[qi] = (int32_t)n;
      double** rows = (double**)malloc(sizeof(double*) * (n > 0 ? n : 1));
      for (long j = 0; j < n; ++j) rows[j] = (double*)malloc(sizeof(double) * D);
      long j = 0;
      for (long u = u0; u <= t; ++u, ++j) {
        long r = win_pos0 ? u - win_pos0[b] : u % W_cap;
        if (r < 0 || r >= W_cap || (!win_pos0 && t - u >= W_cap)) {
          bad = 1;
          r = 0;
        }
        for (int c = 0; c < D; ++c) rows[j][c] = ld(win_kv, wdt, ((size_t)b * W_cap + r) * D + c);
      }
      if (topk_idx) {
        for (int i = 0; i < k; ++i) {
          int e = topk_idx[qi * k + i];
          if (e < 0 || e >= N_cap) continue;
          for (int c = 0; c < D; ++c) rows[j][c] = ld(cmp_cache, cdt, ((size_t)b * N_cap + e) * D + c);
          ++j;
        }
      } else {
        for (long e = 0; e < nv; ++e, ++j)
          for (int c = 0; c < D; ++c) rows[j][c] = ld(cmp_cache, cdt, ((size_t)b * N_cap + e) * D + c);
      }
      double* logit = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
      double* o = (double*)malloc(sizeof(double) * D);
      for (int h = 0; h < H; ++h) {
        size_t qoff = (qi * H + h) * (size_t)D;
        double mx = sink[h];
        for (long c2 = 0; c2 < n; ++c2) {
          double dot = 0.0;
          for (int c = 0; c < D; ++c) dot += ld(q, qdt, qoff + c) * rows[c2][c];
          logit[c2] = scale * dot;
          if (logit[c2] > mx) mx = logit[c2];
        }
        double Z = exp(sink[h] - mx);
        for (long c2 = 0; c2 < n; ++c2) Z += exp(logit[c2] - mx);
        for (int c = 0; c < D; ++c) o[c] = 0.0;
        for (long c2 = 0; c2 < n; ++c2) {
          double p = exp(logit[c2] - mx) / Z;
          for (int c = 0; c < D; ++c) o[c] += p * rows[c2][c];
        }
        orc_rope(o + (D - rope_dim), rope_dim, (double)t, rope_base, -1);
        memcpy(out + qoff, o, sizeof(double) * D);
        if (lse) lse[qi * H + h] = mx + log(Z);
      }
      free(o);
      free(logit);
      for (long c2 = 0; c2 < n; ++c2) free(rows[c2]);
      free(rows);
    }
  return bad ? -1 : 0;
}

/* Threads an OpenMP region of this library uses (for reporting CPU timings). */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
