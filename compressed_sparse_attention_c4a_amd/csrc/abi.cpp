// abi.cpp -- the extern "C" boundary of libcsa: host-side argument validation,
// error reporting and dispatch to the kernel launchers.  Nothing here
// allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

#include <cmath>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return CSA_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQ_PTR(p)                                                    \
  do {                                                                \
    if (!(p)) return fail(CSA_ERR_NULL, "%s: %s is NULL", fn, #p);    \
    if (!aligned(p)) return fail(CSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
#define OPT_PTR(p)                                                    \
  do {                                                                \
    if ((p) && !aligned(p)) return fail(CSA_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)
#define REQ(cond, ...)                                                \
  do {                                                                \
    if (!(cond)) return fail(CSA_ERR_SHAPE, __VA_ARGS__);             \
  } while (0)

int check_dtype(const char* fn, int dtype) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "%s: dtype %d is not CSA_F32/CSA_BF16", fn, dtype);
  return CSA_OK;
}

int launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int check_attn_common(const char* fn, const void* q, const void* cmp, const void* win, const int32_t* win_pos0,
                      const float* sink, const int32_t* q_pos, const void* out, const float* lse, int B, int S, int H,
                      int D, int rope_dim, int N_cap, int W_cap, int window, int dtype) {
  if (int rc = check_dtype(fn, dtype)) return rc;
  REQ_PTR(q);
  REQ_PTR(win);
  REQ_PTR(sink);
  REQ_PTR(q_pos);
  REQ_PTR(out);
  OPT_PTR(win_pos0);
  OPT_PTR(lse);
  OPT_PTR(cmp);
  REQ(B >= 1 && S >= 1 && H >= 1, "%s: B, S, H must be >= 1 (got %d, %d, %d)", fn, B, S, H);
  REQ(D >= 2 && D <= 512 && D % 2 == 0, "%s: D must be even and in [2, 512] (got %d)", fn, D);
  REQ(rope_dim >= 0 && rope_dim <= D && rope_dim % 2 == 0, "%s: rope_dim must be even and <= D (got %d)", fn,
      rope_dim);
  REQ(N_cap >= 0, "%s: N_cap must be >= 0", fn);
  REQ(N_cap == 0 || cmp, "%s: cmp_cache is NULL with N_cap > 0", fn);
  REQ(W_cap >= 1 && window >= 1, "%s: W_cap and window must be >= 1", fn);
  REQ(win_pos0 || window <= W_cap, "%s: ring window needs window <= W_cap (got %d > %d)", fn, window, W_cap);
  REQ((size_t)B * S * H <= (size_t)INT32_MAX, "%s: B*S*H too large", fn);
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_version(void) { return 1; }

const char* csa_error_string(int code) {
  switch (code) {
    case CSA_OK: return "ok";
    case CSA_ERR_NULL: return "null pointer";
    case CSA_ERR_SHAPE: return "invalid shape";
    case CSA_ERR_DTYPE: return "invalid dtype";
    case CSA_ERR_UNSUPPORTED: return "unsupported size";
    case CSA_ERR_ALIGN: return "misaligned pointer";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* csa_last_error(void) { return g_err; }

int csa_compress(const void* kv_state, const void* score_state, const float* gamma, void* cache, const int32_t* pos0,
                 int B, int L, int d, int rope_dim, int ratio, int overlap, int N_cap, float eps, float rope_base,
                 int dtype, csa_stream_t stream) {
  const char* fn = "csa_compress";
  if (int rc = check_dtype(fn, dtype)) return rc;
  REQ_PTR(kv_state);
  REQ_PTR(score_state);
  REQ_PTR(gamma);
  REQ_PTR(cache);
  REQ_PTR(pos0);
  REQ(B >= 1 && L >= 1 && N_cap >= 1, "%s: B, L, N_cap must be >= 1", fn);
  REQ(d >= 2 && d <= 512 && d % 2 == 0, "%s: d must be even and in [2, 512] (got %d)", fn, d);
  REQ(rope_dim >= 0 && rope_dim <= d && rope_dim % 2 == 0, "%s: rope_dim must be even and <= d", fn);
  REQ(ratio >= 1 && ratio <= 4096, "%s: ratio must be in [1, 4096]", fn);
  REQ(overlap == 0 || overlap == 1, "%s: overlap must be 0 or 1", fn);
  REQ(eps >= 0.f, "%s: eps must be >= 0", fn);
  REQ((L + ratio - 1) / ratio + 1 <= 65535 * 1024, "%s: L too large", fn);
  REQ(B <= 65535, "%s: B must be <= 65535", fn);
  const csa::CompressJob job{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap};
  return launched(fn, csa_host::launch_compress(&job, 1, pos0, B, L, ratio, eps, rope_base, dtype,
                                                (hipStream_t)stream));
}

int csa_compress_kv_index(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                          int rope_dim, int overlap, int N_cap, const void* idx_kv_state,
                          const void* idx_score_state, const float* idx_gamma, void* idx_cache, int di,
                          int idx_rope_dim, int idx_N_cap, const int32_t* pos0, int B, int L, int ratio, float eps,
                          float rope_base, int dtype, csa_stream_t stream) {
  const char* fn = "csa_compress_kv_index";
  if (int rc = check_dtype(fn, dtype)) return rc;
  REQ_PTR(kv_state);
  REQ_PTR(score_state);
  REQ_PTR(gamma);
  REQ_PTR(cache);
  REQ_PTR(idx_kv_state);
  REQ_PTR(idx_score_state);
  REQ_PTR(idx_gamma);
  REQ_PTR(idx_cache);
  REQ_PTR(pos0);
  REQ(B >= 1 && L >= 1 && N_cap >= 1 && idx_N_cap >= 1, "%s: B, L, N_cap, idx_N_cap must be >= 1", fn);
  REQ(d >= 2 && d <= 512 && d % 2 == 0, "%s: d must be even and in [2, 512] (got %d)", fn, d);
  REQ(di >= 2 && di <= 512 && di % 2 == 0, "%s: di must be even and in [2, 512] (got %d)", fn, di);
  REQ(rope_dim >= 0 && rope_dim <= d && rope_dim % 2 == 0, "%s: rope_dim must be even and <= d", fn);
  REQ(idx_rope_dim >= 0 && idx_rope_dim <= di && idx_rope_dim % 2 == 0, "%s: idx_rope_dim must be even and <= di",
      fn);
  REQ(ratio >= 1 && ratio <= 4096, "%s: ratio must be in [1, 4096]", fn);
  REQ(overlap == 0 || overlap == 1, "%s: overlap must be 0 or 1", fn);
  REQ(eps >= 0.f, "%s: eps must be >= 0", fn);
  REQ((L + ratio - 1) / ratio + 1 <= 65535 * 1024, "%s: L too large", fn);
  REQ(B <= 65535, "%s: B must be <= 65535", fn);
  const csa::CompressJob jobs[2] = {{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap},
                                    {idx_kv_state, idx_score_state, idx_gamma, idx_cache, di, idx_rope_dim, 1,
                                     idx_N_cap}};
  return launched(fn, csa_host::launch_compress(jobs, 2, pos0, B, L, ratio, eps, rope_base, dtype,
                                                (hipStream_t)stream));
}

static int check_index(const char* fn, const void* q_idx, const float* w, const void* idx_cache,
                       const int32_t* q_pos, int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags,
                       int dtype) {
  if (int rc = check_dtype(fn, dtype)) return rc;
  REQ_PTR(q_idx);
  REQ_PTR(w);
  REQ_PTR(idx_cache);
  REQ_PTR(q_pos);
  REQ(B >= 1 && S >= 1 && Hi >= 1 && di >= 1 && N_cap >= 1, "%s: B, S, Hi, di, N_cap must be >= 1", fn);
  REQ(ratio >= 1, "%s: ratio must be >= 1", fn);
  REQ((flags & ~CSA_INDEX_NO_RELU) == 0, "%s: unknown flag bits 0x%x", fn, flags);
  REQ((size_t)B * S <= 65535u, "%s: B*S must be <= 65535", fn);
  return CSA_OK;
}

int csa_index_scores(const void* q_idx, const float* w, const void* idx_cache, const int32_t* q_pos, float* scores,
                     int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags, int dtype,
                     csa_stream_t stream) {
  const char* fn = "csa_index_scores";
  if (int rc = check_index(fn, q_idx, w, idx_cache, q_pos, B, S, Hi, di, N_cap, ratio, flags, dtype)) return rc;
  REQ_PTR(scores);
  return launched(fn, csa_host::launch_index_scores(q_idx, w, idx_cache, q_pos, scores, B, S, Hi, di, N_cap, ratio,
                                                    flags, dtype, (hipStream_t)stream));
}

size_t csa_topk_workspace_size(int B, int S, int N_cap, int k) { return csa_host::topk_workspace_size(B, S, N_cap, k); }

static int check_topk(const char* fn, const float* scores, const int32_t* q_pos, const int32_t* topk_idx,
                      const float* topk_score, int B, int S, int N_cap, int k, int ratio) {
  REQ_PTR(scores);
  REQ_PTR(q_pos);
  REQ_PTR(topk_idx);
  OPT_PTR(topk_score);
  REQ(B >= 1 && S >= 1 && N_cap >= 1, "%s: B, S, N_cap must be >= 1", fn);
  REQ(k >= 1 && k <= 4096, "%s: k must be in [1, 4096] (got %d)", fn, k);
  REQ(ratio >= 1, "%s: ratio must be >= 1", fn);
  REQ((size_t)B * S <= (size_t)INT32_MAX, "%s: B*S too large", fn);
  return CSA_OK;
}

int csa_topk(const float* scores, const int32_t* q_pos, int32_t* topk_idx, float* topk_score, void* workspace,
             size_t workspace_bytes, int B, int S, int N_cap, int k, int ratio, csa_stream_t stream) {
  const char* fn = "csa_topk";
  if (int rc = check_topk(fn, scores, q_pos, topk_idx, topk_score, B, S, N_cap, k, ratio)) return rc;
  const size_t need = csa_host::topk_workspace_size(B, S, N_cap, k);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  return launched(fn, csa_host::launch_topk(scores, q_pos, topk_idx, topk_score, workspace, B, S, N_cap, k, ratio,
                                            (hipStream_t)stream));
}

size_t csa_index_topk_workspace_size(int B, int S, int N_cap, int k) {
  const size_t sc = ((size_t)B * S * N_cap * sizeof(float) + 255) & ~(size_t)255;
  return sc + csa_host::topk_workspace_size(B, S, N_cap, k);
}

int csa_index_topk(const void* q_idx, const float* w, const void* idx_cache, const int32_t* q_pos,
                   int32_t* topk_idx, float* topk_score, void* workspace, size_t workspace_bytes, int B, int S, int Hi,
                   int di, int N_cap, int k, int ratio, unsigned flags, int dtype, csa_stream_t stream) {
  const char* fn = "csa_index_topk";
  if (int rc = check_index(fn, q_idx, w, idx_cache, q_pos, B, S, Hi, di, N_cap, ratio, flags, dtype)) return rc;
  REQ_PTR(topk_idx);
  OPT_PTR(topk_score);
  REQ(k >= 1 && k <= 4096, "%s: k must be in [1, 4096] (got %d)", fn, k);
  const size_t need = csa_index_topk_workspace_size(B, S, N_cap, k);
  if (!workspace || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  float* scores = (float*)workspace;
  void* tws = (char*)workspace + (((size_t)B * S * N_cap * sizeof(float) + 255) & ~(size_t)255);
  hipError_t e = csa_host::launch_index_scores(q_idx, w, idx_cache, q_pos, scores, B, S, Hi, di, N_cap, ratio, flags,
                                               dtype, (hipStream_t)stream);
  if (e != hipSuccess) return launched(fn, e);
  return launched(fn, csa_host::launch_topk(scores, q_pos, topk_idx, topk_score, tws, B, S, N_cap, k, ratio,
                                            (hipStream_t)stream));
}

int csa_compress_index_topk(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                            int rope_dim, int overlap, const void* idx_kv_state, const void* idx_score_state,
                            const float* idx_gamma, void* idx_cache, int idx_rope_dim, const int32_t* state_pos0,
                            int L, const void* q_idx, const float* w, const int32_t* q_pos, int32_t* topk_idx,
                            float* topk_score, void* workspace, size_t workspace_bytes, int B, int S, int Hi, int di,
                            int N_cap, int k, int ratio, unsigned flags, float eps, float rope_base, int dtype,
                            csa_stream_t stream) {
  const char* fn = "csa_compress_index_topk";
  if (int rc = check_index(fn, q_idx, w, idx_cache, q_pos, B, S, Hi, di, N_cap, ratio, flags, dtype)) return rc;
  REQ_PTR(kv_state);
  REQ_PTR(score_state);
  REQ_PTR(gamma);
  REQ_PTR(cache);
  REQ_PTR(idx_kv_state);
  REQ_PTR(idx_score_state);
  REQ_PTR(idx_gamma);
  REQ_PTR(state_pos0);
  REQ_PTR(topk_idx);
  OPT_PTR(topk_score);
  REQ(L >= 1, "%s: L must be >= 1", fn);
  REQ(d >= 2 && d <= 512 && d % 2 == 0, "%s: d must be even and in [2, 512] (got %d)", fn, d);
  REQ(di >= 2 && di <= 512 && di % 2 == 0, "%s: di must be even and in [2, 512] (got %d)", fn, di);
  REQ(rope_dim >= 0 && rope_dim <= d && rope_dim % 2 == 0, "%s: rope_dim must be even and <= d", fn);
  REQ(idx_rope_dim >= 0 && idx_rope_dim <= di && idx_rope_dim % 2 == 0, "%s: idx_rope_dim must be even and <= di",
      fn);
  REQ(ratio <= 4096, "%s: ratio must be in [1, 4096]", fn);
  REQ(overlap == 0 || overlap == 1, "%s: overlap must be 0 or 1", fn);
  REQ(eps >= 0.f, "%s: eps must be >= 0", fn);
  REQ((L + ratio - 1) / ratio + 1 <= 65535 * 1024, "%s: L too large", fn);
  REQ(k >= 1 && k <= 4096, "%s: k must be in [1, 4096] (got %d)", fn, k);
  const size_t need = csa_index_topk_workspace_size(B, S, N_cap, k);
  if (!workspace || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  const csa::CompressJob jobs[2] = {{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap},
                                    {idx_kv_state, idx_score_state, idx_gamma, idx_cache, di, idx_rope_dim, 1, N_cap}};
  float* scores = (float*)workspace;
  void* tws = (char*)workspace + (((size_t)B * S * N_cap * sizeof(float) + 255) & ~(size_t)255);
  const hipStream_t st = (hipStream_t)stream;
  const int gx = (L + ratio - 1) / ratio + 1;
  const csa::FusedCompress F{jobs[0], jobs[1], state_pos0, L, gx, B, 2 * gx * B, eps, std::log2((double)rope_base)};
  if (csa_host::fused_compress_ok(F, S, Hi, di, N_cap, ratio, dtype)) {
    // decode: compressors folded into the indexer (new index entries) and the top-k launch (cache rows)
    hipError_t e = csa_host::launch_index_scores_fused(F, q_idx, w, q_pos, scores, B, S, Hi, N_cap, ratio, flags, st);
    if (e != hipSuccess) return launched(fn, e);
    return launched(fn, csa_host::launch_topk(scores, q_pos, topk_idx, topk_score, tws, B, S, N_cap, k, ratio, st,
                                              &F));
  }
  hipError_t e = csa_host::launch_compress(jobs, 2, state_pos0, B, L, ratio, eps, rope_base, dtype, st);
  if (e != hipSuccess) return launched(fn, e);
  e = csa_host::launch_index_scores(q_idx, w, idx_cache, q_pos, scores, B, S, Hi, di, N_cap, ratio, flags, dtype, st);
  if (e != hipSuccess) return launched(fn, e);
  return launched(fn, csa_host::launch_topk(scores, q_pos, topk_idx, topk_score, tws, B, S, N_cap, k, ratio, st));
}

size_t csa_attn_workspace_size(int B, int S, int H, int D, int n_cand) {
  return csa_host::attn_workspace_size(B, S, H, D, n_cand);
}

int csa_sparse_attn(const void* q, const void* cmp_cache, const int32_t* topk_idx, const void* win_kv,
                    const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int S, int H, int D, int rope_dim, int N_cap,
                    int k, int W_cap, int window, float softmax_scale, float rope_base, int dtype,
                    csa_stream_t stream) {
  const char* fn = "csa_sparse_attn";
  if (int rc = check_attn_common(fn, q, cmp_cache, win_kv, win_pos0, sink, q_pos, out, lse, B, S, H, D, rope_dim,
                                 N_cap, W_cap, window, dtype))
    return rc;
  REQ(k >= 0 && k <= 65536, "%s: k must be in [0, 65536]", fn);
  if (k > 0) REQ_PTR(topk_idx);
  const size_t need = csa_host::attn_workspace_size(B, S, H, D, window + k);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  return launched(fn, csa_host::launch_attn(q, cmp_cache, topk_idx, k, 0, 1, win_kv, win_pos0, sink,
                                            q_pos, out, lse, workspace, B, S, H, D, rope_dim, N_cap, W_cap, window,
                                            softmax_scale, rope_base, dtype, (hipStream_t)stream));
}

int hca_attn(const void* q, const void* cmp_cache, const void* win_kv, const int32_t* win_pos0, const float* sink,
             const int32_t* q_pos, void* out, float* lse, void* workspace, size_t workspace_bytes, int B, int S, int H,
             int D, int rope_dim, int N_cap, int ratio, int W_cap, int window, float softmax_scale, float rope_base,
             int dtype, csa_stream_t stream) {
  const char* fn = "hca_attn";
  if (int rc = check_attn_common(fn, q, cmp_cache, win_kv, win_pos0, sink, q_pos, out, lse, B, S, H, D, rope_dim,
                                 N_cap, W_cap, window, dtype))
    return rc;
  REQ(ratio >= 1, "%s: ratio must be >= 1", fn);
  const size_t need = csa_host::attn_workspace_size(B, S, H, D, window + N_cap);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  return launched(fn, csa_host::launch_attn(q, cmp_cache, nullptr, 0, 1, ratio, win_kv, win_pos0, sink, q_pos, out, lse,
                                            workspace, B, S, H, D, rope_dim, N_cap, W_cap, window, softmax_scale,
                                            rope_base, dtype, (hipStream_t)stream));
}

}  // extern "C"
