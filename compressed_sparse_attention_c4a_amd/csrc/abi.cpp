// abi.cpp -- the extern "C" boundary of libcsa: host-side argument validation,
// error reporting and dispatch to the kernel launchers.  Nothing here
// allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

#include <cmath>
#include <mutex>

// Scratch of csa_compress_index_topk_noalloc: one copy per GPU, resolved to
// a device address once per device (the array's name is a host-side stand-in
// in host code: only the address returned by hipGetSymbolAddress is passed to
// kernels).
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

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

// Compressor entry points: CSA_BF16_KV_FP8 means bf16 states with the main
// cache (d = 512, rope_dim = 64) in FP8 rows; the index-key cache stays bf16.
int check_dtype_cmp(const char* fn, int dtype, int d, int rope_dim) {
  if (dtype == CSA_BF16_KV_FP8) {
    if (d != 512 || rope_dim != 64)
      return fail(CSA_ERR_UNSUPPORTED, "%s: an FP8 cache needs d = 512 and rope_dim = 64", fn);
    return CSA_OK;
  }
  return check_dtype(fn, dtype);
}

// the element type of states and bf16 caches
int elem_dtype(int dtype) { return dtype == CSA_BF16_KV_FP8 ? CSA_BF16 : dtype; }

int launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

int check_attn_common(const char* fn, const void* q, const void* cmp, const void* win, const int32_t* win_pos0,
                      const float* sink, const int32_t* q_pos, const void* out, const float* lse, int B, int S, int H,
                      int D, int rope_dim, int N_cap, int W_cap, int window, int dtype) {
  if (dtype == CSA_BF16_KV_FP8) {
    // FP8 KV rows are read by the MFMA kernel only
    if (D != 512 || rope_dim != 64 || H % 16 != 0 || window > 1024)
      return fail(CSA_ERR_UNSUPPORTED, "%s: FP8 KV rows need D = 512, rope_dim = 64, H %% 16 == 0, window <= 1024",
                  fn);
  } else if (int rc = check_dtype(fn, dtype)) {
    return rc;
  }
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
  if (int rc = check_dtype_cmp(fn, dtype, d, rope_dim)) return rc;
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
  REQ(((long)L + ratio - 1) / ratio <= 65535L * 1024, "%s: L too large", fn);
  REQ(B <= 65535, "%s: B must be <= 65535", fn);
  const csa::CompressJob job{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap,
                             dtype == CSA_BF16_KV_FP8};
  return launched(fn, csa_host::launch_compress(&job, 1, pos0, B, L, ratio, eps, rope_base, elem_dtype(dtype),
                                                (hipStream_t)stream));
}

int csa_compress_kv_index(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                          int rope_dim, int overlap, int N_cap, const void* idx_kv_state,
                          const void* idx_score_state, const float* idx_gamma, void* idx_cache, int di,
                          int idx_rope_dim, int idx_N_cap, const int32_t* pos0, int B, int L, int ratio, float eps,
                          float rope_base, int dtype, csa_stream_t stream) {
  const char* fn = "csa_compress_kv_index";
  if (int rc = check_dtype_cmp(fn, dtype, d, rope_dim)) return rc;
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
  REQ(((long)L + ratio - 1) / ratio <= 65535L * 1024, "%s: L too large", fn);
  REQ(B <= 65535, "%s: B must be <= 65535", fn);
  const csa::CompressJob jobs[2] = {{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap,
                                     dtype == CSA_BF16_KV_FP8},
                                    {idx_kv_state, idx_score_state, idx_gamma, idx_cache, di, idx_rope_dim, 1,
                                     idx_N_cap, 0}};
  return launched(fn, csa_host::launch_compress(jobs, 2, pos0, B, L, ratio, eps, rope_base, elem_dtype(dtype),
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
  if (B < 1 || S < 1 || N_cap < 1 || k < 1 || k > 4096) return 0;
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

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (resolved on the first
// call on that device).
int scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSA_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CSA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}
}  // namespace

int csa_compress_index_topk_noalloc(const void* kv_state, const void* score_state, const float* gamma, void* cache,
                                    int d, int rope_dim, int overlap, const void* idx_kv_state,
                                    const void* idx_score_state, const float* idx_gamma, void* idx_cache,
                                    int idx_rope_dim, const int32_t* state_pos0, int L, const void* q_idx,
                                    const float* w, const int32_t* q_pos, int32_t* topk_idx, float* topk_score, int B,
                                    int S, int Hi, int di, int N_cap, int k, int ratio, unsigned flags, float eps,
                                    float rope_base, int dtype, csa_stream_t stream) {
  const char* fn = "csa_compress_index_topk_noalloc";
  if (B < 1 || S < 1 || N_cap < 1 || k < 1)
    return fail(CSA_ERR_SHAPE, "%s: B, S, N_cap and k must be >= 1", fn);
  const size_t need = csa_index_topk_workspace_size(B, S, N_cap, k);
  if (need > CSA_NOALLOC_SCRATCH_BYTES)
    return fail(CSA_ERR_WORKSPACE, "%s: %zu bytes of scratch needed, the static array holds %zu", fn, need,
                (size_t)CSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_address(fn, &ws)) return rc;
  return csa_compress_index_topk(kv_state, score_state, gamma, cache, d, rope_dim, overlap, idx_kv_state,
                                 idx_score_state, idx_gamma, idx_cache, idx_rope_dim, state_pos0, L, q_idx, w, q_pos,
                                 topk_idx, topk_score, ws, need, B, S, Hi, di, N_cap, k, ratio, flags, eps, rope_base,
                                 dtype, stream);
}

int csa_compress_index_topk(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                            int rope_dim, int overlap, const void* idx_kv_state, const void* idx_score_state,
                            const float* idx_gamma, void* idx_cache, int idx_rope_dim, const int32_t* state_pos0,
                            int L, const void* q_idx, const float* w, const int32_t* q_pos, int32_t* topk_idx,
                            float* topk_score, void* workspace, size_t workspace_bytes, int B, int S, int Hi, int di,
                            int N_cap, int k, int ratio, unsigned flags, float eps, float rope_base, int dtype,
                            csa_stream_t stream) {
  const char* fn = "csa_compress_index_topk";
  if (int rc = check_dtype_cmp(fn, dtype, d, rope_dim)) return rc;
  const int dt = elem_dtype(dtype);
  if (int rc = check_index(fn, q_idx, w, idx_cache, q_pos, B, S, Hi, di, N_cap, ratio, flags, dt)) return rc;
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
  REQ(((long)L + ratio - 1) / ratio <= 65535L * 1024, "%s: L too large", fn);
  REQ(k >= 1 && k <= 4096, "%s: k must be in [1, 4096] (got %d)", fn, k);
  const size_t need = csa_index_topk_workspace_size(B, S, N_cap, k);
  if (!workspace || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  const csa::CompressJob jobs[2] = {{kv_state, score_state, gamma, cache, d, rope_dim, overlap, N_cap,
                                     dtype == CSA_BF16_KV_FP8},
                                    {idx_kv_state, idx_score_state, idx_gamma, idx_cache, di, idx_rope_dim, 1, N_cap, 0}};
  float* scores = (float*)workspace;
  void* tws = (char*)workspace + (((size_t)B * S * N_cap * sizeof(float) + 255) & ~(size_t)255);
  const hipStream_t st = (hipStream_t)stream;
  const int gx = csa_host::compress_gx(L, ratio);
  const csa::FusedCompress F{jobs[0], jobs[1], state_pos0, L, gx, B, 2 * gx * B, eps, std::log2((double)rope_base)};
  if (csa_host::fused_compress_ok(F, S, Hi, di, N_cap, ratio, dt)) {
    // decode: compressors folded into the indexer (new index entries) and the top-k launch (cache rows)
    hipError_t e = csa_host::launch_index_scores_fused(F, q_idx, w, q_pos, scores, B, S, Hi, N_cap, ratio, flags, st);
    if (e != hipSuccess) return launched(fn, e);
    return launched(fn, csa_host::launch_topk(scores, q_pos, topk_idx, topk_score, tws, B, S, N_cap, k, ratio, st,
                                              &F));
  }
  hipError_t e = csa_host::launch_compress(jobs, 2, state_pos0, B, L, ratio, eps, rope_base, dt, st);
  if (e != hipSuccess) return launched(fn, e);
  e = csa_host::launch_index_scores(q_idx, w, idx_cache, q_pos, scores, B, S, Hi, di, N_cap, ratio, flags, dt, st);
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
  if (dtype == CSA_BF16_KV_FP8 && k > 2048) return fail(CSA_ERR_UNSUPPORTED, "%s: FP8 KV rows need k <= 2048", fn);
  const size_t need = csa_host::attn_workspace_size(B, S, H, D, (long)window + k);
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
  const size_t need = csa_host::attn_workspace_size(B, S, H, D, (long)window + N_cap);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  return launched(fn, csa_host::launch_attn(q, cmp_cache, nullptr, 0, 1, ratio, win_kv, win_pos0, sink, q_pos, out, lse,
                                            workspace, B, S, H, D, rope_dim, N_cap, W_cap, window, softmax_scale,
                                            rope_base, dtype, (hipStream_t)stream));
}

int swa_attn(const void* q, const void* win_kv, const int32_t* win_pos0, const float* sink, const int32_t* q_pos,
             void* out, float* lse, void* workspace, size_t workspace_bytes, int B, int S, int H, int D, int rope_dim,
             int W_cap, int window, float softmax_scale, float rope_base, int dtype, csa_stream_t stream) {
  const char* fn = "swa_attn";
  if (int rc = check_attn_common(fn, q, nullptr, win_kv, win_pos0, sink, q_pos, out, lse, B, S, H, D, rope_dim, 0,
                                 W_cap, window, dtype))
    return rc;
  const size_t need = csa_host::attn_workspace_size(B, S, H, D, window);
  if (need && (!workspace || workspace_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  OPT_PTR(workspace);
  return launched(fn, csa_host::launch_attn(q, nullptr, nullptr, 0, 0, 1, win_kv, win_pos0, sink, q_pos, out, lse,
                                            workspace, B, S, H, D, rope_dim, 0, W_cap, window, softmax_scale,
                                            rope_base, dtype, (hipStream_t)stream));
}

// ---- FP8 KV rows -------------------------------------------------------------
static int check_fp8_rows(const char* fn, const void* src, const void* dst, long rows, int D, int rope_dim,
                          size_t src_row, size_t dst_row) {
  REQ_PTR(src);
  REQ_PTR(dst);
  REQ(rows >= 0 && rows <= (1L << 32), "%s: rows must be in [0, 2^32]", fn);
  REQ(D == 512 && rope_dim == 64, "%s: FP8 rows are defined for D = 512 and rope_dim = 64", fn);
  const char *a = (const char*)src, *b = (const char*)dst;
  REQ(a + rows * src_row <= b || b + rows * dst_row <= a, "%s: src and dst overlap", fn);
  return 0;
}

int csa_quantize_rows(const void* src, void* dst, long rows, int D, int rope_dim, csa_stream_t stream) {
  const char* fn = "csa_quantize_rows";
  if (int rc = check_fp8_rows(fn, src, dst, rows, D, rope_dim, 1024, CSA_FP8_ROW_BYTES)) return rc;
  return launched(fn, csa_host::launch_quantize_rows(src, dst, rows, (hipStream_t)stream));
}

int csa_dequantize_rows(const void* src, void* dst, long rows, int D, int rope_dim, csa_stream_t stream) {
  const char* fn = "csa_dequantize_rows";
  if (int rc = check_fp8_rows(fn, src, dst, rows, D, rope_dim, CSA_FP8_ROW_BYTES, 1024)) return rc;
  return launched(fn, csa_host::launch_dequantize_rows(src, dst, rows, (hipStream_t)stream));
}

// ---- projections around the attention --------------------------------------
static size_t max_sz(size_t a, size_t b) { return a > b ? a : b; }

int csa_pack_weights(const void* w, void* packed, int groups, int N, int K, csa_stream_t stream) {
  const char* fn = "csa_pack_weights";
  REQ_PTR(w);
  REQ_PTR(packed);
  REQ(groups >= 1 && N >= 64 && N % 64 == 0 && K >= 512 && K % 512 == 0,
      "%s: N must be a positive multiple of 64 and K of 512", fn);
  REQ((double)groups * N * (double)K <= 1e12, "%s: groups*N*K too large", fn);
  const size_t bytes = (size_t)groups * N * (size_t)K * 2;
  const char *a = (const char*)w, *b = (const char*)packed;
  REQ(a + bytes <= b || b + bytes <= a, "%s: w and packed overlap", fn);
  return launched(fn, csa_host::launch_pack_weights(w, packed, groups, N, K, (hipStream_t)stream));
}

size_t csa_q_proj_workspace_size(int M, int d_model, int q_rank, int H, int D) {
  if (M < 1 || M > (1 << 20) || d_model < 512 || d_model > (1 << 20) || q_rank < 512 || q_rank > 2048 || H < 1 ||
      D < 2 || (long)H * D > (1 << 20))
    return 0;  // outside what csa_q_proj accepts
  return max_sz(csa_host::gemm_partial_bytes(1, M, q_rank, d_model),
                csa_host::gemm_partial_bytes(1, M, H * D, q_rank));
}

int csa_q_proj(const void* x, const void* wq_a, const float* gamma_q, const void* wq_b, const int32_t* pos, void* qr,
               void* q, void* workspace, size_t workspace_bytes, int B, int S, int d_model, int q_rank, int H, int D,
               int rope_dim, float eps, float rope_base, csa_stream_t stream) {
  const char* fn = "csa_q_proj";
  REQ_PTR(x);
  REQ_PTR(wq_a);
  REQ_PTR(gamma_q);
  REQ_PTR(wq_b);
  REQ_PTR(pos);
  REQ_PTR(qr);
  REQ_PTR(q);
  REQ(B >= 1 && S >= 1 && (long)B * S <= (1 << 20), "%s: B*S must be in [1, 2^20]", fn);
  REQ(d_model >= 512 && d_model % 512 == 0 && d_model <= (1 << 20), "%s: d_model must be a multiple of 512 (<= 2^20)",
      fn);
  REQ(q_rank >= 512 && q_rank % 512 == 0 && q_rank <= 2048, "%s: q_rank must be 512, 1024, 1536 or 2048", fn);
  REQ(H >= 1 && D >= 256 && D <= 2048 && D % 256 == 0, "%s: D must be a multiple of 256 in [256, 2048]", fn);
  REQ((long)H * D <= (1 << 20), "%s: H*D must be <= 2^20", fn);
  REQ(rope_dim >= 0 && rope_dim <= D && rope_dim % 2 == 0, "%s: rope_dim must be even and <= D", fn);
  REQ(eps >= 0.0f && std::isfinite(eps), "%s: eps must be finite and >= 0", fn);
  const int M = B * S;
  const size_t need = csa_q_proj_workspace_size(M, d_model, q_rank, H, D);
  if (!workspace || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  REQ_PTR(workspace);
  hipStream_t st = (hipStream_t)stream;
  float* part = (float*)workspace;
  int ks = 0;
  hipError_t e = csa_host::launch_gemm_nt(x, wq_a, part, 1, M, q_rank, d_model, d_model, 0, 0, &ks, st);
  if (e == hipSuccess)
    e = csa_host::launch_rows_finish(part, qr, gamma_q, nullptr, M, q_rank, q_rank, q_rank, ks, 1, 0, 1, eps,
                                     rope_base, st);
  if (e == hipSuccess)
    e = csa_host::launch_gemm_nt(qr, wq_b, part, 1, M, H * D, q_rank, q_rank, 0, 0, &ks, st);
  if (e == hipSuccess)
    e = csa_host::launch_rows_finish(part, q, nullptr, pos, M, H * D, H * D, D, ks, 1, rope_dim, S, eps, rope_base,
                                     st);
  return launched(fn, e);
}

// Segment width of a plain (no norm) finishing pass: 1024 or 512 or 256
// columns, whichever divides the row.
static int finish_seg(int ncols) {
  for (int s = 1024; s >= 256; s >>= 1)
    if (ncols % s == 0) return s;
  return 0;
}

size_t csa_o_proj_workspace_size(int M, int H, int D, int groups, int o_rank, int d_model) {
  if (M < 1 || M > (1 << 20) || H < 1 || D < 1 || groups < 1 || H % groups != 0 || o_rank < 1 || d_model < 1 ||
      d_model > (1 << 20) || (long)H * D > (1 << 20) || (long)groups * o_rank > (1 << 20))
    return 0;  // outside what csa_o_proj accepts
  const int gdim = H / groups * D;
  return max_sz(csa_host::gemm_partial_bytes(groups, M, o_rank, gdim),
                csa_host::gemm_partial_bytes(1, M, d_model, groups * o_rank));
}

int csa_o_proj(const void* o, const void* wo_a, const void* wo_b, void* r, void* y, void* workspace,
               size_t workspace_bytes, int M, int H, int D, int groups, int o_rank, int d_model,
               csa_stream_t stream) {
  const char* fn = "csa_o_proj";
  REQ_PTR(o);
  REQ_PTR(wo_a);
  REQ_PTR(wo_b);
  REQ_PTR(r);
  REQ_PTR(y);
  REQ(M >= 1 && M <= (1 << 20), "%s: M must be in [1, 2^20]", fn);
  REQ(H >= 1 && D >= 1 && groups >= 1 && H % groups == 0, "%s: groups must divide H", fn);
  const long gdim = (long)H / groups * D;
  REQ(gdim % 512 == 0 && (long)H * D <= (1 << 20), "%s: (H/groups)*D must be a multiple of 512 (H*D <= 2^20)", fn);
  REQ(o_rank >= 64 && o_rank % 64 == 0, "%s: o_rank must be a positive multiple of 64", fn);
  REQ((long)groups * o_rank % 512 == 0 && (long)groups * o_rank <= (1 << 20),
      "%s: groups*o_rank must be a multiple of 512 (<= 2^20)", fn);
  REQ(d_model >= 256 && d_model % 256 == 0 && d_model <= (1 << 20), "%s: d_model must be a multiple of 256", fn);
  const size_t need = csa_o_proj_workspace_size(M, H, D, groups, o_rank, d_model);
  if (!workspace || workspace_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", fn, need, workspace_bytes);
  REQ_PTR(workspace);
  hipStream_t st = (hipStream_t)stream;
  float* part = (float*)workspace;
  const int rcols = groups * o_rank;
  int ks = 0;
  hipError_t e = csa_host::launch_gemm_nt(o, wo_a, part, groups, M, o_rank, (int)gdim, H * D, gdim,
                                          (long)o_rank * gdim, &ks, st);
  if (e == hipSuccess)
    e = csa_host::launch_rows_finish(part, r, nullptr, nullptr, M, rcols, o_rank, finish_seg(rcols), ks, 0, 0, 1,
                                     0.f, 10000.f, st);
  if (e == hipSuccess)
    e = csa_host::launch_gemm_nt(r, wo_b, part, 1, M, d_model, rcols, rcols, 0, 0, &ks, st);
  if (e == hipSuccess)
    e = csa_host::launch_rows_finish(part, y, nullptr, nullptr, M, d_model, d_model, finish_seg(d_model), ks, 0, 0,
                                     1, 0.f, 10000.f, st);
  return launched(fn, e);
}

}  // extern "C"
