/*
 * csa.h -- C ABI of the MI355X (gfx950) compressed attention library
 * (libcsa.so): DeepSeek-V4 token-level compressors (C4A, C128A), the
 * indexer with top-k selection, and multi-query attention over a sliding
 * window plus compressed entries with a learned sink and inverse RoPE.
 *
 * Sources (page titles as published):
 *   [P1] "DeepSeek-V4-Pro 架构：一个 token 的旅程" (hs-black.github.io)
 *   [P5] "图解DeepSeek V4：详细计算流程解析" (jsqmd.com)
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays owned
 *     by the caller.  The library never allocates, frees or synchronises; it
 *     enqueues kernels on `stream` (a hipStream_t; NULL is the null stream)
 *     and returns.  Kernels may still be running when a call returns.
 *   - `dtype` is CSA_F32 or CSA_BF16 and applies to q, q_idx, caches, window
 *     rows, compressor states and attention outputs.  gamma, w, sink and
 *     scores are always fp32; positions and indices are int32.
 *   - Positions are per batch row (device int32 arrays of length B), so every
 *     request may have its own length.  Visibility, windows and RoPE angles
 *     are derived from them inside the kernels.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     violation the call returns a negative CSA_ERR_* code, enqueues nothing,
 *     and csa_last_error() (thread-local) describes the problem.  A launch
 *     failure returns CSA_ERR_HIP.  Values inside device arrays (positions,
 *     indices) are not visible to the host: kernels skip entries that fall
 *     outside the buffers instead of reading out of bounds.
 *   - Every pointer must be 16-byte aligned (CSA_ERR_ALIGN otherwise).
 *   - Calls are re-entrant: no state is kept between calls.
 *   - The *_workspace_size functions return 0 for shapes their calls reject.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* csa_stream_t; /* identical to hipStream_t */

#define CSA_F32 0
#define CSA_BF16 1
/* bf16 activations (q, out, compressor states) with window and compressed KV
 * rows in the FP8 row format of csa_quantize_rows (attention and compressor
 * entry points; the index-key cache stays bf16).  Compressors write fresh
 * main-cache entries quantised from their float32 values (d = 512 and
 * rope_dim = 64 required, CSA_ERR_UNSUPPORTED otherwise). */
#define CSA_BF16_KV_FP8 2

#define CSA_OK 0
#define CSA_ERR_NULL (-1)        /* a required pointer is NULL */
#define CSA_ERR_SHAPE (-2)       /* a size is out of range or sizes disagree */
#define CSA_ERR_DTYPE (-3)       /* dtype is neither CSA_F32 nor CSA_BF16 */
#define CSA_ERR_UNSUPPORTED (-4) /* no kernel instantiation for this size */
#define CSA_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned */
#define CSA_ERR_WORKSPACE (-6)   /* workspace missing or too small */
#define CSA_ERR_HIP (-7)         /* the HIP runtime reported a launch error */

/* Flags of csa_index_scores / csa_index_topk. */
#define CSA_INDEX_NO_RELU 1u /* score = sum_h w_h * (q_h . k), without ReLU */

/* FP8 KV rows: bytes per row of D = 512 values (see csa_quantize_rows). */
#define CSA_FP8_ROW_BYTES 640

int csa_version(void);
const char* csa_error_string(int code);
const char* csa_last_error(void); /* detail of the calling thread's last error */

/*
 * csa_compress -- token-level compressor, [P1] "压缩是逐通道的 learned pooling",
 * "一个通道，逐项算出压缩结果", "压缩条目必须等整组完成后才可见"; [P5] 2.1 (C4A) and
 * 3.1 (C128A).
 *
 * kv_state, score_state: [B, L, m*d], m = 2 if overlap else 1.  Row r of
 *   batch b holds the compressor projections of absolute token pos0[b] + r.
 *   With overlap (C4A), channels [0,d) of a token feed the NEXT entry and
 *   channels [d,2d) feed the token's own entry.  A rolling [2*ratio, 2*d]
 *   state buffer whose pre half holds the previous group is a valid argument
 *   (L = 2*ratio, pos0 = first token of the previous group).
 * gamma: [d] RMSNorm gain.  cache: [B, N_cap, d]; only rows of completed
 *   entries are written.  pos0: [B] device int32.
 * Entry g (tokens [g*ratio, g*ratio+ratio)) is written iff all its tokens
 *   lie in the buffer and, with overlap, g == 0 or the previous group's
 *   tokens do too, and g < N_cap.  For every channel c the entry's slots
 *   are weighted by a softmax of their scores over the token axis (missing
 *   previous-group slots of entry 0 get weight 0), summed, then the row is
 *   RMS-normalised (eps) and scaled by gamma, and its last rope_dim dims are
 *   rotated (interleaved pairs, base rope_base) at position g*ratio.
 * Requires: 1 <= d <= 512, d even, 0 <= rope_dim <= d, rope_dim even,
 *   ratio >= 1, L >= 1, B >= 1, N_cap >= 1.
 */
int csa_compress(const void* kv_state, const void* score_state, const float* gamma, void* cache,
                 const int32_t* pos0, int B, int L, int d, int rope_dim, int ratio, int overlap, int N_cap,
                 float eps, float rope_base, int dtype, csa_stream_t stream);

/*
 * csa_compress_kv_index -- both compressors of a CSA layer in one launch: the
 * main KV cache (as csa_compress with d, rope_dim, overlap, N_cap) and the
 * index-key cache, which [P5] 2.2 builds with its own C4A compressor
 * (always overlapping; di, idx_rope_dim, idx_gamma, idx_N_cap).  Both state
 * buffers cover the same tokens: [B, L, m*d] and [B, L, 2*di] with row r at
 * absolute token pos0[b] + r.  Results are identical to two csa_compress
 * calls.  Requires what csa_compress requires, for both jobs.
 */
int csa_compress_kv_index(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                          int rope_dim, int overlap, int N_cap, const void* idx_kv_state,
                          const void* idx_score_state, const float* idx_gamma, void* idx_cache, int di,
                          int idx_rope_dim, int idx_N_cap, const int32_t* pos0, int B, int L, int ratio, float eps,
                          float rope_base, int dtype, csa_stream_t stream);

/*
 * csa_index_scores -- indexer scores, [P1] "少读 KV 之前，Indexer 仍要给历史打分";
 * [P5] 2.2.
 *
 * q_idx: [B, S, Hi, di]; w: [B, S, Hi] fp32 signed per-head weights, already
 *   scaled (1/sqrt(di)/sqrt(Hi) in the model); idx_cache: [B, N_cap, di];
 *   q_pos: [B] device int32, query s of batch b sits at q_pos[b] + s.
 * scores: [B, S, N_cap] fp32 output.  For entry e < nvis = min((t+1)/ratio,
 *   N_cap): sum_h w[h] * ReLU(q_idx[h] . idx_cache[e]); entries e >= nvis
 *   are set to -inf.
 * Requires: Hi >= 1, di >= 1, S >= 1.
 */
int csa_index_scores(const void* q_idx, const float* w, const void* idx_cache, const int32_t* q_pos, float* scores,
                     int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags, int dtype,
                     csa_stream_t stream);

/*
 * csa_topk -- keeps at most k compressed entries per query, [P5] sections 2
 * and 2.2.
 *
 * scores: [B, S, N_cap] fp32; only entries e < nvis (same rule as above) are
 *   candidates.  topk_idx: [B, S, k] int32 output: the min(k, nvis) entries
 *   with the largest scores (ties go to the lower entry index), in no
 *   particular order, then -1 in the remaining slots.  topk_score: [B, S, k]
 *   fp32 output of the matching scores (-inf on padding), may be NULL.
 * workspace: device scratch of csa_topk_workspace_size() bytes (may be NULL
 *   when that size is 0).
 * Requires: 1 <= k <= 4096.
 */
size_t csa_topk_workspace_size(int B, int S, int N_cap, int k);
int csa_topk(const float* scores, const int32_t* q_pos, int32_t* topk_idx, float* topk_score, void* workspace,
             size_t workspace_bytes, int B, int S, int N_cap, int k, int ratio, csa_stream_t stream);

/*
 * csa_index_topk -- csa_index_scores followed by csa_topk.  The score buffer
 * ([P1]: the query x candidate score buffer is temporary memory) lives at the
 * start of `workspace` as [B, S, N_cap] fp32 and holds the scores afterwards.
 */
size_t csa_index_topk_workspace_size(int B, int S, int N_cap, int k);
int csa_index_topk(const void* q_idx, const float* w, const void* idx_cache, const int32_t* q_pos,
                   int32_t* topk_idx, float* topk_score, void* workspace, size_t workspace_bytes, int B, int S,
                   int Hi, int di, int N_cap, int k, int ratio, unsigned flags, int dtype, csa_stream_t stream);

/*
 * csa_compress_index_topk -- csa_compress_kv_index followed by csa_index_topk
 * over the index cache it writes ([P1] "少读 KV 之前，Indexer 仍要给历史打分": the
 * indexer scores the entries the compressor has completed, this step's
 * included; [P5] 2.2).  Arguments as in those two calls; both caches hold
 * N_cap entries (cache [B, N_cap, d], idx_cache [B, N_cap, di]) and the
 * index-key compressor always overlaps.  Results are identical to the two
 * calls.  When every query is a single position per sequence (S == 1), the
 * state buffer holds at most 2*ratio tokens (decode) and the indexer takes
 * its MFMA path, the compressors run inside the indexer launch: the wave that
 * scores a freshly written index entry computes that entry itself, so no
 * workgroup waits for another.  workspace: csa_index_topk_workspace_size.
 */
int csa_compress_index_topk(const void* kv_state, const void* score_state, const float* gamma, void* cache, int d,
                            int rope_dim, int overlap, const void* idx_kv_state, const void* idx_score_state,
                            const float* idx_gamma, void* idx_cache, int idx_rope_dim, const int32_t* state_pos0,
                            int L, const void* q_idx, const float* w, const int32_t* q_pos, int32_t* topk_idx,
                            float* topk_score, void* workspace, size_t workspace_bytes, int B, int S, int Hi, int di,
                            int N_cap, int k, int ratio, unsigned flags, float eps, float rope_base, int dtype,
                            csa_stream_t stream);

/*
 * csa_compress_index_topk_noalloc -- csa_compress_index_topk without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The score buffer and the top-k round buffers live in a static
 * device array of the library, CSA_NOALLOC_SCRATCH_BYTES on every GPU the
 * library runs on (held until the process ends).  Arguments, results and
 * launches are those of csa_compress_index_topk; the scores are not
 * returned.  The first call on a device resolves the array's address on that
 * device (hipGetSymbolAddress, done once per device: make that first call
 * outside graph capture); no call allocates or frees anything.  Every call on
 * one GPU uses the same array: calls that may overlap in time on one GPU
 * (different streams without ordering) race.  Returns CSA_ERR_WORKSPACE when
 * csa_index_topk_workspace_size(B, S, N_cap, k) exceeds
 * CSA_NOALLOC_SCRATCH_BYTES (decode up to B * N_cap = 16M entries; longer
 * prefill chunks need the workspace form).
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int csa_compress_index_topk_noalloc(const void* kv_state, const void* score_state, const float* gamma, void* cache,
                                    int d, int rope_dim, int overlap, const void* idx_kv_state,
                                    const void* idx_score_state, const float* idx_gamma, void* idx_cache,
                                    int idx_rope_dim, const int32_t* state_pos0, int L, const void* q_idx,
                                    const float* w, const int32_t* q_pos, int32_t* topk_idx, float* topk_score, int B,
                                    int S, int Hi, int di, int N_cap, int k, int ratio, unsigned flags, float eps,
                                    float rope_base, int dtype, csa_stream_t stream);

/*
 * csa_sparse_attn -- multi-query attention over the window plus the selected
 * compressed entries, [P1] "局部和压缩记忆，共用一次归一化" (one candidate set, one
 * softmax, per-head sink adds to the denominator only), "输出投影也分组…"
 * (o = inverse_RoPE(o)); [P5] 2 (window ring, <= window+topK reads) and 2.3
 * (sink, MQA, de-rotation).
 *
 * q: [B, S, H, D] (already normalised and rotated); cmp_cache: [B, N_cap, D];
 * topk_idx: [B, S, k] int32 (entries < 0 or >= N_cap are skipped);
 * win_kv: [B, W_cap, D] window rows.  With win_pos0 == NULL the window is a
 *   ring: position u lives in row u % W_cap.  Otherwise row u - win_pos0[b].
 * sink: [H] fp32 logits; q_pos: [B] device int32.
 * out: [B, S, H, D]; lse: [B, S, H] fp32 log of the softmax denominator
 *   (sink included), may be NULL.
 * For query position t, the candidates are the window rows of positions
 *   [max(0, t-window+1), t] and the listed entries; logit = softmax_scale *
 *   (q_h . row); o_h = sum exp(logit) row / (sum exp(logit) + exp(sink_h));
 *   the last rope_dim dims of o_h are rotated back by position t.  The same
 *   row is key and value.
 * Requires: 1 <= window <= W_cap (ring mode), D <= 512, D even, rope_dim
 *   even <= D, k >= 0.  The MFMA path runs for dtype CSA_BF16, D == 512,
 *   H % 16 == 0, k <= 2048 and window <= 1024; other shapes use a vector-ALU
 *   kernel.  dtype CSA_BF16_KV_FP8: q and out bf16, cmp_cache and win_kv rows
 *   in the FP8 row format of csa_quantize_rows ([.., CSA_FP8_ROW_BYTES]
 *   bytes per row), read as their dequantised values; MFMA path only
 *   (D == 512, rope_dim == 64, H % 16 == 0, k <= 2048, window <= 1024;
 *   CSA_ERR_UNSUPPORTED otherwise).
 * workspace: csa_attn_workspace_size(B, S, H, D, n_cand) bytes with n_cand =
 *   window + k (csa_sparse_attn) or window + N_cap (hca_attn); 0 means none
 *   is needed and workspace may be NULL.  When small batches split each
 *   query's candidates over several workgroups, the workspace holds their
 *   partial results until a second kernel on the same stream merges them.
 *   Its contents need no initialisation; calls that may run at the same
 *   time need separate workspaces.
 */
size_t csa_attn_workspace_size(int B, int S, int H, int D, int n_cand);
int csa_sparse_attn(const void* q, const void* cmp_cache, const int32_t* topk_idx, const void* win_kv,
                    const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int S, int H, int D, int rope_dim, int N_cap,
                    int k, int W_cap, int window, float softmax_scale, float rope_base, int dtype,
                    csa_stream_t stream);

/*
 * hca_attn -- as csa_sparse_attn, but the compressed candidates are ALL
 * entries e < min((t+1)/ratio, N_cap) (HCA has no indexer, [P5] 3).
 */
int hca_attn(const void* q, const void* cmp_cache, const void* win_kv, const int32_t* win_pos0, const float* sink,
             const int32_t* q_pos, void* out, float* lse, void* workspace, size_t workspace_bytes, int B, int S,
             int H, int D, int rope_dim, int N_cap, int ratio, int W_cap, int window, float softmax_scale,
             float rope_base, int dtype, csa_stream_t stream);

/*
 * swa_attn -- sliding-window attention layer ([P5] 1: the model's third
 * attention type, SWA): multi-query attention over the window rows alone,
 * with the per-head sink and the inverse RoPE of csa_sparse_attn ([P1]
 * "局部和压缩记忆，共用一次归一化", "输出投影也分组…"; [P5] 2 window ring, 2.3).
 * Arguments and results are those of csa_sparse_attn without a compressed
 * channel (no cache, no list: N_cap = k = 0); workspace:
 * csa_attn_workspace_size(B, S, H, D, window).
 */
int swa_attn(const void* q, const void* win_kv, const int32_t* win_pos0, const float* sink, const int32_t* q_pos,
             void* out, float* lse, void* workspace, size_t workspace_bytes, int B, int S, int H, int D, int rope_dim,
             int W_cap, int window, float softmax_scale, float rope_base, int dtype, csa_stream_t stream);

/*
 * csa_quantize_rows -- KV rows to the FP8 row format, [P5] §2 (CSA模块): the
 * rope_head_dim part of a window KV row is rotated, the rest is quantised (the
 * page states neither format nor granularity; the reading taken):
 *   bytes [0, 448): OCP FP8 E4M3 codes (bias 7, largest 448, no infinity) of
 *     dims 0..447 divided by 2^k_b, rounded to nearest, ties to the even code;
 *   bytes [448, 576): dims 448..511 (the RoPE dims) as bf16, unchanged;
 *   bytes [576, 583): k_0..k_6 as int8, k_b the smallest integer with
 *     max over block b (dims 64b..64b+63) of |x| <= 448 * 2^k_b (0 for an
 *     all-zero block), clamped to [-120, 120]; bytes [583, 640): zero.
 * A stored value reads back as E4M3 value * 2^k_b, exactly a bf16 value.
 * src: [rows, 512] bf16; dst: [rows, CSA_FP8_ROW_BYTES] bytes; no overlap.
 * Requires D == 512 and rope_dim == 64.
 */
int csa_quantize_rows(const void* src, void* dst, long rows, int D, int rope_dim, csa_stream_t stream);

/*
 * csa_dequantize_rows -- FP8 rows back to bf16 [rows, 512] (exact).
 */
int csa_dequantize_rows(const void* src, void* dst, long rows, int D, int rope_dim, csa_stream_t stream);

/*
 * csa_pack_weights -- the weight layout read by csa_q_proj and csa_o_proj.
 * w: groups x [N][K] bf16 row-major (a weight applied as x W^T); packed:
 * groups x N*K bf16, written, not overlapping w.  Group g, block (c, h) of
 * 16 columns x 512 dims sits at element g*N*K + (c*K/512 + h) * 8192 and holds,
 * for k-step j in [0, 16) and lane l in [0, 64), the eight values
 * W[16c + l%16][512h + 32j + 8*(l/16) + e] (e in [0, 8)) at (64j + l)*8 + e.
 * A pure permutation: packing is exact.  Done once per weight, off the hot path.
 * Requires: N a positive multiple of 64, K of 512.
 */
int csa_pack_weights(const void* w, void* packed, int groups, int N, int K, csa_stream_t stream);

/*
 * csa_q_proj -- low-rank query projection, [P1] "低秩 Q：两次矩阵乘法接起来":
 *   qr = RMSNorm(x wq_a^T) with gain gamma_q;  q = qr wq_b^T as [M, H, D];
 *   each head divided by sqrt(mean over D of q^2 + eps); RoPE (the pair
 *   rotation of the compressed entries) on the last rope_dim dims of every
 *   head at the row's position.  Rows are M = B*S tokens, sequence-major:
 *   row m is token m % S of sequence m / S, at position pos[m / S] + m % S.
 *
 * x: [M, d_model] bf16; wq_a: [q_rank, d_model] bf16 and wq_b: [H*D, q_rank]
 *   bf16, both packed by csa_pack_weights (groups = 1); gamma_q: [q_rank]
 *   fp32; pos: [B] device int32.
 * qr: [M, q_rank] bf16, written (it is also the second product's input);
 * q: [M, H, D] bf16, written: the attention's query layout.
 * Products accumulate in fp32; qr and q are rounded to bf16 once.
 * workspace: csa_q_proj_workspace_size(M, ...) bytes, device memory of fp32
 *   split-K partials; no initialisation needed; calls that may overlap need
 *   separate workspaces.  The call enqueues four kernels on `stream`.
 * Requires: d_model a multiple of 512; q_rank in {512, 1024, 1536, 2048};
 *   D a multiple of 256 in [256, 2048]; rope_dim even <= D; eps >= 0.
 */
size_t csa_q_proj_workspace_size(int M, int d_model, int q_rank, int H, int D);
int csa_q_proj(const void* x, const void* wq_a, const float* gamma_q, const void* wq_b, const int32_t* pos, void* qr,
               void* q, void* workspace, size_t workspace_bytes, int B, int S, int d_model, int q_rank, int H, int D,
               int rope_dim, float eps, float rope_base, csa_stream_t stream);

/*
 * csa_o_proj -- grouped output projection, [P1] "输出投影也分组，并且降低中间维度"
 * (the inverse RoPE that section starts with is already in the attention
 * output): heads h = g*(H/groups) .. (g+1)*(H/groups)-1 form group g;
 *   r[m, g] = o[m, group g's (H/groups)*D dims] wo_a[g]^T;
 *   y = r (flattened group-major) wo_b^T.
 *
 * o: [M, H, D] bf16 (attention output); wo_a: [groups, o_rank, H/groups*D]
 *   bf16 packed by csa_pack_weights(groups, o_rank, H/groups*D); wo_b:
 *   [d_model, groups*o_rank] bf16 packed with groups = 1.
 * r: [M, groups*o_rank] bf16, written; y: [M, d_model] bf16, written.
 * Products accumulate in fp32; r and y are rounded to bf16 once.
 * workspace: csa_o_proj_workspace_size(M, ...) bytes of fp32 partials, as
 *   for csa_q_proj.  The call enqueues four kernels on `stream`.
 * Requires: groups divides H; (H/groups)*D and groups*o_rank multiples of
 *   512; o_rank a multiple of 64; d_model a multiple of 256.
 */
size_t csa_o_proj_workspace_size(int M, int H, int D, int groups, int o_rank, int d_model);
int csa_o_proj(const void* o, const void* wo_a, const void* wo_b, void* r, void* y, void* workspace,
               size_t workspace_bytes, int M, int H, int D, int groups, int o_rank, int d_model,
               csa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
