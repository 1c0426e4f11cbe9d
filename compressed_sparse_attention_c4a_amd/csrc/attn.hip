// attn.hip -- multi-query attention over the sliding window plus compressed
// entries, with a learned per-head sink and inverse RoPE on the output.
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", section "局部和压缩记忆，共用一次归一化": the
// window entries and the selected compressed entries form one candidate set
// under one softmax; each head's learned sink adds to the denominator and has
// no value.  Section "输出投影也分组…": o = inverse_RoPE(o) before the output
// projection.  "图解DeepSeek V4" 2: the window KV lives in a ring of window_size
// rows, the compressed channel contributes <= topK entries; 2.3: every head
// attends to the same KV row (MQA) and the output is de-rotated.
//
// Candidate list of query position t (virtual index j):
//   j <  nwin : window position u = t - nwin + 1 + j (nwin = min(window, t+1))
//   j >= nwin : compressed entry topk_idx[j - nwin] (sparse, CSA) or
//               j - nwin (dense, HCA: every visible entry)
// Entries outside [0, N_cap) (the -1 padding) are skipped.
#include "common.hpp"

namespace csa {

struct AttnArgs {
  const void* q;
  const void* cmp;
  const int32_t* topk_idx;  // sparse mode: [B, S, k] entry list
  const void* win;
  const int32_t* win_pos0;  // NULL => ring
  const float* sink;
  const int32_t* q_pos;
  void* out;
  float* lse;
  int dense;  // 1: every visible entry (HCA); 0: the listed entries (CSA)
  int S, H, D, rope_dim, N_cap, k, ratio, W_cap, window;
  float scale, base;
};

// Row pointer (element offset) of candidate j of query (b, t); -1 when skipped.
__device__ __forceinline__ long cand_row(const AttnArgs& a, int b, long t, int qi, int nwin, int j, bool* is_win) {
  if (j < nwin) {
    *is_win = true;
    const long u = t - nwin + 1 + j;
    long r = a.win_pos0 ? u - a.win_pos0[b] : u % a.W_cap;
    if (r < 0 || r >= a.W_cap) return -1;
    return ((long)b * a.W_cap + r) * a.D;
  }
  *is_win = false;
  const int jj = j - nwin;
  const long e = a.dense ? (long)jj : (long)a.topk_idx[(size_t)qi * a.k + jj];
  if (e < 0 || e >= a.N_cap) return -1;
  return ((long)b * a.N_cap + e) * a.D;
}

// One wave per (query, head); lane owns dims lane + 64*i.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int qi = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int b = qi / a.S, s = qi % a.S;
  const long t = (long)a.q_pos[b] + s;
  const int lane = threadIdx.x;
  const int nwin = (int)(t + 1 < a.window ? t + 1 : a.window);
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const T* q = (const T*)a.q + ((size_t)qi * a.H + h) * a.D;
  const T* win = (const T*)a.win;
  const T* cmp = (const T*)a.cmp;
  constexpr int MAXV = 8;  // D <= 512
  float qv[MAXV], acc[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = lane + 64 * i;
    qv[i] = c < a.D ? Elt<T>::ld(q, c) : 0.f;
    acc[i] = 0.f;
  }
  const float sink = a.sink[h];
  float m = sink, l = (sink == -INFINITY) ? 0.f : 1.f;
  for (int j = 0; j < nwin + ncmp; ++j) {
    bool is_win;
    const long off = cand_row(a, b, t, qi, nwin, j, &is_win);
    if (off < 0) continue;
    const T* row = is_win ? win + off : cmp + off;
    float rv[MAXV];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = lane + 64 * i;
      rv[i] = c < a.D ? Elt<T>::ld(row, c) : 0.f;
      part += qv[i] * rv[i];
    }
    const float x = a.scale * wave_sum(part);
    if (x > m) {
      const float r = expf(m - x);
      l *= r;
#pragma unroll
      for (int i = 0; i < MAXV; ++i) acc[i] *= r;
      m = x;
    }
    const float p = expf(x - m);
    l += p;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) acc[i] += p * rv[i];
  }
  __shared__ float o[512];
  const float invl = 1.f / l;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = lane + 64 * i;
    if (c < a.D) o[c] = acc[i] * invl;
  }
  __syncthreads();
  T* out = (T*)a.out + ((size_t)qi * a.H + h) * a.D;
  const int tail0 = a.D - a.rope_dim;
  for (int p = lane; p < a.D / 2; p += 64) {
    float x0 = o[2 * p], x1 = o[2 * p + 1];
    if (2 * p >= tail0) {
      float cs, sn;
      rope_cos_sin((double)t, p - tail0 / 2, a.rope_dim, a.base, &cs, &sn);
      // inverse rotation: angle -theta
      const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    Elt<T>::st(out, 2 * p, x0);
    Elt<T>::st(out, 2 * p + 1, x1);
  }
  if (a.lse && lane == 0) a.lse[(size_t)qi * a.H + h] = m + logf(l);
}

}  // namespace csa

namespace csa_host {
using namespace csa;

size_t attn_workspace_size(int, int, int, int, int) { return 0; }

hipError_t launch_attn(const void* q, const void* cmp, const int32_t* topk_idx, int k, int dense, int ratio,
                       const void* win,
                       const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                       void* ws, int B, int S, int H, int D, int rope_dim, int N_cap, int W_cap, int window,
                       float scale, float base, int dtype, hipStream_t st) {
  (void)ws;
  AttnArgs a{q, cmp, topk_idx, win, win_pos0, sink, q_pos, out, lse, dense, S, H, D, rope_dim, N_cap, k, ratio,
             W_cap, window, scale, base};
  const unsigned blocks = (unsigned)((size_t)B * S * H);
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(blocks), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<bf16>, dim3(blocks), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa_host
