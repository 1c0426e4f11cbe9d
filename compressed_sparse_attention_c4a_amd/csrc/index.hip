// index.hip -- indexer scores.
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", section "少读 KV 之前，Indexer 仍要给历史打分":
// 64 heads of 128 dims score every visible compressed index entry against one
// shared 128-dim index cache, with signed per-head weights w (not a softmax).
// "图解DeepSeek V4" 2.2: the index keys come from their own C4A compressor.
// Score(t, e) = sum_h w[t,h] * ReLU(q_idx[t,h] . k[e]) for e < (t+1)/ratio.
//
// Generic kernel: one thread per (query, entry), fp32 accumulation, any sizes
// and both element types.
#include "common.hpp"

namespace csa {

template <typename T>
__global__ __launch_bounds__(256) void index_scores_generic(const T* __restrict__ q, const float* __restrict__ w,
                                                            const T* __restrict__ K,
                                                            const int32_t* __restrict__ q_pos,
                                                            float* __restrict__ scores, int S, int Hi, int di,
                                                            int N_cap, int ratio, unsigned flags) {
  const int qi = blockIdx.y;
  const int b = qi / S, s = qi % S;
  const long t = (long)q_pos[b] + s;
  const long nv = visible_entries(t, ratio, N_cap);
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= N_cap) return;
  float* out = scores + (size_t)qi * N_cap;
  if (e >= nv) {
    out[e] = -INFINITY;
    return;
  }
  const T* qq = q + (size_t)qi * Hi * di;
  const T* kk = K + ((size_t)b * N_cap + e) * di;
  const float* ww = w + (size_t)qi * Hi;
  float acc = 0.f;
  for (int h = 0; h < Hi; ++h) {
    float dot = 0.f;
    for (int c = 0; c < di; ++c) dot += Elt<T>::ld(qq, (size_t)h * di + c) * Elt<T>::ld(kk, c);
    const float f = (flags & CSA_INDEX_NO_RELU) ? dot : fmaxf(dot, 0.f);
    acc += ww[h] * f;
  }
  out[e] = acc;
}

}  // namespace csa

namespace csa_host {
using namespace csa;

hipError_t launch_index_scores(const void* q, const float* w, const void* K, const int32_t* q_pos, float* scores,
                               int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags, int dtype,
                               hipStream_t st) {
  dim3 grid((unsigned)((N_cap + 255) / 256), (unsigned)(B * S));
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(index_scores_generic<float>, grid, dim3(256), 0, st, (const float*)q, w, (const float*)K,
                       q_pos, scores, S, Hi, di, N_cap, ratio, flags);
  else
    hipLaunchKernelGGL(index_scores_generic<bf16>, grid, dim3(256), 0, st, (const bf16*)q, w, (const bf16*)K, q_pos,
                       scores, S, Hi, di, N_cap, ratio, flags);
  return hipGetLastError();
}

}  // namespace csa_host
