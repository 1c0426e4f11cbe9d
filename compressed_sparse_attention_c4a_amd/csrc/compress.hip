// compress.hip -- token-level compressors C4A (ratio 4, overlapping 2*ratio
// state) and C128A (ratio 128, non-overlapping).
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", sections "压缩是逐通道的 learned pooling"
// (softmax over the token axis per channel, then RMSNorm, then RoPE on the
// tail dims), "一个通道，逐项算出压缩结果" (entry 0 has no previous group: those
// slots weigh 0) and "压缩条目必须等整组完成后才可见" (an entry exists once its
// group is complete).  "图解DeepSeek V4" 2.1: a C4A entry pools the previous
// group's first-half channels together with its own group's second-half
// channels; 3.1: C128A pools its own 128 tokens only.
//
// One workgroup per (sequence, candidate group, job); thread p owns the
// channel pair (2p, 2p+1), which is also a RoPE pair.  Slots are folded with an online
// softmax in fp32.  Memory-bound and tiny next to the indexer and attention.
#include "common.hpp"

#include <cmath>

namespace csa {

// blockIdx.z selects the job (j0 or j1): both compressors of a CSA layer
// (main KV and index keys) run in one launch.
template <typename T>
__global__ __launch_bounds__(256) void compress_kernel(CompressJob j0, CompressJob j1, const int32_t* __restrict__ pos0,
                                                       int L, int ratio, float eps, double log2_base) {
  const CompressJob& J = blockIdx.z == 0 ? j0 : j1;
  const T* __restrict__ kv = (const T*)J.kv;
  const T* __restrict__ sc = (const T*)J.sc;
  const float* __restrict__ gamma = J.gamma;
  T* __restrict__ cache = (T*)J.cache;
  const int d = J.d, rope_dim = J.rope_dim, overlap = J.overlap, N_cap = J.N_cap;
  const int b = blockIdx.y;
  const int p = threadIdx.x;
  const bool active = 2 * p < d;
  // gamma does not depend on the position: its load overlaps the pos0 round trip
  float gm0 = 0.f, gm1 = 0.f;
  if (active) {
    gm0 = gamma[2 * p];
    gm1 = gamma[2 * p + 1];
  }
  const long p0 = pos0[b];
  const long g = floor_div(p0, ratio) + blockIdx.x;
  const long first = g * ratio, last = first + ratio - 1;
  // The whole block takes the same exit: every condition depends on (b, g) only.
  if (g < 0 || g >= N_cap || first < p0 || last > p0 + L - 1) return;
  if (overlap && g > 0 && first - ratio < p0) return;

  const int m = overlap ? 2 : 1;
  const size_t row_w = (size_t)m * d;
  const T* kvb = kv + (size_t)b * L * row_w;
  const T* scb = sc + (size_t)b * L * row_w;

  float y[2] = {0.f, 0.f};
  if (active) {
    // Slots are processed in chunks of 16 whose loads are all issued before
    // any of them is used, so the memory latency is paid once per chunk.
    constexpr int CH = 16;
    const int nslot = overlap ? 2 * ratio : ratio;
    float mx[2] = {-INFINITY, -INFINITY}, den[2] = {0.f, 0.f}, num[2] = {0.f, 0.f};
    for (int j0 = 0; j0 < nslot; j0 += CH) {
      float sv[CH][2], vv[CH][2];
#pragma unroll
      for (int jj = 0; jj < CH; ++jj) {
        const int j = j0 + jj;
        sv[jj][0] = sv[jj][1] = -INFINITY;
        vv[jj][0] = vv[jj][1] = 0.f;
        if (j >= nslot) continue;
        long tok;
        int ch;
        if (overlap && j < ratio) {
          if (g == 0) continue;  // missing previous group: weight 0
          tok = first - ratio + j;
          ch = 2 * p;
        } else {
          tok = first + (overlap ? j - ratio : j);
          ch = overlap ? d + 2 * p : 2 * p;
        }
        const size_t off = (size_t)(tok - p0) * row_w + ch;
        Elt<T>::ld2(scb, off, sv[jj][0], sv[jj][1]);
        Elt<T>::ld2(kvb, off, vv[jj][0], vv[jj][1]);
      }
#pragma unroll
      for (int jj = 0; jj < CH; ++jj)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float sj = sv[jj][h];
          if (sj == -INFINITY) continue;
          if (sj > mx[h]) {
            const float r = expf(mx[h] - sj);
            den[h] *= r;
            num[h] *= r;
            mx[h] = sj;
          }
          const float e = expf(sj - mx[h]);
          den[h] += e;
          num[h] += e * vv[jj][h];
        }
    }
    y[0] = num[0] / den[0];
    y[1] = num[1] / den[1];
  }

  // RMSNorm over the d channels of the entry.
  __shared__ float part[4];
  float ss = wave_sum(y[0] * y[0] + y[1] * y[1]);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  if (!active) return;
  float a = y[0] * inv * gm0, bb = y[1] * inv * gm1;
  const int tail0 = d - rope_dim;
  if (2 * p >= tail0) {
    float cs, sn;
    rope_cos_sin((double)first, p - tail0 / 2, rope_dim, log2_base, &cs, &sn);
    const float ra = a * cs - bb * sn, rb = a * sn + bb * cs;
    a = ra;
    bb = rb;
  }
  T* dst = cache + ((size_t)b * N_cap + g) * d;
  Elt<T>::st(dst, 2 * p, a);
  Elt<T>::st(dst, 2 * p + 1, bb);
}

}  // namespace csa

namespace csa_host {
using namespace csa;

hipError_t launch_compress(const CompressJob* jobs, int njobs, const int32_t* pos0, int B, int L, int ratio,
                           float eps, float base, int dtype, hipStream_t st) {
  // Groups that can intersect [pos0, pos0 + L): at most ceil(L / ratio) + 1.
  dim3 grid((unsigned)((L + ratio - 1) / ratio + 1), (unsigned)B, (unsigned)njobs);
  const CompressJob j1 = njobs > 1 ? jobs[1] : jobs[0];
  const double l2b = std::log2((double)base);
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(256), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
  else
    hipLaunchKernelGGL(compress_kernel<bf16>, grid, dim3(256), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
  return hipGetLastError();
}

}  // namespace csa_host
