// compress_dev.hpp -- device routines of the token-level compressors C4A
// (ratio 4, overlapping 2*ratio state) and C128A (ratio 128, non-overlapping),
// shared by the compressor kernel and the fused compress + indexer kernel.
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", sections "压缩是逐通道的 learned pooling"
// (softmax over the token axis per channel, then RMSNorm, then RoPE on the
// tail dims), "一个通道，逐项算出压缩结果" (entry 0 has no previous group: those
// slots weigh 0) and "压缩条目必须等整组完成后才可见" (an entry exists once its
// group is complete).  "图解DeepSeek V4" 2.1: a C4A entry pools the previous
// group's first-half channels together with its own group's second-half
// channels; 3.1: C128A pools its own 128 tokens only.
//
// The lane (thread) owning channel pair p = (2p, 2p+1), also a RoPE pair, runs
// the same instruction sequence in every caller, so an entry's values do not
// depend on which kernel computes them.
#pragma once
#include "common.hpp"

namespace csa {

// Group g = floor(p0 / ratio) + x of a sequence whose state buffer starts at
// absolute position p0 and holds L tokens, if the compressor writes it: its
// tokens lie in the buffer and (overlap) so do the previous group's, unless
// g == 0.  Else -1.
__device__ __forceinline__ long compress_group(const CompressJob& J, long p0, int x, int L, int ratio) {
  const long g = floor_div(p0, ratio) + x;
  const long first = g * ratio, last = first + ratio - 1;
  if (g < 0 || g >= J.N_cap || first < p0 || last > p0 + L - 1) return -1;
  if (J.overlap && g > 0 && first - ratio < p0) return -1;
  return g;
}

// Scores and values of up to 16 slots (j0 .. j0+15) of channels 2p, 2p+1 of
// entry g of sequence b; missing slots get score -inf.
struct PoolRegs {
  float sv[16][2], vv[16][2];
};

template <typename T>
__device__ __forceinline__ void compress_load16(const CompressJob& J, int b, long g, long p0, int L, int ratio, int p,
                                                int j0, PoolRegs& R) {
  const T* __restrict__ kv = (const T*)J.kv;
  const T* __restrict__ sc = (const T*)J.sc;
  const int d = J.d, overlap = J.overlap;
  const size_t row_w = (size_t)(overlap ? 2 : 1) * d;
  const T* kvb = kv + (size_t)b * L * row_w;
  const T* scb = sc + (size_t)b * L * row_w;
  const long first = g * ratio;
  const int nslot = overlap ? 2 * ratio : ratio;
  // Every load is unconditional (a masked slot reads row 0 of the buffer and
  // is then given score -inf), and the offsets are formed with selects: with
  // no branch among them the 32 loads are all in flight before the first wait.
  size_t off[16];
  bool ok[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = j0 + jj;
    const bool prev = overlap && j < ratio;  // slot of the previous group's half
    ok[jj] = j < nslot && (!prev || g != 0);  // missing previous group: weight 0
    const long tok = prev ? first - ratio + j : first + (overlap ? j - ratio : j);
    const int ch = (overlap && !prev) ? d + 2 * p : 2 * p;
    off[jj] = ok[jj] ? (size_t)(tok - p0) * row_w + ch : (size_t)ch;
  }
  float s0[16], s1[16], v0[16], v1[16];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    Elt<T>::ld2(scb, off[jj], s0[jj], s1[jj]);
    Elt<T>::ld2(kvb, off[jj], v0[jj], v1[jj]);
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    R.sv[jj][0] = ok[jj] ? s0[jj] : -INFINITY;
    R.sv[jj][1] = ok[jj] ? s1[jj] : -INFINITY;
    R.vv[jj][0] = ok[jj] ? v0[jj] : 0.f;
    R.vv[jj][1] = ok[jj] ? v1[jj] : 0.f;
  }
}

constexpr float CMP_LOG2E = 1.4426950408889634f;

// The slot softmax runs in the exp2 domain: running maxima are scores times
// log2(e), and exp2 is one hardware instruction (expf's library form costs a
// dozen and made the C128A pooling, 128 slots per channel, VALU-bound).

// Fold of 16 loaded slots into the running (max, denominator, numerator):
// the block's own max first, then its exponentials and sums in slot order,
// then one online step (no dependency chain through the max slot by slot).
__device__ __forceinline__ void compress_fold16(const PoolRegs& R, float (&mx)[2], float (&den)[2], float (&num)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float s2[16];
    float cm = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      s2[jj] = R.sv[jj][h] * CMP_LOG2E;  // -inf stays -inf
      cm = fmaxf(cm, s2[jj]);
    }
    if (cm == -INFINITY) continue;  // no slot in this block
    float cd = 0.f, cn = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float e = __builtin_amdgcn_exp2f(s2[jj] - cm);  // 0 for missing slots
      cd += e;
      cn += e * R.vv[jj][h];
    }
    if (cm > mx[h]) {
      const float r = __builtin_amdgcn_exp2f(mx[h] - cm);
      den[h] = den[h] * r + cd;
      num[h] = num[h] * r + cn;
      mx[h] = cm;
    } else {
      const float r = __builtin_amdgcn_exp2f(cm - mx[h]);
      den[h] += cd * r;
      num[h] += cn * r;
    }
  }
}

// bf16 states, 32 slots j0 .. j0+31 per round trip: the raw bf16 pairs stay
// packed in registers (one VGPR per slot and tensor) until folded, so a
// 1024-thread workgroup keeps twice the loads of compress_load16 in flight.
// Slots >= jend (or missing) are skipped.  The 32 slots are folded as one
// block (their max, then their exponentials), not slot by slot.
__device__ __forceinline__ void compress_fold32_bf16(const CompressJob& J, int b, long g, long p0, int L, int ratio,
                                                     int p, int j0, int jend, float (&mx)[2], float (&den)[2],
                                                     float (&num)[2]) {
  const bf16* __restrict__ kv = (const bf16*)J.kv;
  const bf16* __restrict__ sc = (const bf16*)J.sc;
  const int d = J.d, overlap = J.overlap;
  const size_t row_w = (size_t)(overlap ? 2 : 1) * d;
  const bf16* kvb = kv + (size_t)b * L * row_w;
  const bf16* scb = sc + (size_t)b * L * row_w;
  const int nslot = overlap ? 2 * ratio : ratio;
  // slot j reads state row r0 + j (both halves of an overlapping state use the
  // same rows: the previous group's slots are the rows before the group's own)
  const int r0 = (int)(g * ratio - (overlap ? ratio : 0) - p0);
  const int jlim = min(nslot, jend);
  const int first_ok = (overlap && g == 0) ? ratio : 0;  // missing previous group
  uint32_t kr[32], sr[32];
  bool ok[32];
#pragma unroll
  for (int jj = 0; jj < 32; ++jj) {
    const int j = j0 + jj;
    ok[jj] = j < jlim && j >= first_ok;
    const int ch = (overlap && j >= ratio) ? d + 2 * p : 2 * p;
    const uint32_t off = (uint32_t)((ok[jj] ? r0 + j : 0) * (int)row_w + ch);
    kr[jj] = *(const uint32_t*)(kvb + off);
    sr[jj] = *(const uint32_t*)(scb + off);
  }
  // the chunk's own max first (independent max ops), then its exponentials and
  // sums in slot order, then one online step into the running state: no
  // dependency chain through the running max slot by slot
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float s2[32];
    float cm = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const uint32_t u = h == 0 ? sr[jj] << 16 : sr[jj] & 0xFFFF0000u;
      s2[jj] = ok[jj] ? __uint_as_float(u) * CMP_LOG2E : -INFINITY;
      cm = fmaxf(cm, s2[jj]);
    }
    if (cm == -INFINITY) continue;  // no slot in this chunk
    float cd = 0.f, cn = 0.f;
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      const float e = __builtin_amdgcn_exp2f(s2[jj] - cm);  // 0 for missing slots
      const uint32_t u = h == 0 ? kr[jj] << 16 : kr[jj] & 0xFFFF0000u;
      cd += e;
      cn += e * __uint_as_float(u);
    }
    if (cm > mx[h]) {
      const float r = __builtin_amdgcn_exp2f(mx[h] - cm);
      den[h] = den[h] * r + cd;
      num[h] = num[h] * r + cn;
      mx[h] = cm;
    } else {
      const float r = __builtin_amdgcn_exp2f(cm - mx[h]);
      den[h] += cd * r;
      num[h] += cn * r;
    }
  }
}

// Softmax-pooled value (fp32) of channels 2p, 2p+1 of entry g of sequence b
// (2p < d).  Slots are processed in chunks of 16 whose loads are all issued
// before any of them is used, so the memory latency is paid once per chunk.
template <typename T>
__device__ __forceinline__ float2 compress_pool(const CompressJob& J, int b, long g, long p0, int L, int ratio, int p) {
  const int nslot = J.overlap ? 2 * ratio : ratio;
  float mx[2] = {-INFINITY, -INFINITY}, den[2] = {0.f, 0.f}, num[2] = {0.f, 0.f};
  for (int j0 = 0; j0 < nslot; j0 += 16) {
    PoolRegs R;
    compress_load16<T>(J, b, g, p0, L, ratio, p, j0, R);
    compress_fold16(R, mx, den, num);
  }
  return make_float2(num[0] / den[0], num[1] / den[1]);
}

// Pooled value from one loaded chunk (entries with at most 16 slots).
__device__ __forceinline__ float2 compress_pool16(const PoolRegs& R) {
  float mx[2] = {-INFINITY, -INFINITY}, den[2] = {0.f, 0.f}, num[2] = {0.f, 0.f};
  compress_fold16(R, mx, den, num);
  return make_float2(num[0] / den[0], num[1] / den[1]);
}

// RMSNorm (sum of squares `tot` over the d channels), gamma, and RoPE at the
// group's first position for the tail pairs: the stored values of pair p.
__device__ __forceinline__ float2 compress_finish(const CompressJob& J, float2 y, float tot, long g, int ratio,
                                                  float eps, double log2_base, int p, float gm0, float gm1) {
  const int d = J.d;
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  float a = y.x * inv * gm0, bb = y.y * inv * gm1;
  const int tail0 = d - J.rope_dim;
  if (2 * p >= tail0) {
    float cs, sn;
    rope_cos_sin((double)(g * ratio), p - tail0 / 2, J.rope_dim, log2_base, &cs, &sn);
    const float ra = a * cs - bb * sn, rb = a * sn + bb * cs;
    a = ra;
    bb = rb;
  }
  return make_float2(a, bb);
}

// Store the values of pair p of entry g of sequence b.  FP8 rows (J.fp8): the
// 32 threads of pairs 32c .. 32c+31 hold block c (64 dims) and sit in one
// half-wave, so the block maximum is an xor-shuffle reduction over 32 lanes;
// each thread writes its two codes, the block's first thread the exponent,
// pairs 224..255 the RoPE dims as bf16, threads 0..56 the zero tail.  The
// values are decided from the float32 results (the rounding is that of
// csa_quantize_rows).  Called by every thread of whole waves.
template <typename T>
__device__ __forceinline__ void store_entry(const CompressJob& J, int b, long g, int p, float2 v) {
  if (!J.fp8) {
    T* dst = (T*)J.cache + ((size_t)b * J.N_cap + g) * J.d;
    Elt<T>::st(dst, 2 * p, v.x);
    Elt<T>::st(dst, 2 * p + 1, v.y);
    return;
  }
  uint8_t* row = (uint8_t*)J.cache + ((size_t)b * J.N_cap + g) * FP8_ROW_BYTES;
  float amax = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (2 * p < FP8_NQ) {
    const int k = fp8_block_exp(amax);
    const uint32_t c = fp8_e4m3_rne(ldexpf(v.x, -k)) | (fp8_e4m3_rne(ldexpf(v.y, -k)) << 8);
    *(uint16_t*)(row + 2 * p) = (uint16_t)c;
    if ((p & 31) == 0) row[FP8_SCALE_OFF + (p >> 5)] = (uint8_t)(int8_t)k;
  } else {
    *(uint32_t*)(row + FP8_NQ + 4 * (p - FP8_NQ / 2)) = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  }
  if (p < FP8_ROW_BYTES - FP8_SCALE_OFF - 7) row[FP8_SCALE_OFF + 7 + p] = 0;
}

// One group of 256 consecutive threads (thread p = threadIdx.x % 256 owns
// channel pair p, d <= 512) writes entry floor(p0/ratio) + x of sequence b if
// the compressor writes it; valid == false makes the group a bystander.
// Every thread of the workgroup calls this (it contains a barrier).  The
// RMSNorm sum is reduced per wave and then over the group's 4 waves in a
// fixed order (red4: 4 floats of LDS per group); for d <= 128 only the
// group's first wave contributes and the total equals its wave_sum exactly.
template <typename T>
__device__ __forceinline__ void compress_task(const CompressJob& J, const int32_t* __restrict__ pos0, int b, int x,
                                              bool valid, int L, int ratio, float eps, double log2_base,
                                              float* red4) {
  const int p = threadIdx.x & 255;
  long g = -1, p0 = 0;
  if (valid) {
    p0 = pos0[b];
    g = compress_group(J, p0, x, L, ratio);
  }
  const bool active = g >= 0 && 2 * p < J.d;
  float gm0 = 0.f, gm1 = 0.f;
  float2 y = make_float2(0.f, 0.f);
  if (active) {
    gm0 = J.gamma[2 * p];
    gm1 = J.gamma[2 * p + 1];
    y = compress_pool<T>(J, b, g, p0, L, ratio, p);
  }
  const float ss = wave_sum(y.x * y.x + y.y * y.y);
  if ((threadIdx.x & 63) == 0) red4[p >> 6] = ss;
  __syncthreads();
  const float tot = red4[0] + red4[1] + red4[2] + red4[3];
  if (!active) return;
  const float2 v = compress_finish(J, y, tot, g, ratio, eps, log2_base, p, gm0, gm1);
  store_entry<T>(J, b, g, p, v);
}

// Wide form for entries with many slots (C128A: 128 tokens): a workgroup of
// 1024 threads, thread (p = tid % 256, q = tid / 256) folds slots q*SQ ..
// q*SQ+SQ-1 (SQ = nslot/4, in chunks of 16) of channel pair p; the four
// partial softmax states of a pair are then combined in q order through LDS
// (red: 4*256 float4 of LDS), and the first 256 threads finish the entry as
// compress_task does.  Four times the loads in flight per round trip.
template <typename T>
__device__ __forceinline__ void compress_task_wide(const CompressJob& J, const int32_t* __restrict__ pos0, int b, int x,
                                                   int L, int ratio, float eps, double log2_base, float4* red,
                                                   float* red4) {
  const int p = threadIdx.x & 255, q = threadIdx.x >> 8;
  const long p0 = pos0[b];
  const long g = compress_group(J, p0, x, L, ratio);
  if (g < 0) return;  // uniform: depends on (b, x) only
  const bool active = 2 * p < J.d;
  const int nslot = J.overlap ? 2 * ratio : ratio;
  const int sq = (nslot + 3) / 4;
  float mx[2] = {-INFINITY, -INFINITY}, den[2] = {0.f, 0.f}, num[2] = {0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
    if (active) {
      const int jend = min(nslot, (q + 1) * sq);
      for (int j0 = q * sq; j0 < jend; j0 += 32)
        compress_fold32_bf16(J, b, g, p0, L, ratio, p, j0, jend, mx, den, num);
    }
  } else if (active) {
    for (int j0 = q * sq; j0 < min(nslot, (q + 1) * sq); j0 += 16) {
      PoolRegs R;
      compress_load16<T>(J, b, g, p0, L, ratio, p, j0, R);
      // slots of the next quarter belong to another thread
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        if (j0 + jj >= (q + 1) * sq) R.sv[jj][0] = R.sv[jj][1] = -INFINITY;
      compress_fold16(R, mx, den, num);
    }
  }
  red[threadIdx.x] = make_float4(mx[0], mx[1], den[0], den[1]);
  red[1024 + threadIdx.x] = make_float4(num[0], num[1], 0.f, 0.f);
  __syncthreads();
  float2 y = make_float2(0.f, 0.f);
  if (q == 0 && active) {
    float m2[2] = {-INFINITY, -INFINITY}, d2[2] = {0.f, 0.f}, n2[2] = {0.f, 0.f};
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const float4 a = red[qq * 256 + p], c = red[1024 + qq * 256 + p];
      const float qm[2] = {a.x, a.y}, qd[2] = {a.z, a.w}, qn[2] = {c.x, c.y};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (qm[h] == -INFINITY) continue;  // no slot in this quarter
        if (qm[h] > m2[h]) {
          const float r = __builtin_amdgcn_exp2f(m2[h] - qm[h]);
          d2[h] *= r;
          n2[h] *= r;
          m2[h] = qm[h];
        }
        const float r = __builtin_amdgcn_exp2f(qm[h] - m2[h]);
        d2[h] += qd[h] * r;
        n2[h] += qn[h] * r;
      }
    }
    y = make_float2(n2[0] / d2[0], n2[1] / d2[1]);
  }
  if (q == 0) {
    const float ss = wave_sum(y.x * y.x + y.y * y.y);
    if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = ss;
  }
  __syncthreads();
  if (q != 0 || !active) return;
  const float tot = red4[0] + red4[1] + red4[2] + red4[3];
  const float2 v = compress_finish(J, y, tot, g, ratio, eps, log2_base, p, J.gamma[2 * p], J.gamma[2 * p + 1]);
  store_entry<T>(J, b, g, p, v);
}

}  // namespace csa
