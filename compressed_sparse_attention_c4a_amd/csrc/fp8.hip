// fp8.hip -- conversion of bf16 KV rows (D = 512, RoPE on the last 64 dims)
// to and from the FP8 row format ("图解DeepSeek V4：详细计算流程解析" 2: the
// rope_head_dim part of a KV row is rotated, the rest is quantised).  The format
// and the rounding are defined with the helpers in common.hpp.
//
// One wave per row.  Lane l < 56 owns dims 8l .. 8l+7 (block l / 8 of 64
// dims), lane l >= 56 the bf16 RoPE dims 448 + 8(l - 56) .. +8.  The block
// maximum is reduced over the block's 8 lanes with xor shuffles.
#include "common.hpp"

namespace csa {

constexpr int FQ_WAVES = 4;

__global__ __launch_bounds__(64 * FQ_WAVES) void quantize_rows_kernel(const bf16* __restrict__ src,
                                                                      uint8_t* __restrict__ dst, long rows) {
  const long r = (long)blockIdx.x * FQ_WAVES + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const uint4 raw = *(const uint4*)(src + (size_t)r * 512 + 8 * lane);
  uint8_t* row = dst + (size_t)r * FP8_ROW_BYTES;
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  const int k = fp8_block_exp(amax);
  if (lane < 56) {
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i >> 2] |= fp8_e4m3_rne(ldexpf(v[i], -k)) << (8 * (i & 3));
    *(uint2*)(row + 8 * lane) = make_uint2(c[0], c[1]);
  } else {
    *(uint4*)(row + FP8_NQ + 16 * (lane - 56)) = raw;
  }
  // exponents of the 7 blocks (lane 8b holds block b's) and the zero tail
  uint32_t s0 = 0u, s1 = 0u;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint32_t kb = (uint32_t)(uint8_t)(int8_t)__builtin_amdgcn_readlane(k, 8 * b);
    if (b < 4) s0 |= kb << (8 * b);
    else s1 |= kb << (8 * (b - 4));
  }
  if (lane == 0) *(uint2*)(row + FP8_SCALE_OFF) = make_uint2(s0, s1);
  if (lane >= 1 && lane <= 7) *(uint2*)(row + FP8_SCALE_OFF + 8 * lane) = make_uint2(0u, 0u);
}

__global__ __launch_bounds__(64 * FQ_WAVES) void dequantize_rows_kernel(const uint8_t* __restrict__ src,
                                                                        bf16* __restrict__ dst, long rows) {
  const long r = (long)blockIdx.x * FQ_WAVES + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const uint8_t* row = src + (size_t)r * FP8_ROW_BYTES;
  uint4 out;
  if (lane < 56) {
    const uint2 c = *(const uint2*)(row + 8 * lane);
    const int k = (int)(int8_t)row[FP8_SCALE_OFF + (lane >> 3)];
    out.x = fp8_pair_to_bf16x2(c.x & 0xFFFFu, k);
    out.y = fp8_pair_to_bf16x2(c.x >> 16, k);
    out.z = fp8_pair_to_bf16x2(c.y & 0xFFFFu, k);
    out.w = fp8_pair_to_bf16x2(c.y >> 16, k);
  } else {
    out = *(const uint4*)(row + FP8_NQ + 16 * (lane - 56));
  }
  *(uint4*)(dst + (size_t)r * 512 + 8 * lane) = out;
}

}  // namespace csa

namespace csa_host {
using namespace csa;

hipError_t launch_quantize_rows(const void* src, void* dst, long rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((rows + FQ_WAVES - 1) / FQ_WAVES)), dim3(64 * FQ_WAVES), 0,
                     st, (const bf16*)src, (uint8_t*)dst, rows);
  return hipGetLastError();
}

hipError_t launch_dequantize_rows(const void* src, void* dst, long rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_rows_kernel, dim3((unsigned)((rows + FQ_WAVES - 1) / FQ_WAVES)), dim3(64 * FQ_WAVES),
                     0, st, (const uint8_t*)src, (bf16*)dst, rows);
  return hipGetLastError();
}

}  // namespace csa_host
