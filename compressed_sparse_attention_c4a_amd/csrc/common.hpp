// common.hpp -- device helpers shared by the gfx950 kernels of libcsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// bf16 is stored as its raw 16-bit pattern (the high half of an IEEE binary32).
struct bf16 {
  uint16_t x;
};

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  // two adjacent elements (i even)
  static __device__ __forceinline__ void ld2(const float* p, size_t i, float& a, float& b) {
    const float2 v = *(const float2*)(p + i);
    a = v.x;
    b = v.y;
  }
  static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <>
struct Elt<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p, size_t i) { return bf2f(p[i].x); }
  static __device__ __forceinline__ void ld2(const bf16* p, size_t i, float& a, float& b) {
    const uint32_t v = *(const uint32_t*)(p + i);
    a = __uint_as_float(v << 16);
    b = __uint_as_float(v & 0xFFFF0000u);
  }
  static __device__ __forceinline__ void st(bf16* p, size_t i, float v) { p[i].x = f2bf(v); }
};

// floor(a / b) for b > 0
__device__ __forceinline__ long floor_div(long a, long b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Number of compressed entries visible to query position t: (t+1)/ratio, clamped to [0, N_cap].
__device__ __forceinline__ long visible_entries(long t, int ratio, int N_cap) {
  long nv = floor_div(t + 1, ratio);
  if (nv < 0) nv = 0;
  if (nv > N_cap) nv = N_cap;
  return nv;
}

// RoPE rotation of interleaved pair i of a rope_dim-wide tail at position pos:
// theta = pos * base^(-2i/rope_dim), with log2_base = log2(base).  The angle
// is formed in double and reduced modulo 2*pi by a two-constant Cody-Waite
// step (|theta| < 2^31 keeps the reduction exact to ~1e-9 rad), so a float
// sine/cosine of the small remainder keeps full fp32 accuracy for positions
// up to 2^20 and beyond.
__device__ __forceinline__ void rope_cos_sin(double pos, int i, int rope_dim, double log2_base, float* c, float* s) {
  const double inv_freq = exp2(-2.0 * (double)i / (double)rope_dim * log2_base);
  const double th = pos * inv_freq;
  const double k = rint(th * 0.15915494309189535);             // th / (2 pi)
  double r = fma(-k, 6.283185307179586, th);                    // 2 pi, leading part
  r = fma(-k, 2.4492935982947064e-16, r);                       // 2 pi, trailing part
  sincosf((float)r, s, c);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block L -> XCD L % 8),
// each with its own L2.  This bijection on [0, total) gives every XCD one
// contiguous range of work items, so items that share data (e.g. the head
// groups of one query) run under the same L2.
__device__ __forceinline__ int xcd_remap(int L, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = L % 8, j = L / 8;
  return x * per + (x < rem ? x : rem) + j;
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies (gfx950 global_load_lds_dwordx4): each lane's 16
// bytes land at lds_wave_base + 16 * lane.  The copy is issued from inline asm
// on purpose: the compiler's wait-count pass cannot tell which LDS buffer an
// in-flight copy targets and would otherwise put vmcnt(0) before unrelated LDS
// reads, draining every prefetch.  The asm writes no VGPR (its destination is
// LDS through M0, saved and restored here), so nothing in a register can be
// overwritten while the copy is in flight.  Callers wait for completion with
// WAIT_VMCNT before reading the data; compiler-inserted waits for ordinary
// loads stay correct because unseen copies only make them stricter.
__device__ __forceinline__ void dma16(const void* gaddr, const void* lds_wave_base) {
  // the LDS base is wave-uniform by contract; readfirstlane puts it in an SGPR for M0
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)lds_wave_base));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(m)
      : "memory");
}

// Same copy with a wave-uniform 64-bit base (SGPRs) and a per-lane 32-bit
// byte offset: no per-lane address arithmetic at the call site.
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t lane_off, const void* lds_wave_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) void*)lds_wave_base));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(lane_off), "s"(sbase), "s"(m)
      : "memory");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0], expcnt
// [6:4] = 7, lgkmcnt [11:8] = 15, vmcnt[5:4] in [15:14]).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n)&15) | (((n) >> 4) << 14)) | 0x0F70)

// s_waitcnt vmcnt(n) for a run-time n in [0, 30] (the count is an immediate;
// larger n waits for everything).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define IX_W(k) \
  case k:       \
    WAIT_VMCNT(k); \
    break;
    IX_W(0) IX_W(1) IX_W(2) IX_W(3) IX_W(4) IX_W(5) IX_W(6) IX_W(7) IX_W(8) IX_W(9) IX_W(10) IX_W(11) IX_W(12)
    IX_W(13) IX_W(14) IX_W(15) IX_W(16) IX_W(17) IX_W(18) IX_W(19) IX_W(20) IX_W(21) IX_W(22) IX_W(23) IX_W(24)
    IX_W(25) IX_W(26) IX_W(27) IX_W(28) IX_W(29) IX_W(30)
#undef IX_W
    default:
      WAIT_VMCNT(0);
  }
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads/writes are
// complete (lgkmcnt 0) and the compiler may not move memory accesses across
// it.  Copies in flight are not waited for (explicit vmcnt waits track them);
// __syncthreads() would drain them through its release fence.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// FP8 KV rows ("图解DeepSeek V4" 2: the non-RoPE part of a KV row is quantised).
// D = 512 values: bytes [0, 448) OCP E4M3 codes of the first 448 dims, one
// power-of-two scale 2^k per 64-dim block; [448, 576) the 64 RoPE dims as bf16;
// [576, 583) the 7 exponents k as int8; [583, 640) zero.
constexpr int FP8_ROW_BYTES = 640;
constexpr int FP8_NQ = 448;       // quantised dims
constexpr int FP8_SCALE_OFF = 576;

// Smallest k with amax <= 448 * 2^k (0 for amax == 0), clamped to [-120, 120].
// With amax in [2^(E-1), 2^E) the answer is E - 9 when amax <= 448 * 2^(E-9)
// (= 0.875 * 2^E) and E - 8 otherwise.
__device__ __forceinline__ int fp8_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  (void)frexpf(amax, &E);
  const int k = (amax <= ldexpf(448.f, E - 9)) ? E - 9 : E - 8;
  return k < -120 ? -120 : (k > 120 ? 120 : k);
}

// E4M3 code of v (|v| <= 448): the nearest E4M3 value, ties to the even code.
// Below 2^-6 the spacing is 2^-9 (codes 0..8, 8 being 2^-6); a value in
// [2^e, 2^(e+1)) rounds its 3 mantissa bits.  The sign bit is v's own.
__device__ __forceinline__ uint32_t fp8_e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);
  int E;
  (void)frexpf(a, &E);
  int e = E - 1;
  int mant = (int)rintf((ldexpf(a, -e) - 1.f) * 8.f);
  if (mant == 8) {
    e += 1;
    mant = 0;
  }
  return sign | ((uint32_t)(e + 7) << 3) | (uint32_t)mant;
}

// bf16 pair of the E4M3 codes in bits [0, 16) times 2^k (k in [-120, 120]):
// exact (a value has at most 4 significant bits), one scaled conversion.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8_pair_to_bf16x2(uint32_t two_codes, int k) {
  const float scale = __uint_as_float((uint32_t)(k + 127) << 23);  // 2^k
  const bf16x2v_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)two_codes, scale, false);
  return __builtin_bit_cast(uint32_t, r);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): shifts by 1, 2, 4, 8 inside each 16-lane row, then row 15
// into rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sum of x over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48),
// returned in every lane: two gfx950 permlane swaps, no LDS round trip.
__device__ __forceinline__ float row_sum4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0<->1, 2<->3
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t uy = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(uy, uy, false, false);  // halves
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace csa

namespace csa {
// One compression job (see compress.hip).
struct CompressJob {
  const void* kv;
  const void* sc;
  const float* gamma;
  void* cache;
  int d, rope_dim, overlap, N_cap;
  int fp8;  // 1: cache rows in the FP8 row format (d == 512, rope_dim == 64)
};

// Both compressors of a CSA decode step folded into the indexer and top-k
// launches (see index.hip and topk.hip): j0 main KV, j1 index keys (j1.cache
// is the index cache); gx group candidates per sequence, ntasks = 2*gx*B.
struct FusedCompress {
  CompressJob j0, j1;
  const int32_t* pos0;
  int L, gx, B, ntasks;
  float eps;
  double log2_base;
};
}  // namespace csa

// Host-side launch helpers implemented per kernel file; called from abi.cpp.
namespace csa_host {
// Groups g = floor(p0 / ratio) + x that can be complete inside a buffer of L
// tokens starting at p0: with p0 = a*ratio + b and L = c*ratio + e (0 <= b, e
// < ratio) the last complete group is floor((p0 + L) / ratio) - 1, so x <=
// c + floor((b + e) / ratio) - 1 <= ceil(L / ratio) - 1.
inline int compress_gx(int L, int ratio) { return (L + ratio - 1) / ratio; }
hipError_t launch_compress(const csa::CompressJob* jobs, int njobs, const int32_t* pos0, int B, int L, int ratio,
                           float eps, float base, int dtype, hipStream_t st);
hipError_t launch_index_scores(const void* q, const float* w, const void* K, const int32_t* q_pos, float* scores,
                               int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags, int dtype,
                               hipStream_t st);
bool fused_compress_ok(const csa::FusedCompress& F, int S, int Hi, int di, int N_cap, int ratio, int dtype);
hipError_t launch_index_scores_fused(const csa::FusedCompress& F, const void* q, const float* w,
                                     const int32_t* q_pos, float* scores, int B, int S, int Hi, int N_cap, int ratio,
                                     unsigned flags, hipStream_t st);
size_t topk_workspace_size(int B, int S, int N_cap, int k);
hipError_t launch_topk(const float* scores, const int32_t* q_pos, int32_t* idx, float* val, void* ws, int B, int S,
                       int N_cap, int k, int ratio, hipStream_t st, const csa::FusedCompress* F = nullptr);
size_t attn_workspace_size(int B, int S, int H, int D, long n_cand);
hipError_t launch_attn(const void* q, const void* cmp, const int32_t* topk_idx, int k, int dense, int ratio,
                       const void* win,
                       const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                       void* ws, int B, int S, int H, int D, int rope_dim, int N_cap, int W_cap, int window,
                       float scale, float base, int dtype, hipStream_t st);
hipError_t launch_quantize_rows(const void* src, void* dst, long rows, hipStream_t st);
hipError_t launch_dequantize_rows(const void* src, void* dst, long rows, hipStream_t st);
size_t gemm_partial_bytes(int groups, int M, int N, int K);
hipError_t launch_gemm_nt(const void* A, const void* Bp, float* C, int groups, int M, int N, int K, int lda, long sa,
                          long sb, int* ksplit_out, hipStream_t st);
hipError_t launch_pack_weights(const void* W, void* P, int groups, int N, int K, hipStream_t st);
hipError_t launch_rows_finish(const float* part, void* out, const float* gamma, const int32_t* pos, int M, int ncols,
                              int gcols, int seg, int ksplit, int norm, int rope_dim, int S, float eps, float base,
                              hipStream_t st);
}  // namespace csa_host
