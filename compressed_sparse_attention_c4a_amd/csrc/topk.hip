// topk.hip -- keep at most k compressed entries per query.
//
// "图解DeepSeek V4" section 2: the index module keeps <= topK compressed tokens;
// 2.2: it outputs their indices.  Selection rule: the min(k, visible) largest
// scores, ties to the lower entry index; outputs are a set (any order) padded
// with -1.
//
// One workgroup (16 waves) per query runs an MSD radix select over
// order-preserving 32-bit keys of the fp32 scores: four 8-bit digit passes
// find the k-th largest key K*; one ordered pass (wave ballots + a block
// scan) then emits every key > K* and the lowest-index keys == K*, each group
// in entry order.  Keys live in LDS when a query's scores fit (<= 36864
// entries, 144 KiB), otherwise each pass re-reads the fp32 scores.
#include "common.hpp"

namespace csa {

__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_LDS_MAX = 36864;

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(TOPK_THREADS) void topk_radix_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos,
                                                                  int32_t* __restrict__ out_idx,
                                                                  float* __restrict__ out_val, int S, int N_cap,
                                                                  int k, int ratio) {
  extern __shared__ uint32_t skeys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining, s_count, s_base;
  __shared__ int wtot[TOPK_THREADS / 64], wtot_eq[TOPK_THREADS / 64];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qi = blockIdx.x;
  const int b = qi / S, s = qi % S;
  const long t = (long)q_pos[b] + s;
  const int nv = (int)visible_entries(t, ratio, N_cap);
  const float* sc = scores + (size_t)qi * N_cap;
  int32_t* oi = out_idx + (size_t)qi * k;
  float* ov = out_val ? out_val + (size_t)qi * k : nullptr;
  const int kk = k < nv ? k : nv;

  if (KEYS_IN_LDS) {
    for (int e = tid; e < nv; e += TOPK_THREADS) skeys[e] = ord_key(sc[e]);
    __syncthreads();
  }
  auto key_at = [&](int e) -> uint32_t { return KEYS_IN_LDS ? skeys[e] : ord_key(sc[e]); };

  if (kk == nv) {
    // every visible entry is kept
    for (int e = tid; e < nv; e += TOPK_THREADS) {
      oi[e] = e;
      if (ov) ov[e] = sc[e];
    }
  } else {
    uint32_t prefix = 0, mask = 0;
    int remaining = kk;  // how many of the keys matching `prefix` are still to take
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += TOPK_THREADS) hist[i] = 0;
      __syncthreads();
      for (int e = tid; e < nv; e += TOPK_THREADS) {
        const uint32_t key = key_at(e);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0, dsel = 0;
        for (int dg = 255; dg >= 0; --dg) {
          const int c = (int)hist[dg];
          if (above + c >= remaining) {
            dsel = dg;
            break;
          }
          above += c;
        }
        s_remaining = remaining - above;
        s_prefix = prefix | ((uint32_t)dsel << shift);
      }
      __syncthreads();
      remaining = s_remaining;
      prefix = s_prefix;
      mask |= 0xFFu << shift;
    }
    // prefix == K* (the k-th largest key).  Keys > K* all stay; of the keys
    // == K*, the `remaining` lowest-index ones stay.  One ordered pass writes
    // both groups in entry order, so the output is deterministic.
    const int n_gt = kk - remaining;
    if (tid == 0) {
      s_count = 0;
      s_base = 0;
    }
    __syncthreads();
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    for (int c0 = 0; c0 < nv; c0 += TOPK_THREADS) {
      const int e = c0 + tid;
      const uint32_t key = e < nv ? key_at(e) : 0u;
      const bool fg = e < nv && key > prefix;
      const bool fe = e < nv && key == prefix;
      const unsigned long long bg = __ballot(fg), be = __ballot(fe);
      if (lane == 0) {
        wtot[wid] = __popcll(bg);
        wtot_eq[wid] = __popcll(be);
      }
      __syncthreads();
      int before_g = 0, before_e = 0;
      for (int w = 0; w < wid; ++w) {
        before_g += wtot[w];
        before_e += wtot_eq[w];
      }
      const int base_g = s_count, base_e = s_base;
      if (fg) {
        const int pos = base_g + before_g + __popcll(bg & lt_mask);
        oi[pos] = e;
        if (ov) ov[pos] = sc[e];
      }
      if (fe) {
        const int r = base_e + before_e + __popcll(be & lt_mask);
        if (r < remaining) {
          oi[n_gt + r] = e;
          if (ov) ov[n_gt + r] = sc[e];
        }
      }
      __syncthreads();
      if (tid == 0) {
        int tg = 0, te = 0;
        for (int w = 0; w < TOPK_THREADS / 64; ++w) {
          tg += wtot[w];
          te += wtot_eq[w];
        }
        s_count = base_g + tg;
        s_base = base_e + te;
      }
      __syncthreads();
    }
  }
  for (int j = kk + tid; j < k; j += TOPK_THREADS) {
    oi[j] = -1;
    if (ov) ov[j] = -INFINITY;
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

size_t topk_workspace_size(int, int, int, int) { return 0; }

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int32_t* idx, float* val, void*, int B, int S,
                       int N_cap, int k, int ratio, hipStream_t st) {
  const unsigned blocks = (unsigned)(B * S);
  if (N_cap <= TOPK_LDS_MAX)
    hipLaunchKernelGGL(topk_radix_kernel<true>, dim3(blocks), dim3(TOPK_THREADS), (size_t)N_cap * 4, st, scores,
                       q_pos, idx, val, S, N_cap, k, ratio);
  else
    hipLaunchKernelGGL(topk_radix_kernel<false>, dim3(blocks), dim3(TOPK_THREADS), 0, st, scores, q_pos, idx, val,
                       S, N_cap, k, ratio);
  return hipGetLastError();
}

}  // namespace csa_host
