// topk.hip -- keep at most k compressed entries per query.
//
// "图解DeepSeek V4" section 2: the index module keeps <= topK compressed tokens;
// 2.2: it outputs their indices.  Selection rule: the min(k, visible) largest
// scores, ties to the lower entry index; outputs are a set padded with -1.
//
// One workgroup (16 waves) per query runs an MSD radix select over
// order-preserving 32-bit keys of the fp32 scores.  Four 8-bit digit passes
// find K*, the k-th largest key: every wave counts into its own 256-bin LDS
// histogram (atomics only contend inside a wave), the 16 histograms are
// summed per bin and a parallel suffix scan over the bins picks the digit
// where the running count reaches the number of keys still wanted.  One
// ordered pass then keeps every key > K* and the lowest-index keys == K*:
// thread t owns a contiguous run of entries, so a single block-wide scan of
// per-thread counts gives every kept entry its output slot (entry order,
// deterministic).  Keys live in LDS when a query's scores fit (<= 32768
// entries); otherwise each pass re-reads the fp32 scores.
#include "common.hpp"

namespace csa {

__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
constexpr int TOPK_LDS_MAX = 32768;

// Inclusive prefix sum over the 1024 threads; returns it and sets *total.
__device__ __forceinline__ int block_inclusive_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_w[wid] = v;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TOPK_WAVES; ++w) {
    const int x = s_w[w];
    before += (w < wid) ? x : 0;
    tot += x;
  }
  __syncthreads();  // s_w may be reused by the caller
  *total = tot;
  return v + before;
}

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(TOPK_THREADS) void topk_radix_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos,
                                                                  int32_t* __restrict__ out_idx,
                                                                  float* __restrict__ out_val, int S, int N_cap,
                                                                  int k, int ratio) {
  extern __shared__ uint32_t skeys[];
  __shared__ uint32_t whist[TOPK_WAVES][256];
  __shared__ int s_w[TOPK_WAVES];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;

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
    for (int e = tid; e < nv; e += TOPK_THREADS) {  // every visible entry is kept
      oi[e] = e;
      if (ov) ov[e] = sc[e];
    }
  } else {
    uint32_t prefix = 0, mask = 0;
    int remaining = kk;  // keys matching `prefix` still to take
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = lane; i < 256; i += 64) whist[wid][i] = 0;
      __syncthreads();
      for (int e = tid; e < nv; e += TOPK_THREADS) {
        const uint32_t key = key_at(e);
        if ((key & mask) == prefix) atomicAdd(&whist[wid][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // thread r < 256 handles digit 255 - r: suffix counts from the top digit
      int cnt = 0;
      if (tid < 256) {
#pragma unroll
        for (int w = 0; w < TOPK_WAVES; ++w) cnt += (int)whist[w][255 - tid];
      }
      int tot;
      const int incl = block_inclusive_scan(tid < 256 ? cnt : 0, s_w, &tot);
      if (tid < 256 && incl >= remaining && incl - cnt < remaining) {  // exactly one digit
        s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
        s_remaining = remaining - (incl - cnt);
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      mask |= 0xFFu << shift;
    }
    // prefix == K*.  Keys > K* all stay; of the keys == K*, the `remaining`
    // lowest-index ones stay.  Thread tid owns entries [e0, e1).
    const int per = (nv + TOPK_THREADS - 1) / TOPK_THREADS;
    const int e0 = min(nv, tid * per), e1 = min(nv, e0 + per);
    int ngt = 0, neq = 0;
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = key_at(e);
      ngt += key > prefix;
      neq += key == prefix;
    }
    int tot_gt, tot_eq;
    const int gt_before = block_inclusive_scan(ngt, s_w, &tot_gt) - ngt;
    const int eq_before = block_inclusive_scan(neq, s_w, &tot_eq) - neq;
    const int n_gt = kk - remaining;  // == tot_gt
    int pg = gt_before, pe = eq_before;
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = key_at(e);
      if (key > prefix) {
        oi[pg] = e;
        if (ov) ov[pg] = sc[e];
        ++pg;
      } else if (key == prefix) {
        if (pe < remaining) {
          oi[n_gt + pe] = e;
          if (ov) ov[n_gt + pe] = sc[e];
        }
        ++pe;
      }
    }
    (void)tot_gt;
    (void)tot_eq;
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
