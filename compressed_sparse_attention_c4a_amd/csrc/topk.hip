// topk.hip -- keep at most k compressed entries per query.
//
// "图解DeepSeek V4" section 2: the index module keeps <= topK compressed tokens;
// 2.2: it outputs their indices.  Selection rule: the min(k, visible) largest
// scores, ties to the lower entry index; outputs are a set padded with -1.
//
// One workgroup (16 waves) per query runs an MSD radix select over
// order-preserving 32-bit keys of the fp32 scores.  Three digit passes (bits
// 31..21, 20..10, 9..0) find K*, the k-th largest key.  Every pass counts the
// keys that still match the digits chosen so far into an LDS histogram (2048
// bins; the top digit holds the sign, the exponent and two mantissa bits, so
// even the first pass spreads real score distributions over many bins and the
// LDS atomics rarely collide).  Wave 0 then locates the digit where the count
// from the top reaches the number of keys still wanted: each lane sums 32
// bins, a DPP prefix sum over the lanes finds the lane, and that lane walks
// its bins; meanwhile the other waves clear the second histogram for the next
// pass, so a pass costs two barriers.  Keys stay in registers (8 or 32 per
// thread) when a query's scores fit, else every pass re-reads them.  Output:
// every key > K* and the lowest-index keys == K*; thread t owns entries t,
// t + 1024, ... and one block-wide scan of per-thread counts gives each kept
// entry its slot (deterministic).  When more keys equal K* than slots remain
// (ties across the k-th score), the ties are taken in entry order by a second,
// contiguous pass.
#include "compress_dev.hpp"

namespace csa {

__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
constexpr int TOPK_BINS = 2048;

// Block-wide exclusive prefix sums of two per-thread counts (1024 threads);
// totals in *ta, *tb.  Ends with a barrier, so s_w can be reused at once.
__device__ __forceinline__ void block_excl_scan2(int a, int b, int2* s_w, int* ea, int* eb, int* ta, int* tb) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) s_w[wid] = make_int2(ia, ib);
  __syncthreads();
  int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < TOPK_WAVES; ++w) {
    const int2 x = s_w[w];
    pa += (w < wid) ? x.x : 0;
    pb += (w < wid) ? x.y : 0;
    sa += x.x;
    sb += x.y;
  }
  __syncthreads();
  *ea = pa + ia - a;
  *eb = pb + ib - b;
  *ta = sa;
  *tb = sb;
}

// Wave 0 only: the digit d (of 64 * PER bins, counted from the top) where the
// number of keys on digits >= d first reaches `remaining`.  Lane l holds the
// PER bins just below 64*PER - l*PER in registers (vector LDS reads), a DPP
// prefix sum over the lanes finds the lane, and that lane walks its bins.
template <int PER>
__device__ __forceinline__ void find_digit(const uint32_t* h, int lane, uint32_t prefix, int shift, int remaining,
                                           uint32_t* s_prefix, int* s_remaining) {
  const int bottom = (63 - lane) * PER;  // lowest digit of this lane's range
  uint32_t v[PER];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const uint4 x = *(const uint4*)&h[bottom + 4 * i];
    v[4 * i] = x.x;
    v[4 * i + 1] = x.y;
    v[4 * i + 2] = x.z;
    v[4 * i + 3] = x.w;
  }
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) c += (int)v[i];
  const int incl = wave_incl_scan(c);
  const uint64_t hit = __builtin_amdgcn_ballot_w64(incl >= remaining);
  if (lane == (int)__builtin_ctzll(hit)) {  // first lane whose range reaches `remaining`
    int before = incl - c;
    int d = bottom;  // reached by the counts; the default only guards the walk
    bool found = false;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      const int hc = (int)v[i];
      if (!found && before + hc >= remaining) {
        d = bottom + i;
        found = true;
      }
      if (!found) before += hc;
    }
    *s_prefix = prefix | ((uint32_t)d << shift);
    *s_remaining = remaining - before;
  }
}

// KPT > 0: each thread holds the keys of entries tid + 1024*j, j < KPT, in
// registers (requires N_cap <= 1024 * KPT); KPT == 0: keys are re-read.
// CMP: workgroups n_topk.. of the launch run the decode step's compressor
// tasks instead (FusedCompress, four 256-thread tasks per workgroup) on the
// CUs the top-k leaves idle; the indexer before this launch has already
// scored the new index-key entries from its own copies of them.
template <int KPT, bool CMP>
__global__ __launch_bounds__(TOPK_THREADS) void topk_radix_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos,
                                                                  int32_t* __restrict__ out_idx,
                                                                  float* __restrict__ out_val, int S, int N_cap,
                                                                  int k, int ratio, int n_topk, FusedCompress F) {
  if constexpr (CMP) {
    if ((int)blockIdx.x >= n_topk) {  // uniform per workgroup
      __shared__ float red[4][4];
      const int gq = threadIdx.x >> 8;
      const int task = ((int)blockIdx.x - n_topk) * 4 + gq;
      const bool valid = task < F.ntasks;
      int z = 0, bb = 0, x = 0;
      if (valid) {
        z = task / (F.gx * F.B);
        const int rem = task % (F.gx * F.B);
        bb = rem / F.gx;
        x = rem % F.gx;
      }
      compress_task<bf16>(z == 0 ? F.j0 : F.j1, F.pos0, bb, x, valid, F.L, ratio, F.eps, F.log2_base, red[gq]);
      return;
    }
  }
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][TOPK_BINS];
  __shared__ int2 s_w[TOPK_WAVES];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qi = blockIdx.x;
  const float* sc = scores + (size_t)qi * N_cap;
  constexpr int KR = KPT > 0 ? KPT : 1;
  // the score loads do not wait for the position: entries past the visible
  // range are masked below
  float kf[KR];
  if (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int e = tid + TOPK_THREADS * j;
      kf[j] = e < N_cap ? sc[e] : 0.f;
    }
  }
  const int b = qi / S, s = qi % S;
  const int t = q_pos[b] + s;
  const int nv = (int)visible_entries(t, ratio, N_cap);
  int32_t* oi = out_idx + (size_t)qi * k;
  float* ov = out_val ? out_val + (size_t)qi * k : nullptr;
  const int kk = k < nv ? k : nv;
  uint32_t key[KR];
#pragma unroll
  for (int j = 0; j < KR; ++j) key[j] = ord_key(kf[j]);
  for (int i = tid; i < TOPK_BINS; i += TOPK_THREADS) hist[0][i] = 0;

  if (kk == nv) {
    for (int e = tid; e < nv; e += TOPK_THREADS) {  // every visible entry is kept
      oi[e] = e;
      if (ov) ov[e] = sc[e];
    }
  } else if (kk > 0) {
    uint32_t prefix = 0, mask = 0;
    int remaining = kk;  // keys matching `prefix` still to take
    __syncthreads();     // hist[0] cleared
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t nb = pass == 2 ? 1024u : 2048u;
      uint32_t* h = hist[pass & 1];
      if (KPT > 0) {
#pragma unroll
        for (int j = 0; j < KR; ++j) {
          const int e = tid + TOPK_THREADS * j;
          if (e < nv && (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> shift) & (nb - 1)], 1u);
        }
      } else {
        for (int e = tid; e < nv; e += TOPK_THREADS) {
          const uint32_t kv = ord_key(sc[e]);
          if ((kv & mask) == prefix) atomicAdd(&h[(kv >> shift) & (nb - 1)], 1u);
        }
      }
      __syncthreads();  // histogram complete
      if (wid == 0) {
        if (nb == 2048)
          find_digit<32>(h, lane, prefix, shift, remaining, &s_prefix, &s_remaining);
        else
          find_digit<16>(h, lane, prefix, shift, remaining, &s_prefix, &s_remaining);
      } else {
        uint32_t* hn = hist[(pass + 1) & 1];
        for (int i = tid - 64; i < TOPK_BINS; i += TOPK_THREADS - 64) hn[i] = 0;
      }
      __syncthreads();  // digit chosen; next histogram cleared
      prefix = s_prefix;
      remaining = s_remaining;
      mask |= (nb - 1) << shift;
    }
    // prefix == K*.  Keys > K* all stay (n_gt of them); of the keys == K*,
    // the `remaining` lowest-index ones stay.
    int ngt = 0, neq = 0;
    if (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        const int e = tid + TOPK_THREADS * j;
        ngt += (e < nv && key[j] > prefix) ? 1 : 0;
        neq += (e < nv && key[j] == prefix) ? 1 : 0;
      }
    } else {
      for (int e = tid; e < nv; e += TOPK_THREADS) {
        const uint32_t kv = ord_key(sc[e]);
        ngt += kv > prefix;
        neq += kv == prefix;
      }
    }
    int gt_before, eq_before, tot_gt, tot_eq;
    block_excl_scan2(ngt, neq, s_w, &gt_before, &eq_before, &tot_gt, &tot_eq);
    const int n_gt = kk - remaining;  // == tot_gt
    const bool all_ties = tot_eq == remaining;
    int pg = gt_before, pe = n_gt + eq_before;
    if (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        const int e = tid + TOPK_THREADS * j;
        if (e < nv) {
          if (key[j] > prefix) {
            oi[pg] = e;
            if (ov) ov[pg] = kf[j];
            ++pg;
          } else if (all_ties && key[j] == prefix) {
            oi[pe] = e;
            if (ov) ov[pe] = kf[j];
            ++pe;
          }
        }
      }
    } else {
      for (int e = tid; e < nv; e += TOPK_THREADS) {
        const float f = sc[e];
        const uint32_t kv = ord_key(f);
        if (kv > prefix) {
          oi[pg] = e;
          if (ov) ov[pg] = f;
          ++pg;
        } else if (all_ties && kv == prefix) {
          oi[pe] = e;
          if (ov) ov[pe] = f;
          ++pe;
        }
      }
    }
    if (!all_ties) {
      // ties straddle the k-th score: the lowest-index `remaining` of them, in
      // entry order (thread tid owns the contiguous run [e0, e1))
      const int per = (nv + TOPK_THREADS - 1) / TOPK_THREADS;
      const int e0 = min(nv, tid * per), e1 = min(nv, e0 + per);
      int cnt = 0;
      for (int e = e0; e < e1; ++e) cnt += ord_key(sc[e]) == prefix;
      int q, unused0, unused1, unused2;
      block_excl_scan2(cnt, 0, s_w, &q, &unused0, &unused1, &unused2);
      for (int e = e0; e < e1 && q < remaining; ++e) {
        const float f = sc[e];
        if (ord_key(f) == prefix) {
          oi[n_gt + q] = e;
          if (ov) ov[n_gt + q] = f;
          ++q;
        }
      }
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

template <int KPT>
static void launch_topk_kpt(const float* scores, const int32_t* q_pos, int32_t* idx, float* val, int B, int S,
                            int N_cap, int k, int ratio, hipStream_t st, const FusedCompress* F) {
  const int n_topk = B * S;
  if (F) {
    const unsigned blocks = (unsigned)(n_topk + (F->ntasks + 3) / 4);
    hipLaunchKernelGGL((topk_radix_kernel<KPT, true>), dim3(blocks), dim3(TOPK_THREADS), 0, st, scores, q_pos, idx,
                       val, S, N_cap, k, ratio, n_topk, *F);
  } else {
    hipLaunchKernelGGL((topk_radix_kernel<KPT, false>), dim3(n_topk), dim3(TOPK_THREADS), 0, st, scores, q_pos, idx,
                       val, S, N_cap, k, ratio, n_topk, FusedCompress{});
  }
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int32_t* idx, float* val, void*, int B, int S,
                       int N_cap, int k, int ratio, hipStream_t st, const FusedCompress* F) {
  if (N_cap <= 8 * TOPK_THREADS)
    launch_topk_kpt<8>(scores, q_pos, idx, val, B, S, N_cap, k, ratio, st, F);
  else if (N_cap <= 32 * TOPK_THREADS)
    launch_topk_kpt<32>(scores, q_pos, idx, val, B, S, N_cap, k, ratio, st, F);
  else
    launch_topk_kpt<0>(scores, q_pos, idx, val, B, S, N_cap, k, ratio, st, F);
  return hipGetLastError();
}

}  // namespace csa_host
