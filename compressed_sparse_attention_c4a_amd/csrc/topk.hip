// topk.hip -- keep at most k compressed entries per query.
//
// "图解DeepSeek V4" section 2: the index module keeps <= topK compressed tokens;
// 2.2: it outputs their indices.  Selection rule: the min(k, visible) largest
// scores, ties to the lower entry index; outputs are a set padded with -1
// (this implementation writes the kept entries in ascending entry order).
//
// A workgroup (16 waves) selects from a chunk of CH = 1024 * KPT elements
// held in registers: wave w, slot j, lane l holds element w*64*KPT + 64*j + l,
// so element order is entry order and every load instruction reads 256
// contiguous bytes.  An MSD radix select over order-preserving 32-bit keys of
// the fp32 scores finds K*, the k-th largest key, in three digit passes (bits
// 31..20, 19..9, 8..0).  Every pass counts the keys that still match the
// digits chosen so far into an LDS histogram (4096, 2048, 512 bins; the top
// digit holds the sign, the exponent and three mantissa bits, so index scores,
// which crowd a few binades, still spread over many bins and the LDS atomics
// collide less).  Wave 0 then locates the digit where the count from the top
// reaches the number of keys still wanted: each lane sums its 1/64 of the
// bins, a DPP prefix sum over the lanes finds the lane's range, and a second
// prefix sum over that range finds the digit; meanwhile the other waves clear
// the second histogram for the next pass, so a pass costs two barriers.  Kept:
// every key > K* and the first `remaining` keys == K* in element order;
// ballots give each kept element its rank, so the output is compact and in
// entry order.
//
// Rows longer than one chunk are cut into chunks whose kept lists (k values
// and entry indices each, padded with -inf / -1) are concatenated and selected
// from again, until one chunk remains.  This is exact: an entry among the k
// best of the row (score descending, then index ascending: a total order) has
// fewer than k entries of its own chunk ahead of it, so its chunk keeps it;
// and since each chunk's list is in entry order and chunks cover ascending
// entry ranges, element order in the concatenation is still entry order, so
// ties still go to the lower entry index.
#include "compress_dev.hpp"

namespace csa {

__device__ __forceinline__ uint32_t ord_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_val(uint32_t key) {  // inverse of ord_key
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
constexpr int TOPK_BINS = 4096;

// Wave 0 only: the digit d (of 64 * PER bins, counted from the top) where the
// number of keys on digits >= d first reaches `remaining`.  Lane l sums the
// PER bins just below 64*PER - l*PER (vector LDS reads) and a DPP prefix sum
// over the lanes finds the range; then lanes 0..PER-1 take one bin each of
// that range, from its top, and a second prefix sum finds the digit.
template <int PER>
__device__ __forceinline__ void find_digit(const uint32_t* h, int lane, uint32_t prefix, int shift, int remaining,
                                           uint32_t* s_prefix, int* s_remaining, int* s_count) {
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    const uint4 x = *(const uint4*)&h[(63 - lane) * PER + 4 * i];
    c += (int)(x.x + x.y + x.z + x.w);
  }
  const int incl = wave_incl_scan(c);
  const int hl = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(incl >= remaining));  // uniform
  const int above = __builtin_amdgcn_readlane(incl - c, hl);  // keys on digits above that range
  const int d = (63 - hl) * PER + PER - 1 - lane;
  const int hc = lane < PER ? (int)h[lane < PER ? d : 0] : 0;
  const int incl2 = above + wave_incl_scan(hc);
  if (lane == (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < PER && incl2 >= remaining))) {
    *s_prefix = prefix | ((uint32_t)d << shift);
    *s_remaining = remaining - (incl2 - hc);
    *s_count = hc;
  }
}

struct TopkShared {
  uint32_t hist[2][TOPK_BINS];
  int2 s_w[TOPK_WAVES];
  int s_n[TOPK_WAVES];
  uint32_t s_prefix;
  int s_remaining;
  int s_count;  // keys on the chosen digit
};

// Histogram pass over the keys matching `prefix` under `mask`, then wave 0
// picks the digit while the other waves clear the other histogram.  PASS0:
// every valid key (key != 0) counts.
template <int KPT, bool PASS0, int NB>
__device__ __forceinline__ void radix_pass(const uint32_t (&key)[KPT], uint32_t mask, int shift, uint32_t* h,
                                           uint32_t* hn, TopkShared& sh, uint32_t prefix, int remaining) {
  constexpr uint32_t nb = NB;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (PASS0 ? key[j] != 0u : (key[j] & mask) == prefix) atomicAdd(&h[(key[j] >> shift) & (nb - 1)], 1u);
  __syncthreads();  // histogram complete
  if (wid == 0) {
    find_digit<NB / 64>(h, lane, prefix, shift, remaining, &sh.s_prefix, &sh.s_remaining, &sh.s_count);
  } else {
    for (int i = tid - 64; i < TOPK_BINS; i += TOPK_THREADS - 64) hn[i] = 0;
  }
  __syncthreads();  // digit chosen; next histogram cleared
}

// K* and `rem` such that the kk largest valid keys are every key > K* plus
// the first rem keys == K* (K* the kk-th largest key, or just below a digit
// whose keys are all taken); 1 <= kk < number of valid keys.  Invalid slots hold key 0 and
// valid keys are >= 2^21, so only the first pass tests validity: every later
// prefix has a nonzero top digit.  hist[0] must be zero and a barrier passed
// since it was cleared.  Uniform per workgroup.
template <int KPT>
__device__ __forceinline__ void radix_kth(const uint32_t (&key)[KPT], int kk, TopkShared& sh, uint32_t* kstar,
                                          int* rem) {
  // When every key on the chosen digit is wanted, the keys >= that digit's
  // lowest key are exactly the kept set: K* is set just below it and no tie
  // is ranked (later passes skipped).
  radix_pass<KPT, true, 4096>(key, 0u, 20, sh.hist[0], sh.hist[1], sh, 0u, kk);
  uint32_t prefix = sh.s_prefix;
  int remaining = sh.s_remaining;
  if (sh.s_count != remaining) {
    radix_pass<KPT, false, 2048>(key, 0xfff00000u, 9, sh.hist[1], sh.hist[0], sh, prefix, remaining);
    prefix = sh.s_prefix;
    remaining = sh.s_remaining;
    if (sh.s_count != remaining) {
      radix_pass<KPT, false, 512>(key, 0xfffffe00u, 0, sh.hist[0], sh.hist[1], sh, prefix, remaining);
      *kstar = sh.s_prefix;
      *rem = sh.s_remaining;
      return;
    }
  }
  *kstar = prefix - 1u;  // prefix >= 2^21: valid keys only
  *rem = 0;
}

__device__ __forceinline__ int wave_total(int x) {  // sum over the 64 lanes
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// Calls emit(pos, j, key) for every kept slot j of this thread, pos being its rank
// in element order among the kept elements of the chunk.  Kept: every valid
// element (key != 0) when `all`, else the keys above kstar and the first
// `rem` keys equal to kstar.  Uniform per workgroup (one barrier).
template <int KPT, class Emit>
__device__ __forceinline__ void emit_kept(const uint32_t (&key_in)[KPT], bool all, uint32_t kstar, int rem, int2* s_w,
                                          Emit emit) {
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) key[j] = key_in[j];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t gt_above = all ? 0u : kstar;  // kept without rank: key > gt_above
  const uint32_t eq_key = all ? 0u : kstar;    // ranked ties (none when all: key 0 is invalid)
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    ngt += key[j] > gt_above;
    neq += !all && key[j] == eq_key;
  }
  // the compares are cheap to redo below; without this fence the compiler
  // keeps all 2*KPT lane masks of this loop in SGPRs for the next one
#pragma unroll
  for (int j = 0; j < KPT; ++j) asm volatile("" : "+v"(key[j]));
  ngt = wave_total(ngt);
  neq = wave_total(neq);
  if (lane == 0) s_w[wid] = make_int2(ngt, neq);
  __syncthreads();
  int gb = 0, eb = 0;
#pragma unroll
  for (int w = 0; w < TOPK_WAVES; ++w) {
    const int2 x = s_w[w];
    gb += w < wid ? x.x : 0;
    eb += w < wid ? x.y : 0;
  }
  int out = gb + min(eb, rem);  // kept elements of the waves before this one
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool eq = !all && key[j] == eq_key;
    const uint64_t eqb = __builtin_amdgcn_ballot_w64(eq);
    const bool keep = key[j] > gt_above || (eq && eb + __builtin_popcountll(eqb & below) < rem);
    const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
    if (keep) emit(out + __builtin_popcountll(kb & below), j, key[j]);
    out += __builtin_popcountll(kb);
    eb += __builtin_popcountll(eqb);
  }
}

// One chunk of one query per workgroup: blockIdx.x = qi * nchunk + chunk.
// RAW: the input row is the query's scores [N_cap] (len == N_cap), valid up
// to the visible count of its position; otherwise it is a kept list [len]
// of values and entry indices from the previous round (-1 = padding).  The
// chunk's kept list (at most k, ascending entry order, padded to k with -1 /
// -inf) goes to out_idx/out_val + (qi * nchunk + chunk) * k; out_val may be
// NULL.  CMP: workgroups n_sel.. of the launch run the decode step's
// compressor tasks instead (FusedCompress, four 256-thread tasks per
// workgroup) on the CUs the top-k leaves idle; the indexer before this launch
// has already scored the new index-key entries from its own copies of them.
template <int KPT, bool RAW, bool CMP>
__global__ __launch_bounds__(TOPK_THREADS) void topk_select_kernel(const float* __restrict__ in_val,
                                                                   const int32_t* __restrict__ in_idx,
                                                                   const int32_t* __restrict__ q_pos,
                                                                   int32_t* __restrict__ out_idx,
                                                                   float* __restrict__ out_val, int len, int S, int k,
                                                                   int ratio, int nchunk, int n_sel, FusedCompress F) {
  if constexpr (CMP) {
    if ((int)blockIdx.x >= n_sel) {  // uniform per workgroup
      __shared__ float red[4][4];
      const int gq = threadIdx.x >> 8;
      const int task = ((int)blockIdx.x - n_sel) * 4 + gq;
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
  __shared__ __attribute__((aligned(16))) TopkShared sh;
  constexpr int CH = TOPK_THREADS * KPT;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qi = (int)blockIdx.x / nchunk, ch = (int)blockIdx.x - qi * nchunk;
  const size_t row = (size_t)qi * len;
  const int first = ch * CH + wid * 64 * KPT + lane;  // element of slot 0
  // loads first (clamped into the row; validity is decided separately)
  uint32_t key[KPT];
  int32_t idx[RAW ? 1 : KPT];  // entry indices of a kept-list input
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = min(first + 64 * j, len - 1);
    key[j] = ord_key(in_val[row + p]);
    if constexpr (!RAW) idx[j] = in_idx[row + p];
  }
  int limit = len;
  if (RAW) {
    const int b = qi / S, s = qi - b * S;
    limit = (int)visible_entries(q_pos[b] + s, ratio, len);
  }
  for (int i = tid; i < TOPK_BINS; i += TOPK_THREADS) sh.hist[0][i] = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {  // invalid slots: key 0; valid keys >= 2^21
    bool v = first + 64 * j < limit;
    if constexpr (!RAW) v = v && idx[j] >= 0;
    key[j] = v ? max(key[j], 1u << 21) : 0u;
    cnt += v;
  }
  cnt = wave_total(cnt);
  if (lane == 0) sh.s_n[wid] = cnt;
  __syncthreads();  // counts written; hist[0] cleared
  int n_ok = 0;
#pragma unroll
  for (int w = 0; w < TOPK_WAVES; ++w) n_ok += sh.s_n[w];
  const int kk = min(k, n_ok);
  int32_t* oi = out_idx + ((size_t)qi * nchunk + ch) * k;
  float* ov = out_val ? out_val + ((size_t)qi * nchunk + ch) * k : nullptr;
  if (kk > 0) {
    uint32_t kstar = 0;
    int rem = 0;
    const bool all = kk == n_ok;
    if (!all) radix_kth<KPT>(key, kk, sh, &kstar, &rem);
    emit_kept<KPT>(key, all, kstar, rem, sh.s_w, [&](int pos, int j, uint32_t kj) {
      if constexpr (RAW)
        oi[pos] = first + 64 * j;
      else
        oi[pos] = idx[j];
      if (ov) ov[pos] = key_val(kj);
    });
  }
  for (int j = kk + tid; j < k; j += TOPK_THREADS) {
    oi[j] = -1;
    if (ov) ov[j] = -INFINITY;
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

// Chunk size (keys per thread) and number of selection rounds for a row of n
// entries: one chunk when the row fits 32 keys per thread, else the smallest
// chunk that needs two rounds, else 32 keys per thread and as many rounds as
// it takes (each round shrinks the row by CH / k >= 2).
struct TopkPlan {
  int kpt;
  int rounds;
  int nchunk[8];  // chunks of each round
  int len[8];     // row length entering each round
};

static TopkPlan topk_plan(int N_cap, int k) {
  TopkPlan P{};
  const int kpts[3] = {8, 16, 32};
  int kpt = 32;
  if (N_cap <= TOPK_THREADS * 32) {
    for (int i = 0; i < 3; ++i)
      if (N_cap <= TOPK_THREADS * kpts[i]) {
        kpt = kpts[i];
        break;
      }
  } else {
    for (int i = 0; i < 3; ++i) {
      const long ch = (long)TOPK_THREADS * kpts[i];
      const long m = (N_cap + ch - 1) / ch * k;
      if (m <= ch) {
        kpt = kpts[i];
        break;
      }
    }
  }
  const long ch = (long)TOPK_THREADS * kpt;
  P.kpt = kpt;
  long n = N_cap;
  int r = 0;
  for (;;) {
    const int nc = (int)((n + ch - 1) / ch);
    P.len[r] = (int)n;
    P.nchunk[r] = nc;
    ++r;
    if (nc == 1) break;
    n = (long)nc * k;
  }
  P.rounds = r;
  return P;
}

// Kept lists of the intermediate rounds: two ping-pong buffers of values and
// indices, each sized for the first round's output.
size_t topk_workspace_size(int B, int S, int N_cap, int k) {
  if (B < 1 || S < 1 || N_cap < 1 || k < 1 || k > 4096) return 0;  // invalid shapes: the calls reject them
  const TopkPlan P = topk_plan(N_cap, k);
  if (P.rounds == 1) return 0;
  const size_t one = (size_t)B * S * P.nchunk[0] * k;
  return 2 * ((one * 8 + 255) & ~(size_t)255);
}

template <int KPT>
static void launch_round(bool raw, const FusedCompress* F, const float* in_val, const int32_t* in_idx,
                         const int32_t* q_pos, int32_t* oi, float* ov, int Q, int len, int S, int k, int ratio,
                         int nchunk, hipStream_t st) {
  const int n_sel = Q * nchunk;
  if (raw && F) {
    const unsigned blocks = (unsigned)(n_sel + (F->ntasks + 3) / 4);
    hipLaunchKernelGGL((topk_select_kernel<KPT, true, true>), dim3(blocks), dim3(TOPK_THREADS), 0, st, in_val, in_idx,
                       q_pos, oi, ov, len, S, k, ratio, nchunk, n_sel, *F);
  } else if (raw) {
    hipLaunchKernelGGL((topk_select_kernel<KPT, true, false>), dim3(n_sel), dim3(TOPK_THREADS), 0, st, in_val,
                       in_idx, q_pos, oi, ov, len, S, k, ratio, nchunk, n_sel, FusedCompress{});
  } else {
    hipLaunchKernelGGL((topk_select_kernel<KPT, false, false>), dim3(n_sel), dim3(TOPK_THREADS), 0, st, in_val,
                       in_idx, q_pos, oi, ov, len, S, k, ratio, nchunk, n_sel, FusedCompress{});
  }
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int32_t* idx, float* val, void* ws, int B, int S,
                       int N_cap, int k, int ratio, hipStream_t st, const FusedCompress* F) {
  const TopkPlan P = topk_plan(N_cap, k);
  const int Q = B * S;
  const size_t one = (size_t)Q * P.nchunk[0] * k;
  const size_t half = (one * 8 + 255) & ~(size_t)255;
  const float* in_val = scores;
  const int32_t* in_idx = nullptr;
  for (int r = 0; r < P.rounds; ++r) {
    const bool last = r == P.rounds - 1;
    char* buf = (char*)ws + (r & 1) * half;
    int32_t* oi = last ? idx : (int32_t*)buf;
    float* ov = last ? val : (float*)(buf + one * 4);
    const FusedCompress* f = r == 0 ? F : nullptr;
    if (P.kpt == 8)
      launch_round<8>(r == 0, f, in_val, in_idx, q_pos, oi, ov, Q, P.len[r], S, k, ratio, P.nchunk[r], st);
    else if (P.kpt == 16)
      launch_round<16>(r == 0, f, in_val, in_idx, q_pos, oi, ov, Q, P.len[r], S, k, ratio, P.nchunk[r], st);
    else
      launch_round<32>(r == 0, f, in_val, in_idx, q_pos, oi, ov, Q, P.len[r], S, k, ratio, P.nchunk[r], st);
    in_val = ov;
    in_idx = oi;
  }
  return hipGetLastError();
}

}  // namespace csa_host
