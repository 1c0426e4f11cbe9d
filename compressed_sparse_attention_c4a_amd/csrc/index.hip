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
#include "compress_dev.hpp"

#include <cmath>

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

// ---------------------------------------------------------------------------
// MFMA kernel (bf16, di == 128, Hi == 16*MT).  HBM-bound streaming of the
// index cache: every candidate row (256 B) is read once per query.
//
// Workgroup = 4 waves (one per CU: ~256 workgroups), one query, a chunk of
// 4*T tiles of 32 candidates (tiles interleaved across the waves so the group
// streams contiguous rows).  Per wave and tile: 8 direct global->LDS copies
// (1 KiB each, 4 rows) into a private ring of IX_NB tiles, IX_NB-1 tiles in
// flight while one is scored.  Scores: v_mfma_f32_16x16x32_bf16 with A =
// q_idx (M = 16 heads, K = 32 dims, kept in VGPRs for the whole kernel) and
// B = k^T from LDS (N = 16 candidates); C lane l holds heads 4*(l/16)+i of
// candidate l%16, so the ReLU * w head reduction is in-lane over 4*MT values
// plus two cross-lane steps.  LDS rows are XOR-swizzled (16-byte granule c of
// row r sits at c ^ (r & 15)) so the rows a quarter-wave reads fall in
// distinct banks.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int IX_TILE = 32;           // candidates per wave tile
constexpr int IX_WAVES = 4;
constexpr int IX_NB = 4;              // tiles per wave ring
constexpr int IX_ROW = 256;           // bytes per index row (128 bf16)
constexpr int IX_TILE_BYTES = IX_TILE * IX_ROW;
constexpr int IX_COPIES = IX_TILE_BYTES / 1024;  // 1 KiB copies per tile and wave
#ifndef IX_MQW
#define IX_MQW 8                      // queries (waves) per workgroup of the multi-query form
#endif

// Fused compressors (decode, FUSED): the wave whose tile holds an index-key
// entry this step writes computes that entry itself (the compressor's own
// routines, so the same values) and puts it into its LDS tile before scoring
// it: no workgroup waits for the compressor.  The entries are written to the
// caches by the top-k launch that follows (topk.hip).  Requires S == 1, an
// overlapping index-key compressor and a state of at most 2*ratio <= 16
// tokens, so every entry has at most 16 slots.  Such a state completes one
// entry g > 0 at most (it needs all 2*ratio tokens); only a state that starts
// at position 0 also completes entry 0, which has no previous group.  Entries
// 0 and 1 are rows 0 and 1 of the first tile of the first chunk, so one wave
// holds both: the later entry is computed when its tile is scored, as usual;
// the other (this rare case only) is computed during the set-up.
template <int MT, bool FUSED>
__global__ __launch_bounds__(256) void index_scores_mfma(const bf16* __restrict__ q, const float* __restrict__ w,
                                                         const bf16* __restrict__ K,
                                                         const int32_t* __restrict__ q_pos,
                                                         float* __restrict__ scores, int S, int N_cap, int ratio,
                                                         unsigned flags, int T, int chunks, FusedCompress F) {
  constexpr int HI = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[HI * IX_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[IX_WAVES][IX_NB][IX_TILE_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  {
    const int qi = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
    const int b = qi / S, s = qi % S;
    const long t = (long)q_pos[b] + s;
    // the state position: a vector load (vmcnt, in order) issued before the
    // copies, so waiting for it never delays them and it lands with them
    [[maybe_unused]] int pos0v = 0;
    if constexpr (FUSED) pos0v = __builtin_nontemporal_load(F.pos0 + b);
    const int nv = (int)visible_entries(t, ratio, N_cap);
    const int g = lane >> 4, n = lane & 15;
    const int e_chunk = chunk * IX_WAVES * T * IX_TILE;
    float* out = scores + (size_t)qi * N_cap;
    const bf16* Kb = K + (size_t)b * N_cap * 128;

    auto tile_e0 = [&](int i) { return e_chunk + (i * IX_WAVES + wave) * IX_TILE; };
    // tiles of this wave that hold visible candidates: i < nt
    int nt = 0;
    {
      const int first = tile_e0(0);
      if (first < nv) nt = min(T, (nv - first + IX_WAVES * IX_TILE - 1) / (IX_WAVES * IX_TILE));
    }
    auto issue = [&](int i) {
      const int e0 = tile_e0(i);
#pragma unroll
      for (int j = 0; j < IX_COPIES; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        int e = e0 + r;
        e = e < nv ? e : nv - 1;  // rows past the visible range reload a valid row (masked below)
        dma16(Kb + (size_t)e * 128 + 8 * c, &lds_k[wave][i % IX_NB][j * 1024]);
      }
    };
    // Set-up in one memory round trip: w into registers, q_idx (swizzled rows)
    // and the first IX_NB-1 tiles into LDS by direct copies, then one wait.
    float wv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[mt][i] = w[(size_t)qi * HI + 16 * mt + 4 * g + i];
    {
      const bf16* qb = q + (size_t)qi * HI * 128;
      for (int j = wave; j < HI / 4; j += IX_WAVES) {  // 1 KiB = 4 q rows per copy
        const int r = 4 * j + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        dma16(qb + (size_t)r * 128 + 8 * c, lds_q + j * 1024);
      }
    }
    for (int i = 0; i < IX_NB - 1 && i < nt; ++i) issue(i);
    // (an empty asm the position passes through: nothing that depends on it
    // is hoisted above the copies, so its wait cannot delay them)
    if constexpr (FUSED) __asm__ volatile("" : "+s"(pos0v));
    [[maybe_unused]] const long pp0 = pos0v;
    // Fused: the index-key entry written this step, if it is visible and in
    // one of this wave's tiles (tile pi, row pr): its slots are loaded now,
    // its value is computed when that tile is scored.
    // (pi2, pr2): a second entry of this wave (entry 0 of a state that starts
    // at position 0), its stored pair pv2 computed here.
    [[maybe_unused]] int pi = -1, pr = 0, pi2 = -1, pr2 = 0;
    [[maybe_unused]] long pg = 0;
    [[maybe_unused]] uint32_t pv2 = 0;
    [[maybe_unused]] PoolRegs pregs;
    if constexpr (FUSED) {
      long pg2 = 0;
      for (int x = 0; x < F.gx; ++x) {
        const long ge = compress_group(F.j1, pp0, x, F.L, ratio);
        if (ge < 0 || ge >= nv) continue;
        const long rel = ge - e_chunk;
        if (rel < 0 || rel >= (long)IX_WAVES * T * IX_TILE) continue;
        const int tg = (int)(rel / IX_TILE);
        if (tg % IX_WAVES != wave) continue;
        if (pi >= 0) {  // keep the earlier entry as the second one
          pi2 = pi;
          pr2 = pr;
          pg2 = pg;
        }
        pi = tg / IX_WAVES;
        pr = (int)(rel % IX_TILE);
        pg = ge;
      }
      if (pi2 >= 0) {
        PoolRegs r2;
        compress_load16<bf16>(F.j1, b, pg2, pp0, F.L, ratio, lane, 0, r2);
        const float2 y = compress_pool16(r2);
        const float tot = wave_sum(y.x * y.x + y.y * y.y);
        const float2 v = compress_finish(F.j1, y, tot, pg2, ratio, F.eps, F.log2_base, lane, F.j1.gamma[2 * lane],
                                         F.j1.gamma[2 * lane + 1]);
        pv2 = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
      }
      if (pi >= 0) compress_load16<bf16>(F.j1, b, pg, pp0, F.L, ratio, lane, 0, pregs);
    }
    WAIT_VMCNT(0);
    __syncthreads();
    bf16x8_t afr[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        afr[mt][kk] = *(const bf16x8_t*)(lds_q + (16 * mt + n) * IX_ROW + 16 * ((4 * kk + g) ^ n));
    const bool relu = !(flags & CSA_INDEX_NO_RELU);

    for (int i = 0; i < T; ++i) {
      const int e0 = tile_e0(i);
      if (e0 >= N_cap) break;  // wave-uniform
      float mine = -INFINITY;
      if (i < nt) {
        if (i + IX_NB - 1 < nt) issue(i + IX_NB - 1);  // into the slot tile i-1 used
        // vector-memory operations issued after tile i's copies: later tiles'
        // copies and the score stores of tiles max(0, i-NB+1) .. i-1
        const int later = min(nt, i + IX_NB) - i - 1;
        wait_vmcnt_dyn(later * IX_COPIES + min(i, IX_NB - 1));
        const uint8_t* kt = lds_k[wave][i % IX_NB];
        if constexpr (FUSED) {
          if (i == pi2)
            *(uint32_t*)(lds_k[wave][i % IX_NB] + pr2 * IX_ROW + 16 * ((lane >> 2) ^ (pr2 & 15)) + 4 * (lane & 3)) = pv2;
          if (i == pi) {  // this step's entry replaces whatever the copy brought
            const float2 y = compress_pool16(pregs);
            const float tot = wave_sum(y.x * y.x + y.y * y.y);
            const float2 v = compress_finish(F.j1, y, tot, pg, ratio, F.eps, F.log2_base, lane,
                                             F.j1.gamma[2 * lane], F.j1.gamma[2 * lane + 1]);
            *(uint32_t*)(lds_k[wave][i % IX_NB] + pr * IX_ROW + 16 * ((lane >> 2) ^ (pr & 15)) + 4 * (lane & 3)) =
                (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
          }
        }
#pragma unroll
        for (int nt2 = 0; nt2 < IX_TILE / 16; ++nt2) {
          f32x4_t acc[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const bf16x8_t bfr = *(const bf16x8_t*)(kt + (16 * nt2 + n) * IX_ROW + 16 * ((4 * kk + g) ^ n));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mt][kk], bfr, acc[mt], 0, 0, 0);
          }
          float v = 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) v += wv[mt][ii] * (relu ? fmaxf(acc[mt][ii], 0.f) : acc[mt][ii]);
          v = row_sum4(v);
          if (g == nt2) mine = v;
        }
        if (e0 + lane >= nv) mine = -INFINITY;
      }
      if (lane < IX_TILE && e0 + lane < N_cap) out[e0 + lane] = mine;
    }
  }

}

// Multi-query form for chunks of positions (S >= 4, prefill): a workgroup of
// IX_MQW waves scores IX_MQW consecutive queries of one sequence against the
// same key tiles.  Each 32-row tile is copied once into a 4-slot ring shared
// by the group (every wave issues its share of the copies) and read by all
// waves, so the index cache crosses into LDS once per IX_MQW queries instead
// of once per query, and with 32 KiB of LDS two groups share a CU (8 queries
// per group measured 5% faster than 4 on the prefill chunk).  One barrier per
// tile: every wave's share of tile i has landed, and every wave is done with
// the slot that the copies of tile i+3 overwrite.  q_idx and w
// of each wave's query go straight to VGPRs.  Same MFMA tiling, head
// reduction and score values as index_scores_mfma.
template <int MT>
__global__ __launch_bounds__(64 * IX_MQW) void index_scores_mq(const bf16* __restrict__ q, const float* __restrict__ w,
                                                       const bf16* __restrict__ K, const int32_t* __restrict__ q_pos,
                                                       float* __restrict__ scores, int S, int N_cap, int ratio,
                                                       unsigned flags, int T, int chunks) {
  constexpr int HI = 16 * MT;
  constexpr int NB = IX_NB;
  constexpr int CPW = IX_COPIES / IX_MQW;  // copies per wave and tile
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[NB][IX_TILE_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int sgroups = (S + IX_MQW - 1) / IX_MQW;
  const int grp = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const int b = grp / sgroups, s0 = (grp % sgroups) * IX_MQW;
  const bool live = s0 + wave < S;                // a wave past S scores the last query and stores nothing
  const int s = min(s0 + wave, S - 1);
  const int qi = b * S + s;
  const long tb = (long)q_pos[b];
  const int nv = (int)visible_entries(tb + s, ratio, N_cap);
  const int nv_max = (int)visible_entries(tb + min(s0 + IX_MQW - 1, S - 1), ratio, N_cap);
  const int e_chunk = chunk * T * IX_TILE;
  int nt = 0;  // tiles holding candidates visible to some query of the group
  if (e_chunk < nv_max) nt = min(T, (nv_max - e_chunk + IX_TILE - 1) / IX_TILE);
  float* out = scores + (size_t)qi * N_cap;
  const bf16* Kb = K + (size_t)b * N_cap * 128;

  auto issue = [&](int i) {
    const int e0 = e_chunk + i * IX_TILE;
#pragma unroll
    for (int jj = 0; jj < CPW; ++jj) {
      const int j = CPW * wave + jj;
      const int r = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      int e = e0 + r;
      e = e < nv_max ? e : nv_max - 1;  // rows past the visible range reload a valid row (masked below)
      dma16(Kb + (size_t)e * 128 + 8 * c, &lds_k[i % NB][j * 1024]);
    }
  };
  // set-up in one round trip: w and q_idx fragments into VGPRs, the first
  // NB-1 tiles into LDS
  float wv[MT][4];
  bf16x8_t afr[MT][4];
  const bf16* qb = q + (size_t)qi * HI * 128;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = w[(size_t)qi * HI + 16 * mt + 4 * g + i];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) afr[mt][kk] = *(const bf16x8_t*)(qb + (size_t)(16 * mt + n) * 128 + 32 * kk + 8 * g);
  }
  for (int i = 0; i < NB - 1 && i < nt; ++i) issue(i);
  WAIT_VMCNT(0);
  const bool relu = !(flags & CSA_INDEX_NO_RELU);

  for (int i = 0; i < nt; ++i) {
    // vector-memory operations issued after tile i's copies: later tiles'
    // copies and the score stores of tiles max(0, i-NB+1) .. i-1
    // (a wave past S stores nothing)
    const int later = min(nt, i + NB - 1) - i - 1;
    wait_vmcnt_dyn(later * CPW + (live ? min(i, NB - 1) : 0));
    lds_barrier();                            // tile i complete; slot of tile i-1 free
    if (i + NB - 1 < nt) issue(i + NB - 1);   // into the slot tile i-1 used
    const int e0 = e_chunk + i * IX_TILE;
    const uint8_t* kt = lds_k[i % NB];
    float mine = -INFINITY;
#pragma unroll
    for (int nt2 = 0; nt2 < IX_TILE / 16; ++nt2) {
      f32x4_t acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t bfr = *(const bf16x8_t*)(kt + (16 * nt2 + n) * IX_ROW + 16 * ((4 * kk + g) ^ n));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mt][kk], bfr, acc[mt], 0, 0, 0);
      }
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v += wv[mt][ii] * (relu ? fmaxf(acc[mt][ii], 0.f) : acc[mt][ii]);
      v = row_sum4(v);
      if (g == nt2) mine = v;
    }
    if (e0 + lane >= nv) mine = -INFINITY;
    if (live && lane < IX_TILE && e0 + lane < N_cap) out[e0 + lane] = mine;
  }
  // the chunk's entries past every query's visible range
  for (int i = nt; i < T; ++i) {
    const int e0 = e_chunk + i * IX_TILE;
    if (e0 >= N_cap) break;
    if (live && lane < IX_TILE && e0 + lane < N_cap) out[e0 + lane] = -INFINITY;
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

template <bool FUSED>
static void launch_index_mfma(const void* q, const float* w, const void* K, const int32_t* q_pos, float* scores,
                              int Q, int S, int Hi, int N_cap, int ratio, unsigned flags, const FusedCompress& F,
                              hipStream_t st) {
  // chunk = 4 waves x T tiles x 32 candidates; aim for ~256 workgroups (one
  // per CU, all in one round) without chunks shorter than one tile per wave
  const long cand = (long)Q * N_cap;
  long per = (cand + 255) / 256;
  int T = (int)((per + IX_WAVES * IX_TILE - 1) / (IX_WAVES * IX_TILE));
  T = T < 1 ? 1 : T;
  const int chunks = (N_cap + IX_WAVES * T * IX_TILE - 1) / (IX_WAVES * T * IX_TILE);
  const dim3 grid((unsigned)((long)Q * chunks));
#define IX_LAUNCH(M) \
  hipLaunchKernelGGL((index_scores_mfma<M, FUSED>), grid, dim3(256), 0, st, (const bf16*)q, w, (const bf16*)K, q_pos, \
                     scores, S, N_cap, ratio, flags, T, chunks, F)
  switch (Hi / 16) {
    case 1: IX_LAUNCH(1); break;
    case 2: IX_LAUNCH(2); break;
    case 3: IX_LAUNCH(3); break;
    default: IX_LAUNCH(4); break;
  }
#undef IX_LAUNCH
}

static bool index_mfma_ok(int Hi, int di, int dtype) {
  return dtype == CSA_BF16 && di == 128 && Hi % 16 == 0 && Hi <= 64;
}

hipError_t launch_index_scores(const void* q, const float* w, const void* K, const int32_t* q_pos, float* scores,
                               int B, int S, int Hi, int di, int N_cap, int ratio, unsigned flags, int dtype,
                               hipStream_t st) {
  const int Q = B * S;
  if (index_mfma_ok(Hi, di, dtype) && S >= 4) {
    // one workgroup per 4 queries and chunk of T tiles; T such that at least
    // ~512 workgroups run (two per CU) when the queries alone are fewer
    const long groups = (long)B * ((S + IX_MQW - 1) / IX_MQW);
    const long tiles = (N_cap + IX_TILE - 1) / IX_TILE;
    long chunks = (512 + groups - 1) / groups;
    chunks = chunks > tiles ? tiles : (chunks < 1 ? 1 : chunks);
    const int T = (int)((tiles + chunks - 1) / chunks);
    const int nch = (int)((tiles + T - 1) / T);
    const dim3 grid((unsigned)(groups * nch));
#define IX_MQ(M)                                                                                                 \
  hipLaunchKernelGGL((index_scores_mq<M>), grid, dim3(64 * IX_MQW), 0, st, (const bf16*)q, w, (const bf16*)K, q_pos, scores, \
                     S, N_cap, ratio, flags, T, nch)
    switch (Hi / 16) {
      case 1: IX_MQ(1); break;
      case 2: IX_MQ(2); break;
      case 3: IX_MQ(3); break;
      default: IX_MQ(4); break;
    }
#undef IX_MQ
    return hipGetLastError();
  }
  if (index_mfma_ok(Hi, di, dtype)) {
    launch_index_mfma<false>(q, w, K, q_pos, scores, Q, S, Hi, N_cap, ratio, flags, FusedCompress{}, st);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((N_cap + 255) / 256), (unsigned)(B * S));
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(index_scores_generic<float>, grid, dim3(256), 0, st, (const float*)q, w, (const float*)K,
                       q_pos, scores, S, Hi, di, N_cap, ratio, flags);
  else
    hipLaunchKernelGGL(index_scores_generic<bf16>, grid, dim3(256), 0, st, (const bf16*)q, w, (const bf16*)K, q_pos,
                       scores, S, Hi, di, N_cap, ratio, flags);
  return hipGetLastError();
}

// Whether the compressors can fold into the indexer and top-k launches: one
// position per sequence, a state of at most 2*ratio <= 16 tokens, an
// overlapping index-key compressor over the scored cache, the MFMA indexer.
bool fused_compress_ok(const FusedCompress& F, int S, int Hi, int di, int N_cap, int ratio, int dtype) {
  return S == 1 && F.L <= 2 * ratio && 2 * ratio <= 16 && F.j1.overlap && F.j1.d == di && F.j1.N_cap == N_cap &&
         index_mfma_ok(Hi, di, dtype);
}

// Index scores over F.j1.cache with this step's index-key entries computed
// by the waves that score them (the caches are written by launch_topk(F)).
hipError_t launch_index_scores_fused(const FusedCompress& F, const void* q, const float* w, const int32_t* q_pos,
                                     float* scores, int B, int S, int Hi, int N_cap, int ratio, unsigned flags,
                                     hipStream_t st) {
  launch_index_mfma<true>(q, w, F.j1.cache, q_pos, scores, B * S, S, Hi, N_cap, ratio, flags, F, st);
  return hipGetLastError();
}

}  // namespace csa_host
