// attn.hip -- multi-query attention over the sliding window plus compressed
// entries, with a learned per-head sink and inverse RoPE on the output.
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", section "局部和压缩记忆，共用一次归一化": the
// window entries and the selected compressed entries form one candidate set
// under one softmax; each head's learned sink adds to the denominator and has
// no value.  Section "输出投影也分组…": o = inverse_RoPE(o) before the output
// projection.  "图解DeepSeek V4" 2: the window KV lives in a ring of window_size
// rows, the compressed channel contributes <= topK entries; 2.3: every head
// attends to the same KV row (MQA) and the output is de-rotated.
//
// Candidate list of query position t (virtual index j):
//   j <  nwin : window position u = t - nwin + 1 + j (nwin = min(window, t+1))
//   j >= nwin : compressed entry topk_idx[j - nwin] (sparse, CSA) or
//               j - nwin (dense, HCA: every visible entry)
// Entries outside [0, N_cap) (the -1 padding) are skipped.
#include "common.hpp"

#include <cmath>

namespace csa {

struct AttnArgs {
  const void* q;
  const void* cmp;
  const int32_t* topk_idx;  // sparse mode: [B, S, k] entry list
  const void* win;
  const int32_t* win_pos0;  // NULL => ring
  const float* sink;
  const int32_t* q_pos;
  void* out;
  float* lse;
  int dense;  // 1: every visible entry (HCA); 0: the listed entries (CSA)
  int S, H, D, rope_dim, N_cap, k, ratio, W_cap, window;
  float scale;
  double log2_base;  // log2 of the RoPE base
};

// Row pointer (element offset) of candidate j of query (b, t); -1 when skipped.
__device__ __forceinline__ long cand_row(const AttnArgs& a, int b, long t, int qi, int nwin, int j, bool* is_win) {
  if (j < nwin) {
    *is_win = true;
    const long u = t - nwin + 1 + j;
    long r = a.win_pos0 ? u - a.win_pos0[b] : u % a.W_cap;
    if (r < 0 || r >= a.W_cap) return -1;
    return ((long)b * a.W_cap + r) * a.D;
  }
  *is_win = false;
  const int jj = j - nwin;
  const long e = a.dense ? (long)jj : (long)a.topk_idx[(size_t)qi * a.k + jj];
  if (e < 0 || e >= a.N_cap) return -1;
  return ((long)b * a.N_cap + e) * a.D;
}

// One wave per (query, head); lane owns dims lane + 64*i.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(AttnArgs a) {
  const int qi = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int b = qi / a.S, s = qi % a.S;
  const long t = (long)a.q_pos[b] + s;
  const int lane = threadIdx.x;
  const int nwin = (int)(t + 1 < a.window ? t + 1 : a.window);
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const T* q = (const T*)a.q + ((size_t)qi * a.H + h) * a.D;
  const T* win = (const T*)a.win;
  const T* cmp = (const T*)a.cmp;
  constexpr int MAXV = 8;  // D <= 512
  float qv[MAXV], acc[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = lane + 64 * i;
    qv[i] = c < a.D ? Elt<T>::ld(q, c) : 0.f;
    acc[i] = 0.f;
  }
  const float sink = a.sink[h];
  float m = sink, l = (sink == -INFINITY) ? 0.f : 1.f;
  for (int j = 0; j < nwin + ncmp; ++j) {
    bool is_win;
    const long off = cand_row(a, b, t, qi, nwin, j, &is_win);
    if (off < 0) continue;
    const T* row = is_win ? win + off : cmp + off;
    float rv[MAXV];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int c = lane + 64 * i;
      rv[i] = c < a.D ? Elt<T>::ld(row, c) : 0.f;
      part += qv[i] * rv[i];
    }
    const float x = a.scale * wave_sum(part);
    if (x > m) {
      const float r = expf(m - x);
      l *= r;
#pragma unroll
      for (int i = 0; i < MAXV; ++i) acc[i] *= r;
      m = x;
    }
    const float p = expf(x - m);
    l += p;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) acc[i] += p * rv[i];
  }
  __shared__ float o[512];
  const float invl = 1.f / l;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int c = lane + 64 * i;
    if (c < a.D) o[c] = acc[i] * invl;
  }
  __syncthreads();
  T* out = (T*)a.out + ((size_t)qi * a.H + h) * a.D;
  const int tail0 = a.D - a.rope_dim;
  for (int p = lane; p < a.D / 2; p += 64) {
    float x0 = o[2 * p], x1 = o[2 * p + 1];
    if (2 * p >= tail0) {
      float cs, sn;
      rope_cos_sin((double)t, p - tail0 / 2, a.rope_dim, a.log2_base, &cs, &sn);
      // inverse rotation: angle -theta
      const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    Elt<T>::st(out, 2 * p, x0);
    Elt<T>::st(out, 2 * p + 1, x1);
  }
  if (a.lse && lane == 0) a.lse[(size_t)qi * a.H + h] = m + logf(l);
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16, D == 512, H % HG == 0 with HG = 16 * NHB heads.
//
// Work item = (query, group of HG heads, split of the candidate list); the
// item -> block map is XCD-aware, so all head groups of one query run under
// one L2 and the query's gathered rows come from HBM once.  Candidates go in
// tiles of 64 rows (64 KiB) through a 2-stage LDS ring.  Workgroup = 8 waves,
// two per SIMD, in two roles:
//   S waves 0-3: wave w owns rows 16w..16w+15 of every tile and holds the q
//     fragments of all HG heads in VGPRs.  S^T[16 rows x HG heads] = R . Q^T
//     over all 512 dims (MFMA 16x16x32, A = rows read from LDS), then the
//     online softmax in the exp2 domain; P (bf16, [head][row]) goes to LDS.
//   O waves 4-7: wave 4+v owns the 128-dim slice 128v..128v+127 of O and
//     copies rows 16v..16v+15 of every tile into the ring (direct
//     global->LDS copies, one whole 1 KiB row per instruction: a coalesced
//     stream of full cache lines).  O^T[128 dims x HG heads] += R^T . P^T
//     over the tile's 64 rows (A = rows read transposed with
//     ds_read_b64_tr_b16, B = P^T from LDS).
// Per tile i two barriers: X_i (tile i landed, the other stage free) ->
// S: logits + softmax of tile i while O: copies of tile i+1 into the other
// stage -> Y_i (P visible) -> O: P.V of tile i, wait for the copies -> X_i+1.
// Each row crosses LDS three times (copy in, logits, transposed read), each
// time for all HG heads; with two waves per SIMD one role's LDS and memory
// waits overlap the other role's matrix work.
// The running max is common to all S waves and moves lazily: a tile whose
// logits exceed it by more than 2^SLACK raises a flag; then the S waves take
// the exact maximum, rewrite P and publish the rescale factors, which the O
// waves apply to O before that tile's P.V.  The sink logit is the initial
// reference of the running max and adds exp2(0) = 1 to the sum exactly once
// (split 0).
//
// Splits: when there are too few (query, head group) items to fill the chip,
// an item's tiles are divided between NS workgroups (16 or 32 heads per
// workgroup as the plan's cost model picks), each of which writes its O
// divided by its own sum (bf16), its running max and its sum (fp32) to the
// workspace; attn_merge_kernel (launched next on the same stream) combines
// them.
// LDS rows are 1088 bytes apart (64 bytes of padding, no permutation): the
// row reads of QK^T (ds_read_b128) and the transposed reads of P.V
// (ds_read_b64_tr_b16) then run at 113-117 B/clk/CU on gfx950, against 95-101
// for XOR-swizzled 1024-byte rows (a probe of exactly these access
// patterns), and every address is one lane base plus immediates.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int AT_D = 512;
constexpr int AT_ROWB = AT_D * 2;
constexpr int AT_TR = 64;                       // rows per tile
constexpr int AT_RS = AT_ROWB + 64;            // LDS bytes per tile row (64 bytes of padding)
constexpr int AT_TILE_B = AT_TR * AT_RS;
constexpr int AT_MAXK = 2048;                   // sparse lists up to this many entries
constexpr int AT_MAXWIN = 1024;                 // windows up to this many rows
constexpr int AT_LIST = AT_MAXWIN + AT_MAXK;    // candidate slots resolved in LDS
constexpr int AT_PST = AT_TR + 8;               // bf16 per P row (padded against bank conflicts)
// One split's partial: O / l as bf16 in the lane layout (4 slices x 8 dim
// tiles x 2 head blocks x 64 lanes x 4), then (m, l) per head as fp32.
constexpr int AT_PART_O = 4 * 8 * 2 * 64 * 4;    // bf16 elements of the O part
constexpr int AT_PART_B = AT_PART_O * 2 + 64 * 4;  // bytes of one partial
constexpr float LOG2E = 1.4426950408889634f;
constexpr float AT_SLACK = 16.f;                // log2 headroom of the lazily updated running max

// Offset (elements) of lane `lane`'s O^T fragment (dim tile dt, head block hb)
// of dim slice `v` inside a partial's O part.
__device__ __forceinline__ int part_off(int v, int dt, int hb, int lane) {
  return (((v * 8 + dt) * 2 + hb) * 64 + lane) * 4;
}

// De-rotation table of position t: (cos, sin) of the rope_dim / 2 tail pairs.
__device__ __forceinline__ void fill_rope_table(float2* tab, int t, int rope_dim, double log2_base, int tid,
                                                int nthreads) {
  for (int p = tid; p < rope_dim / 2; p += nthreads) {
    float c, sn;
    rope_cos_sin((double)t, p, rope_dim, log2_base, &c, &sn);
    tab[p] = make_float2(c, sn);
  }
}

// Lane (g, n) of dim slice v holds O^T[dim 128*v + 16*dt + 4*g + i][head
// h0 + 16*hb + n].  The inverse RoPE of position t is a rotation of each tail
// pair, linear in O: it is applied before the division by the sum as well.
template <int NHB>
__device__ __forceinline__ void derotate(f32x4_t (&o)[8][NHB], int v, int lane, int rope_dim,
                                         const float2* rope_cs) {
  const int g = lane >> 4;
  const int tail0 = AT_D - rope_dim;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int dim = v * 128 + 16 * dt + 4 * g;
    if (dim + 4 <= tail0) continue;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (dim + 2 * pp >= tail0) {
        const float2 cs = rope_cs[(dim + 2 * pp - tail0) / 2];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const float x0 = o[dt][hb][2 * pp], x1 = o[dt][hb][2 * pp + 1];
          o[dt][hb][2 * pp] = x0 * cs.x + x1 * cs.y;
          o[dt][hb][2 * pp + 1] = -x0 * cs.y + x1 * cs.x;
        }
      }
    }
  }
}

// Final output of one dim slice (already de-rotated): divide by the sum,
// store bf16, and the log-sum-exp of the denominator.
template <int NHB>
__device__ __forceinline__ void store_output(const AttnArgs& a, int qi, int h0, int v, int lane,
                                             const f32x4_t (&o)[8][NHB], const float (&l)[NHB],
                                             const float (&m)[NHB]) {
  const int g = lane >> 4, n = lane & 15;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float inv_l = 1.f / l[hb];
    bf16* outp = (bf16*)a.out + ((size_t)qi * a.H + h0 + 16 * hb + n) * AT_D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int dim = v * 128 + 16 * dt + 4 * g;
      float x[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) x[ii] = o[dt][hb][ii] * inv_l;
      uint2 pk;
      pk.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
      pk.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
      *(uint2*)(outp + dim) = pk;
    }
    if (a.lse && v == 0 && g == 0) a.lse[(size_t)qi * a.H + h0 + 16 * hb + n] = (m[hb] + log2f(l[hb])) / LOG2E;
  }
}

// KV8: window and compressed rows in the FP8 row format (common.hpp): each
// 640-byte row goes raw into the top of its LDS row slot with the bf16
// kernel's direct copies, and the wave that copied it dequantises it in place
// (exact, one scaled conversion per two values) into the bf16 row layout
// before the barrier that publishes the tile.  From tile 1 on, the S and the O
// wave of a row block share its 16 rows (8 each): the S wave between its
// softmax and the barrier, the O wave between the halves of its P.V.
// Everything else is the bf16 kernel.
template <int NHB, bool KV8 = false>
__global__ __launch_bounds__(512) void attn_tile_kernel(AttnArgs a, int n_hg, int nsplit, int total_items,
                                                        float* __restrict__ part) {
  constexpr int HG = 16 * NHB;
  constexpr int ROWB = KV8 ? FP8_ROW_BYTES : AT_ROWB;  // bytes per window / compressed row
  __shared__ __attribute__((aligned(16))) uint8_t ring[2][AT_TILE_B];
  __shared__ __attribute__((aligned(16))) __bf16 pbuf[HG][AT_PST];
  __shared__ float mbuf[4][NHB][64];   // S waves' tile maxima (rescale path)
  __shared__ float abuf[NHB][16];      // rescale factors for the O waves
  __shared__ float lbuf[4][NHB][16];   // S waves' sums, then the running max
  __shared__ float mfin[NHB][16];
  __shared__ uint32_t fbuf[4];
  __shared__ __attribute__((aligned(16))) int32_t s_rows[AT_LIST];
  __shared__ uint64_t s_mask[AT_LIST / AT_TR];
  __shared__ float2 rope_cs[AT_D / 2];

  const int item = xcd_remap(blockIdx.x, total_items);
  const int split = item % nsplit, qh = item / nsplit;
  const int qi = qh / n_hg, hgi = qh % n_hg;
  const int b = qi / a.S, s = qi % a.S;
  const int t = a.q_pos[b] + s;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool is_s = wave < 4;          // wave-uniform role
  const int w4 = wave & 3;             // S: row block; O: dim slice and copied rows
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int h0 = hgi * HG;
  const int nwin = max(0, min(t + 1, a.window));
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const int ncand = nwin + ncmp;
  const int nt_all = (ncand + AT_TR - 1) / AT_TR;
  const int tps = (nt_all + nsplit - 1) / nsplit;
  const int tb = min(nt_all, split * tps);
  const int ntiles = min(nt_all, tb + tps) - tb;
  const int jb0 = tb * AT_TR;  // first candidate slot of this split
  const char* winb = (const char*)a.win + (size_t)b * a.W_cap * ROWB;
  const char* cmpb = (const char*)a.cmp + (size_t)b * a.N_cap * ROWB;

  // S waves: the HG q rows of the group once into ring stage 1 (first
  // overwritten by the copies of tile 1, after barrier X_0), swizzled like
  // candidate rows.
  float sinkv[NHB];
  if (is_s) {
    const char* qb = (const char*)a.q + ((size_t)qi * a.H + h0) * AT_ROWB;
#pragma unroll
    for (int rr = 0; rr < HG / 4; ++rr) {
      const int r = w4 * (HG / 4) + rr;
      dma16_sbase(qb + (size_t)r * AT_ROWB, 16u * (uint32_t)lane, ring[1] + r * AT_RS);
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) sinkv[hb] = a.sink[h0 + 16 * hb + n];
  }

  // Candidate slots of this split resolved once into LDS: s_rows[jl] >= 0 is
  // compressed entry s_rows[jl], < 0 is window row -1 - s_rows[jl].  Skipped
  // slots (padding, out-of-range ids, the ragged tail) point at window row 0
  // and have their bit cleared in the per-tile validity mask.  Dense
  // candidates beyond the table are formed on the fly (all valid).
  // Every list load is issued first (unconditional, clamped into the list),
  // then the RoPE table is computed while they are in flight.
  const int nlist = min(ntiles * AT_TR, AT_LIST);
  constexpr int NIT = AT_LIST / 512;  // slot rounds per wave
  int eid[NIT];
  const int wpos0 = a.win_pos0 ? a.win_pos0[b] : 0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int jj = jb0 + wave * 64 + 512 * it + lane - nwin;  // list position of the slot
    eid[it] = (!a.dense && a.k > 0) ? a.topk_idx[(size_t)qi * a.k + min(max(jj, 0), a.k - 1)] : jj;
  }
  fill_rope_table(rope_cs, t, a.rope_dim, a.log2_base, threadIdx.x, 512);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int j0 = wave * 64 + 512 * it;
    if (j0 >= nlist) break;  // wave-uniform
    const int j = jb0 + j0 + lane;
    int id = -1;
    bool ok = false;
    if (j < nwin) {
      const int u = t - nwin + 1 + j;
      const int rw = a.win_pos0 ? u - wpos0 : u % a.W_cap;
      ok = rw >= 0 && rw < a.W_cap;
      id = ok ? -1 - rw : -1;
    } else if (j < ncand) {
      const int e = eid[it];
      ok = e >= 0 && e < a.N_cap;
      id = ok ? e : -1;
    }
    s_rows[j0 + lane] = id;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
    if (lane == 0) s_mask[j0 / AT_TR] = bal;
  }
  // Every ordinary load (and the q copy) is complete here: the compiler then
  // has no pending load to wait for inside the tile loop (such a wait would
  // be vmcnt(0) and drain the copies in flight).
  WAIT_VMCNT(0);
  __syncthreads();

  // O waves: row ids (uniform) of the 16 rows this wave copies of local tile
  // ti, and the copy of one of them into stage ti & 1.
  auto row_ids = [&](int ti, int (&ids)[16]) {
    const int jl = ti * AT_TR + 16 * w4;  // first local slot this wave copies
    if (jl + 16 <= nlist) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int4 x = *(const int4*)&s_rows[jl + 4 * v];
        ids[4 * v] = __builtin_amdgcn_readfirstlane(x.x);
        ids[4 * v + 1] = __builtin_amdgcn_readfirstlane(x.y);
        ids[4 * v + 2] = __builtin_amdgcn_readfirstlane(x.z);
        ids[4 * v + 3] = __builtin_amdgcn_readfirstlane(x.w);
      }
    } else {  // dense candidates past the table
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int j = jb0 + jl + rr;
        ids[rr] = j < ncand ? j - nwin : 0;
      }
    }
  };
  auto copy_tile = [&](int ti) {
    int ids[16];
    row_ids(ti, ids);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int id = ids[rr];
      const char* row = id >= 0 ? cmpb + (size_t)(uint32_t)id * ROWB : winb + (size_t)(uint32_t)(-1 - id) * ROWB;
      dma16_sbase(row, 16u * (uint32_t)lane, ring[ti & 1] + (16 * w4 + rr) * AT_RS);
    }
  };
  // FP8 rows: the 16 rows this wave copies of tile ti go raw into the top of
  // their 1088-byte LDS row slots (bytes 448 .. 1087) with the same direct
  // copies as bf16 rows (lanes 0..39, 640 bytes) ...
  auto copy_tile8 = [&](int ti, int r0, int nr) {
    int ids[16];
    row_ids(ti, ids);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      if (rr < r0 || rr >= r0 + nr) continue;  // uniform
      const int id = ids[rr];
      const char* row = id >= 0 ? cmpb + (size_t)(uint32_t)id * ROWB : winb + (size_t)(uint32_t)(-1 - id) * ROWB;
      if (lane < 40) dma16_sbase(row, 16u * (uint32_t)lane, ring[ti & 1] + (16 * w4 + rr) * AT_RS + FP8_NQ);
    }
  };
  // ... and, once landed, are dequantised in place: the codes of dims d sit at
  // byte 448 + d of the slot and their bf16 values go to byte 2d, so each lane
  // l < 56 reads its 8 codes (dims 8l .. 8l+7) and the 7 exponents (bytes
  // 1024 ..) before the wave writes anything; the RoPE dims are bf16 already
  // and already at bytes 896 .. 1023.  Rows r0 .. r0+nr-1 of the wave's block
  // (nr a multiple of 8), 8 rows per batch: their reads, one wait, the writes.
  auto convert_tile8 = [&](int ti, int r0, int nr) {
#pragma unroll
    for (int b0 = 0; b0 < 16; b0 += 8) {
      if (b0 < r0 || b0 >= r0 + nr) continue;  // uniform
      uint2 c[8], sk[8];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const uint8_t* slot = ring[ti & 1] + (16 * w4 + b0 + rr) * AT_RS;
        c[rr] = make_uint2(0u, 0u);
        if (lane < 56) c[rr] = *(const uint2*)(slot + FP8_NQ + 8 * lane);
        sk[rr] = *(const uint2*)(slot + FP8_NQ + FP8_SCALE_OFF);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): every read of these rows before any write
      if (lane < 56) {
        const int blk = lane >> 3;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          uint8_t* slot = ring[ti & 1] + (16 * w4 + b0 + rr) * AT_RS;
          const int k = (int)(int8_t)(((blk < 4 ? sk[rr].x : sk[rr].y) >> (8 * (blk & 3))) & 0xFFu);
          *(uint4*)(slot + 16 * lane) = make_uint4(fp8_pair_to_bf16x2(c[rr].x & 0xFFFFu, k),
                                                   fp8_pair_to_bf16x2(c[rr].x >> 16, k),
                                                   fp8_pair_to_bf16x2(c[rr].y & 0xFFFFu, k),
                                                   fp8_pair_to_bf16x2(c[rr].y >> 16, k));
        }
      }
    }
  };
  auto tile_mask = [&](int ti) -> uint64_t {
    if (ti * AT_TR < nlist) return s_mask[ti];
    const int left = ncand - (jb0 + ti * AT_TR);  // dense tail past the table
    return left >= 64 ? ~0ull : ((1ull << left) - 1ull);
  };

  float m_run[NHB], l_run[NHB];  // S waves
  f32x4_t o[8][NHB];             // O waves
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) o[dt][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (is_s) {
    // ---------------------------------------------------------------- S waves
    // q fragments (B operand of QK^T): head h0 + 16*hb + n, dims 32*kk + 8*g .. +8
    bf16x8_t qf[NHB][16];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const uint8_t* qr = ring[1] + (16 * hb + n) * AT_RS + 16 * g;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) qf[hb][kk] = *(const bf16x8_t*)(qr + 64 * kk);
    }
    const float sc2 = a.scale * LOG2E;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      m_run[hb] = sinkv[hb] * LOG2E;
      l_run[hb] = (split == 0 && w4 == 0 && g == 0 && sinkv[hb] != -INFINITY) ? 1.f : 0.f;
    }
    lds_barrier();              // X_0 (every wave has its q fragments before tile 1 is copied)
    for (int i = 0; i < ntiles; ++i) {
      if constexpr (KV8) {
        // FP8 rows: this S wave copies (and later dequantises) rows 8..15 of
        // its block of tile i+1, into the stage tile i-1 used
        if (i + 1 < ntiles) copy_tile8(i + 1, 8, 8);
      }
      const uint8_t* myrow = ring[i & 1] + (16 * w4 + n) * AT_RS + 16 * g;
      // 1. logits of this wave's 16 rows for the HG heads (two chains per head block)
      f32x4_t S0[NHB], S1[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) S0[hb] = S1[hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8_t rf[8];
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) {
          const int kk = 8 * half + k2;
          rf[k2] = *(const bf16x8_t*)(myrow + 64 * kk);
        }
#pragma unroll
        for (int k2 = 0; k2 < 8; k2 += 2) {
          const int kk = 8 * half + k2;
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            S0[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf[k2], qf[hb][kk], S0[hb], 0, 0, 0);
            S1[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rf[k2 + 1], qf[hb][kk + 1], S1[hb], 0, 0, 0);
          }
        }
      }
      // 2. P with the current running max; lane (g, n): rows 16w + 4g + ii, heads 16hb + n
      const uint32_t vb = (uint32_t)(tile_mask(i) >> (16 * w4 + 4 * g)) & 0xFu;
      float sv[NHB][4], pv[NHB][4], lm[NHB];
      bool up = false;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const f32x4_t S = S0[hb] + S1[hb];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sv[hb][ii] = ((vb >> ii) & 1u) ? S[ii] * sc2 : -INFINITY;
        lm[hb] = fmaxf(fmaxf(sv[hb][0], sv[hb][1]), fmaxf(sv[hb][2], sv[hb][3]));
        up = up || lm[hb] > m_run[hb] + AT_SLACK;
      }
      const bool moved = __builtin_amdgcn_ballot_w64(up) != 0;
      auto write_p = [&]() {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          // m_run is -inf only while every logit so far is masked (sink -inf):
          // the reference 0 then gives p == 0 instead of NaN
          const float m_ref = (m_run[hb] == -INFINITY) ? 0.f : m_run[hb];
          bf16x4_t pk;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            pv[hb][ii] = __builtin_amdgcn_exp2f(sv[hb][ii] - m_ref);
            pk[ii] = (__bf16)pv[hb][ii];
          }
          *(bf16x4_t*)&pbuf[16 * hb + n][16 * w4 + 4 * g] = pk;
        }
      };
      write_p();
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) mbuf[w4][hb][lane] = lm[hb];
      if (lane == 0) fbuf[w4] = moved ? 1u : 0u;
      lds_barrier();  // Y_i: P, tile maxima and flags visible
      if (fbuf[0] | fbuf[1] | fbuf[2] | fbuf[3]) {
        // rare: some logit left the running max's headroom -> exact maximum,
        // P again, and the factor for O published to the O waves
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          float mt = -INFINITY;
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
            for (int g2 = 0; g2 < 4; ++g2) mt = fmaxf(mt, mbuf[w2][hb][16 * g2 + n]);
          const float m_new = fmaxf(m_run[hb], mt);
          const float alpha = (m_new == m_run[hb]) ? 1.f : __builtin_amdgcn_exp2f(m_run[hb] - m_new);
          l_run[hb] *= alpha;
          if (w4 == 0 && g == 0) abuf[hb][n] = alpha;
          m_run[hb] = m_new;
        }
        write_p();
        lds_barrier();  // Y'_i
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) l_run[hb] += (pv[hb][0] + pv[hb][1]) + (pv[hb][2] + pv[hb][3]);
      if constexpr (KV8) {
        if (i + 1 < ntiles) {
          WAIT_VMCNT(0);  // this wave's copies of tile i+1 have landed
          convert_tile8(i + 1, 8, 8);
        }
      }
      if (i + 1 < ntiles) lds_barrier();  // X_i+1
    }
    // sums over the lane groups, and the running max, for the O waves
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float l = l_run[hb];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      if (g == 0) lbuf[w4][hb][n] = l;
      if (w4 == 0 && g == 0) mfin[hb][n] = m_run[hb];
    }
  } else {
    // ---------------------------------------------------------------- O waves
    const int d0 = w4 * 128;            // P.V dim slice of this wave
    // transposed reads: rows 32c + 8g + (n >> 2) (+4), dims d0 + 16dt + 4(n & 3)
    const int tr_off = (8 * g + (n >> 2)) * AT_RS + 2 * d0 + 8 * (n & 3);
    // Y_i (and Y'_i on a rescale), then this tile's P.V into o
    auto pv_tile = [&](int i, auto&& mid) {
      const uint8_t* tile = ring[i & 1];
      lds_barrier();  // Y_i
      if (fbuf[0] | fbuf[1] | fbuf[2] | fbuf[3]) {
        lds_barrier();  // Y'_i: rescale factors and the new P visible
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const float alpha = abuf[hb][n];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[dt][hb] *= alpha;
        }
      }
      // O^T[128 dims x HG heads] += R^T[128 x 64 rows] P^T[64 rows x HG heads]
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c == 1) mid();  // work that overlaps the first half's matrix ops
        bf16x8_t pf[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) pf[hb] = *(const bf16x8_t*)&pbuf[16 * hb + n][32 * c + 8 * g];
        const uint8_t* pa = tile + tr_off + 32 * c * AT_RS;
        const uint8_t* pb = pa + 4 * AT_RS;
        bf16x4_t lo[8], hi[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          lo[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(pa + 32 * dt));
          hi[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(pb + 32 * dt));
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const bf16x8_t afr = __builtin_shufflevector(lo[dt], hi[dt], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) o[dt][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, pf[hb], o[dt][hb], 0, 0, 0);
        }
      }
    };
    if constexpr (KV8) {
      // the bf16 schedule, with each tile dequantised in place after its
      // copies land, between the two halves of the previous tile's P.V (so
      // the conversion overlaps its matrix ops), before the barrier that
      // publishes it
      if (ntiles > 0) {
        copy_tile8(0, 0, 16);
        WAIT_VMCNT(0);
        convert_tile8(0, 0, 16);
      }
      lds_barrier();  // X_0
      for (int i = 0; i < ntiles; ++i) {
        if (i + 1 < ntiles) copy_tile8(i + 1, 0, 8);  // rows 0..7 of the block; the S wave takes 8..15
        pv_tile(i, [&] {
          if (i + 1 < ntiles) {
            WAIT_VMCNT(0);  // this wave's copies of tile i+1 have landed
            convert_tile8(i + 1, 0, 8);
          }
        });
        if (i + 1 < ntiles) lds_barrier();  // X_i+1
      }
    } else {
      if (ntiles > 0) copy_tile(0);
      WAIT_VMCNT(0);
      lds_barrier();  // X_0
      for (int i = 0; i < ntiles; ++i) {
        if (i + 1 < ntiles) copy_tile(i + 1);  // into the stage tile i-1 used
        pv_tile(i, [] {});
        if (i + 1 < ntiles) {
          WAIT_VMCNT(0);  // this wave's copies of tile i+1 have landed
          lds_barrier();  // X_i+1
        }
      }
    }
  }
  __syncthreads();  // S waves' sums and maximum visible
  if (is_s) return;

  float l_tot[NHB], m_fin[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    l_tot[hb] = (lbuf[0][hb][n] + lbuf[1][hb][n]) + (lbuf[2][hb][n] + lbuf[3][hb][n]);
    m_fin[hb] = mfin[hb][n];
  }
  derotate<NHB>(o, w4, lane, a.rope_dim, rope_cs);
  if (nsplit == 1) {
    store_output<NHB>(a, qi, h0, w4, lane, o, l_tot, m_fin);
    return;
  }
  // partial of this split for attn_merge_kernel: the de-rotated O divided by
  // this split's sum (a convex combination of rows, so bf16 keeps the range),
  // and (m, l) in fp32
  uint8_t* pb = (uint8_t*)part + (size_t)item * AT_PART_B;
  bf16* po = (bf16*)pb;
  float* pml = (float*)(pb + AT_PART_O * 2);
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float inv_l = l_tot[hb] > 0.f ? 1.f / l_tot[hb] : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(o[dt][hb][0] * inv_l) | ((uint32_t)f2bf(o[dt][hb][1] * inv_l) << 16);
      pk.y = (uint32_t)f2bf(o[dt][hb][2] * inv_l) | ((uint32_t)f2bf(o[dt][hb][3] * inv_l) << 16);
      *(uint2*)(po + part_off(w4, dt, hb, lane)) = pk;
    }
  }
  if (w4 == 0 && g == 0) {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      pml[(16 * hb + n) * 2] = m_fin[hb];
      pml[(16 * hb + n) * 2 + 1] = l_tot[hb];
    }
  }
}

// Merge of the NS partials of one (query, head group) (already de-rotated):
// rescale each to the common maximum, add in split order (deterministic),
// divide by the sum and store.  Block = 64 lanes covering one wave's share of the
// partial layout for two of its eight 16-dim tiles (grid: items x 16), so many
// small blocks keep the partial reads in flight; every load is issued before
// any arithmetic.
template <int NHB>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a, int n_hg, int nsplit,
                                                        const uint8_t* __restrict__ part) {
  // the same XCD-aware map as the tile kernel: a (query, head group)'s
  // partials are read on the XCD whose L2 received them
  const int mb = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int qh = mb >> 4, wave = (mb >> 2) & 3, dt0 = 2 * (mb & 3);
  const int qi = qh / n_hg, hgi = qh % n_hg;
  const int lane = threadIdx.x, g = lane >> 4, n = lane & 15;
  const uint8_t* pq = part + (size_t)qh * nsplit * AT_PART_B;
  auto po = [&](int s2) { return (const bf16*)(pq + (size_t)s2 * AT_PART_B); };
  auto pml = [&](int s2) { return (const float*)(pq + (size_t)s2 * AT_PART_B + AT_PART_O * 2); };
  auto unpack = [](uint2 u) {
    return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xFFFF0000u)};
  };
  // all partial loads first (one memory round trip for up to AT_MQ splits)
  constexpr int AT_MQ = 4;
  uint2 v[AT_MQ][NHB][2];
  float2 ml[AT_MQ][NHB];
  const int nq = nsplit < AT_MQ ? nsplit : AT_MQ;
#pragma unroll
  for (int s2 = 0; s2 < AT_MQ; ++s2) {
    if (s2 < nq) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        v[s2][hb][0] = *(const uint2*)(po(s2) + part_off(wave, dt0, hb, lane));
        v[s2][hb][1] = *(const uint2*)(po(s2) + part_off(wave, dt0 + 1, hb, lane));
        ml[s2][hb] = *(const float2*)(pml(s2) + (16 * hb + n) * 2);
      }
    }
  }
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int mi = (16 * hb + n) * 2;
    float mx = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < AT_MQ; ++s2)
      if (s2 < nq) mx = fmaxf(mx, ml[s2][hb].x);
    for (int s2 = AT_MQ; s2 < nsplit; ++s2) mx = fmaxf(mx, pml(s2)[mi]);
    const float mref = (mx == -INFINITY) ? 0.f : mx;
    // weight of split s: l_s * exp2(m_s - max); out = sum w_s (O_s / l_s) / sum w_s
    float l = 0.f;
    f32x4_t o[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s2 = 0; s2 < AT_MQ; ++s2) {
      if (s2 < nq) {
        const float ws = ml[s2][hb].y * __builtin_amdgcn_exp2f(ml[s2][hb].x - mref);
        l += ws;
        o[0] += ws * unpack(v[s2][hb][0]);
        o[1] += ws * unpack(v[s2][hb][1]);
      }
    }
    for (int s2 = AT_MQ; s2 < nsplit; ++s2) {
      const float ws = pml(s2)[mi + 1] * __builtin_amdgcn_exp2f(pml(s2)[mi] - mref);
      l += ws;
      o[0] += ws * unpack(*(const uint2*)(po(s2) + part_off(wave, dt0, hb, lane)));
      o[1] += ws * unpack(*(const uint2*)(po(s2) + part_off(wave, dt0 + 1, hb, lane)));
    }
    const float inv_l = 1.f / l;
    const int h = hgi * 16 * NHB + 16 * hb + n;
    bf16* outp = (bf16*)a.out + ((size_t)qi * a.H + h) * AT_D;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int dim = wave * 128 + 16 * (dt0 + j) + 4 * g;
      float x[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) x[ii] = o[j][ii] * inv_l;
      uint2 pk;
      pk.x = (uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16);
      pk.y = (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16);
      *(uint2*)(outp + dim) = pk;
    }
    if (a.lse && wave == 0 && dt0 == 0 && g == 0) a.lse[(size_t)qi * a.H + h] = (mx + log2f(l)) / LOG2E;
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

// Launch plan of the MFMA kernel: heads per workgroup and candidate splits.
struct AttnPlan {
  int nhb, n_hg, nsplit, total;
  size_t ws_bytes;
};

static AttnPlan attn_plan_nhb(long Q, int H, long n_cand, int nhb) {
  AttnPlan p;
  p.nhb = nhb;
  p.n_hg = H / (16 * p.nhb);
  const long items = Q * p.n_hg;  // >= 1: Q >= 1 and H >= 16 * nhb here
  const long nt = (n_cand + AT_TR - 1) / AT_TR;
  // split the candidate tiles only when the items alone leave CUs idle, and
  // keep at least two tiles per split
  long ns = 1;
  if (items < 256) ns = (256 + items - 1) / items;
  ns = ns > nt / 2 ? nt / 2 : ns;
  ns = ns > 16 ? 16 : ns;
  p.nsplit = ns < 1 ? 1 : (int)ns;
  p.total = (int)(items * p.nsplit);
  p.ws_bytes = p.nsplit > 1 ? (size_t)p.total * AT_PART_B : 0;
  return p;
}

// Predicted time of a plan: one workgroup per CU (the LDS ring takes ~158
// KiB), so ceil(workgroups / 256) rounds, each a set-up plus the tiles of one
// split, and the merge when the list is split.  The constants were measured on
// MI355X at decode shapes (16 and 32 heads per workgroup over 3-18 tiles per
// split, with and without splits): set-up 4.3 / 6.2 us, a 64-row tile 1.37 /
// 1.75 us, the merge 4.7 us.
static double attn_plan_cost(const AttnPlan& p, long n_cand) {
  const long nt = (n_cand + AT_TR - 1) / AT_TR;
  const long tps = (nt + p.nsplit - 1) / p.nsplit;
  const long rounds = (p.total + 255) / 256;
  const double setup = p.nhb == 2 ? 6.2 : 4.3, tile = p.nhb == 2 ? 1.75 : 1.37;
  return (double)rounds * (setup + tps * tile) + (p.nsplit > 1 ? 4.7 : 0.0);
}

// 32 heads per workgroup (each gathered row serves twice the heads per LDS
// pass) or 16 (twice the workgroups, a cheaper set-up and tile), whichever the
// cost model predicts faster: 32 heads for many queries (fewer rounds of
// workgroups) and for long lists split twice (csa_decode_32k), 16 heads for
// short lists at decode (hca_decode_32k, window-only layers: no split, no
// merge) and for few queries (csa_decode_1m: 8 queries, 4 splits instead of 8).
static AttnPlan attn_plan(long Q, int H, long n_cand) {
  const AttnPlan p1 = attn_plan_nhb(Q, H, n_cand, 1);
  if (H % 32 != 0) return p1;
  const AttnPlan p2 = attn_plan_nhb(Q, H, n_cand, 2);
  return attn_plan_cost(p2, n_cand) <= attn_plan_cost(p1, n_cand) ? p2 : p1;
}

size_t attn_workspace_size(int B, int S, int H, int D, long n_cand) {
  if (D != AT_D || H < 16 || H % 16 != 0 || B < 1 || S < 1 || n_cand < 0 || (long)B * S * H > INT32_MAX) return 0;
  return attn_plan((long)B * S, H, n_cand).ws_bytes;
}

hipError_t launch_attn(const void* q, const void* cmp, const int32_t* topk_idx, int k, int dense, int ratio,
                       const void* win,
                       const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                       void* ws, int B, int S, int H, int D, int rope_dim, int N_cap, int W_cap, int window,
                       float scale, float base, int dtype, hipStream_t st) {
  AttnArgs a{q, cmp, topk_idx, win, win_pos0, sink, q_pos, out, lse, dense, S, H, D, rope_dim, N_cap, k, ratio,
             W_cap, window, scale, std::log2((double)base)};
  const long Q = (long)B * S;
  if ((dtype == CSA_BF16 || dtype == CSA_BF16_KV_FP8) && D == AT_D && H % 16 == 0 && (dense || k <= AT_MAXK) &&
      window <= AT_MAXWIN) {
    const AttnPlan p = attn_plan(Q, H, (long)window + (dense ? N_cap : k));
    float* part = p.nsplit > 1 ? (float*)ws : nullptr;
    const int items = p.total / p.nsplit;
    if (dtype == CSA_BF16_KV_FP8) {
      if (p.nhb == 2)
        hipLaunchKernelGGL((attn_tile_kernel<2, true>), dim3(p.total), dim3(512), 0, st, a, p.n_hg, p.nsplit, p.total,
                           part);
      else
        hipLaunchKernelGGL((attn_tile_kernel<1, true>), dim3(p.total), dim3(512), 0, st, a, p.n_hg, p.nsplit, p.total,
                           part);
    } else if (p.nhb == 2) {
      hipLaunchKernelGGL((attn_tile_kernel<2>), dim3(p.total), dim3(512), 0, st, a, p.n_hg, p.nsplit, p.total, part);
    } else {
      hipLaunchKernelGGL((attn_tile_kernel<1>), dim3(p.total), dim3(512), 0, st, a, p.n_hg, p.nsplit, p.total, part);
    }
    if (p.nsplit > 1) {
      if (p.nhb == 2)
        hipLaunchKernelGGL((attn_merge_kernel<2>), dim3(items * 16), dim3(64), 0, st, a, p.n_hg, p.nsplit,
                           (const uint8_t*)part);
      else
        hipLaunchKernelGGL((attn_merge_kernel<1>), dim3(items * 16), dim3(64), 0, st, a, p.n_hg, p.nsplit,
                           (const uint8_t*)part);
    }
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)((size_t)B * S * H);
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(attn_generic_kernel<float>, dim3(blocks), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<bf16>, dim3(blocks), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa_host
