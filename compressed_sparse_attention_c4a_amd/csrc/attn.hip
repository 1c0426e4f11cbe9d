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
  float scale, base;
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
      rope_cos_sin((double)t, p - tail0 / 2, a.rope_dim, a.base, &cs, &sn);
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
// MFMA kernel: bf16, D == 512, H % HG == 0.
//
// Work item = (query, group of HG heads); the item -> block map is XCD-aware
// so all head groups of one query share an L2 and the query's gathered rows
// come from HBM once.  Workgroup = 4 waves; wave w owns heads
// [16*(w % NHW), +16) of the group and the dim slice [DS*(w / NHW), +DS),
// NHW = HG/16, DS = 512*NHW/4.
//
// Candidates stream in tiles of 32 rows (32 KiB) through a 4-stage LDS ring
// filled by direct global->LDS copies (one 1 KiB row per wave instruction,
// each wave copies 8 rows per tile), three tiles ahead of use.  Per tile and
// wave:
//   S^T[32 rows x 16 heads] = R . Q^T over the wave's dims (MFMA 16x16x32, A =
//     rows from LDS, B = q fragments held in VGPRs); the waves sharing a head
//     group add their partial logits through LDS, so all of them hold the
//     same logits and identical softmax statistics;
//   online softmax in the exp2 domain; the sink seeds the running max and sum
//     and so enters the denominator exactly once; O is rescaled only when a
//     running max changes;
//   O^T[DS dims x 16 heads] += R^T . P^T (A = rows read transposed with
//     ds_read_b64_tr_b16, B = P^T taken straight from the S^T lanes).
// Software pipeline: iteration i issues the logit MFMAs of tile i+1 before
// the softmax and P.V of tile i, so the matrix core works under the softmax,
// and ends with ONE barrier that publishes tile i+1's partial logits, makes
// tile i+2 resident for all waves and frees tile i's stage for tile i+4.
// Rows are XOR-swizzled in LDS (16 B granule c of row r sits at c ^ (r & 15))
// so 16 lanes reading 16 rows hit distinct banks.  The epilogue divides by
// the sum, de-rotates the RoPE tail at the query position and stores bf16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int AT_D = 512;
constexpr int AT_ROWS = 32;
constexpr int AT_ROWB = AT_D * 2;
constexpr int AT_TILE_B = AT_ROWS * AT_ROWB;
constexpr int AT_NST = 4;         // ring stages
constexpr int AT_MAXK = 2048;     // sparse lists up to this many entries
constexpr int AT_MAXWIN = 1024;   // windows up to this many rows
constexpr int AT_LIST = AT_MAXWIN + AT_MAXK;  // candidate slots resolved in LDS
constexpr float LOG2E = 1.4426950408889634f;
constexpr float AT_SLACK = 16.f;  // log2 headroom of the lazily updated running max

template <int HG>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a, int n_hg, int total_items) {
  constexpr int NHW = HG / 16;
  constexpr int NDQ = 4 / NHW;
  constexpr int DS = AT_D / NDQ;
  constexpr int KSTEPS = DS / 32;
  constexpr int DTILES = DS / 16;
  __shared__ __attribute__((aligned(16))) uint8_t ring[AT_NST][AT_TILE_B];
  __shared__ __attribute__((aligned(16))) float xch[2][4][2][256];
  __shared__ __attribute__((aligned(16))) int32_t s_rows[AT_LIST];
  __shared__ uint32_t s_mask[AT_LIST / AT_ROWS];
  __shared__ float2 rope_cs[AT_D / 2];

  const int item = xcd_remap(blockIdx.x, total_items);
  const int qi = item / n_hg, hgi = item % n_hg;
  const int b = qi / a.S, s = qi % a.S;
  const int t = a.q_pos[b] + s;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int hw = wave % NHW, dq = wave / NHW;
  const int h0 = hgi * HG + hw * 16;
  const int d0 = dq * DS;
  const int nwin = max(0, min(t + 1, a.window));
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const int ncand = nwin + ncmp;
  const int ntiles = (ncand + AT_ROWS - 1) / AT_ROWS;
  const bf16* win = (const bf16*)a.win + (size_t)b * a.W_cap * AT_D;
  const bf16* cmp = (const bf16*)a.cmp + (size_t)b * a.N_cap * AT_D;

  // q fragments (head h0 + n, dims d0 + 32*kk + 8*g .. +8) and the sink.
  bf16x8_t qf[KSTEPS];
  {
    const bf16* qrow = (const bf16*)a.q + ((size_t)qi * a.H + h0 + n) * AT_D + d0 + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
  }
  const float sink = a.sink[h0 + n];

  // Candidate slots resolved once per query into LDS: s_rows[j] >= 0 is
  // compressed entry s_rows[j], < 0 is window row -1 - s_rows[j].  Skipped
  // slots (padding, out-of-range ids, the ragged tail) point at window row 0
  // and have their bit cleared in the per-tile validity mask s_mask.  Dense
  // candidates beyond the table are computed on the fly (all valid).
  const int nlist = min(ntiles * AT_ROWS, AT_LIST);
  for (int j0 = wave * 64; j0 < nlist; j0 += 256) {
    const int j = j0 + lane;
    int id = -1;
    bool ok = false;
    if (j < nwin) {
      const int u = t - nwin + 1 + j;
      const int rw = a.win_pos0 ? u - a.win_pos0[b] : u % a.W_cap;
      ok = rw >= 0 && rw < a.W_cap;
      id = ok ? -1 - rw : -1;
    } else if (j < ncand) {
      const int e = a.dense ? j - nwin : a.topk_idx[(size_t)qi * a.k + (j - nwin)];
      ok = e >= 0 && e < a.N_cap;
      id = ok ? e : -1;
    }
    if (j < nlist) s_rows[j] = id;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
    if (lane == 0) {
      s_mask[j0 / AT_ROWS] = (uint32_t)bal;
      s_mask[j0 / AT_ROWS + 1] = (uint32_t)(bal >> 32);
    }
  }
  // Every ordinary load is complete before the first tile copy: the compiler
  // then has no pending load to wait for inside the tile loop (such a wait
  // would be vmcnt(0) and drain the ring).
  WAIT_VMCNT(0);
  __syncthreads();

  // per-lane copy offsets of this wave's 8 rows (row r = 8*wave + rr of a tile)
  uint32_t loff[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) loff[rr] = 16u * (uint32_t)(lane ^ ((8 * wave + rr) & 15));

  const char* cmpb = (const char*)cmp;
  const char* winb = (const char*)win;
  auto issue = [&](int ti) {
    const int st = ti & (AT_NST - 1);
    const int jb = ti * AT_ROWS + 8 * wave;  // first slot this wave copies (multiple of 8)
    int ids[8];
    if (jb + 8 <= nlist) {
      const int4 v0 = *(const int4*)&s_rows[jb];
      const int4 v1 = *(const int4*)&s_rows[jb + 4];
      ids[0] = v0.x; ids[1] = v0.y; ids[2] = v0.z; ids[3] = v0.w;
      ids[4] = v1.x; ids[5] = v1.y; ids[6] = v1.z; ids[7] = v1.w;
    } else {  // dense candidates past the table (jb >= nlist >= nwin here)
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) ids[rr] = (jb + rr < ncand) ? jb + rr - nwin : 0;
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int id = __builtin_amdgcn_readfirstlane(ids[rr]);
      const bool isw = id < 0;
      const char* row = (isw ? winb : cmpb) + (size_t)(uint32_t)(isw ? -1 - id : id) * AT_ROWB;
      dma16_sbase(row, loff[rr], &ring[st][(8 * wave + rr) * AT_ROWB]);
    }
  };
  // partial logits of tile ti over this wave's dims (rows n and 16 + n)
  auto qk = [&](int ti, f32x4_t& s0, f32x4_t& s1) {
    const uint8_t* tile = ring[ti & (AT_NST - 1)];
    s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int c = (d0 + 32 * kk) / 8 + g;
      const bf16x8_t a0 = *(const bf16x8_t*)(tile + n * AT_ROWB + 16 * (c ^ n));
      const bf16x8_t a1 = *(const bf16x8_t*)(tile + (16 + n) * AT_ROWB + 16 * (c ^ n));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[kk], s1, 0, 0, 0);
    }
  };
  auto xwrite = [&](int ti, const f32x4_t& s0, const f32x4_t& s1) {
    if constexpr (NDQ > 1) {
      float* xw = &xch[ti & 1][wave][0][0];
      *(f32x4_t*)(xw + lane * 4) = s0;
      *(f32x4_t*)(xw + 256 + lane * 4) = s1;
    }
  };
  auto xread = [&](int ti, f32x4_t& s0, f32x4_t& s1) {
    if constexpr (NDQ > 1) {
      s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q2 = 0; q2 < NDQ; ++q2) {
        const float* xo = &xch[ti & 1][hw + NHW * q2][0][0];
        s0 += *(const f32x4_t*)(xo + lane * 4);
        s1 += *(const f32x4_t*)(xo + 256 + lane * 4);
      }
    }
  };

  const float sc2 = a.scale * LOG2E;
  // Running max (log2 domain) starts at the sink logit, whose exp2(0) = 1 is
  // counted once per head (lane group 0) in the per-lane partial sums.
  float m_run = sink * LOG2E;
  float l_run = (sink == -INFINITY || g != 0) ? 0.f : 1.f;
  f32x4_t o[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // prologue: tiles 0..3 in flight; tiles 0 and 1 resident; logits of tile 0
  f32x4_t S0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0;
#pragma unroll
  for (int p = 0; p < AT_NST; ++p)
    if (p < ntiles) issue(p);
  // de-rotation table for the epilogue, computed while the first tiles land
  // (visible to all waves after the next barrier)
  for (int p = threadIdx.x; p < a.rope_dim / 2; p += 256) {
    float c, sn;
    rope_cos_sin((double)t, p, a.rope_dim, a.base, &c, &sn);
    rope_cs[p] = make_float2(c, sn);
  }
  if (ntiles > 0) {
    const int beyond1 = min(2, max(0, ntiles - 2));  // tiles 2, 3 may stay in flight
    if (beyond1 == 2)
      WAIT_VMCNT(16);
    else if (beyond1 == 1)
      WAIT_VMCNT(8);
    else
      WAIT_VMCNT(0);
    lds_barrier();
    qk(0, S0, S1);
    xwrite(0, S0, S1);
    lds_barrier();
    xread(0, S0, S1);
  }

  const int trow = 4 * g + (n >> 2);  // row of this lane's transposed-read address
  for (int i = 0; i < ntiles; ++i) {
    // 1. logits of the next tile (resident since the previous barrier)
    f32x4_t N0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, N1 = N0;
    const bool has_next = i + 1 < ntiles;
    if (has_next) qk(i + 1, N0, N1);

    // 2. online softmax of tile i (lane: head n; rows 4g+ii and 16+4g+ii).
    //    The running max m_run is shared by the 4 lanes of a head; the sum is
    //    kept per lane and reduced once at the end.  A tile only moves m_run
    //    (cross-lane max + rescale) when one of its logits exceeds m_run by
    //    more than 2^SLACK: exp2(s - m_run) then stays below 2^SLACK, which
    //    neither overflows nor costs precision, and most tiles skip the
    //    cross-lane work entirely.
    const int st = i & (AT_NST - 1);
    uint32_t vmask;
    if (i * AT_ROWS < nlist) {
      vmask = s_mask[i];
    } else {  // dense tail past the table: every slot below ncand is valid
      const int left = ncand - i * AT_ROWS;
      vmask = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
    }
    float sv[8];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      sv[ii] = ((vmask >> (4 * g + ii)) & 1u) ? S0[ii] * sc2 : -INFINITY;
      sv[4 + ii] = ((vmask >> (16 + 4 * g + ii)) & 1u) ? S1[ii] * sc2 : -INFINITY;
    }
    float lm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    if (__builtin_amdgcn_ballot_w64(lm > m_run + AT_SLACK)) {  // wave-uniform, rare
      float mt = fmaxf(lm, __shfl_xor(lm, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // m_new is finite here
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    // m_run is -inf only while every logit seen so far is masked (sink -inf):
    // then all sv are -inf and the reference point 0 gives p == 0, not NaN.
    const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8_t pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(sv[j] - m_ref);  // exp2(-inf) == 0 for masked slots
      l_run += p;
      pf[j] = (__bf16)p;
    }

    // 3. O^T += R^T P^T over this wave's dims
    const uint8_t* trp = ring[st] + trow * AT_ROWB;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const int dim = d0 + 16 * dt + 4 * (n & 3);
      const int c = dim >> 3, half = (dim >> 2) & 1;
      const uint8_t* p1 = trp + 16 * (c ^ (trow & 15)) + 8 * half;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p1));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(p1 + 16 * AT_ROWB));
      const bf16x8_t afr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, pf, o[dt], 0, 0, 0);
    }

    // 4. publish the next tile's partial logits; make tile i+2 resident
    if (has_next) xwrite(i + 1, N0, N1);
    if (i + 3 < ntiles)
      WAIT_VMCNT(8);  // tile i+3 may stay in flight
    else
      WAIT_VMCNT(0);
    lds_barrier();
    if (i + AT_NST < ntiles) issue(i + AT_NST);  // into tile i's stage, free now
    if (has_next) {
      if constexpr (NDQ > 1)
        xread(i + 1, S0, S1);
      else {
        S0 = N0;
        S1 = N1;
      }
    }
  }

  // epilogue: normalise, de-rotate the RoPE tail at position t, store
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.f / l_run;
  const int tail0 = AT_D - a.rope_dim;
  bf16* outp = (bf16*)a.out + ((size_t)qi * a.H + h0 + n) * AT_D;
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) {
    const int dim = d0 + 16 * dt + 4 * g;
    float v[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) v[ii] = o[dt][ii] * inv_l;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (dim + 2 * pp >= tail0) {
        const float2 cs = rope_cs[(dim + 2 * pp - tail0) / 2];
        const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
        v[2 * pp] = x0 * cs.x + x1 * cs.y;
        v[2 * pp + 1] = -x0 * cs.y + x1 * cs.x;
      }
    }
    uint2 pk;
    pk.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    pk.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *(uint2*)(outp + dim) = pk;
  }
  if (a.lse && dq == 0 && g == 0) a.lse[(size_t)qi * a.H + h0 + n] = (m_run + log2f(l_run)) / LOG2E;
}

// ---------------------------------------------------------------------------
// Row-split MFMA kernel for groups of 16 heads (decode batches too small to
// give each workgroup more heads).  bf16, D == 512.
//
// Work item = (query, 16 heads), XCD-aware like the kernel above.  Tiles hold
// 64 candidate rows.  Wave w loads ITS 16 rows of each tile straight into
// VGPRs in the MFMA A layout (lane (row n, group g) holds 16 bytes per 32-dim
// step), one tile ahead, and computes those rows' logits over all 512 dims:
// no partial-logit exchange.  It then writes the rows once to LDS, and after
// the tile's single barrier every wave reads its 128-dim slice of all 64 rows
// transposed (ds_read_b64_tr_b16) for O^T += R^T P^T: each row byte crosses
// LDS twice instead of three times.  P (bf16, [head][row]) is shared through
// LDS.  The running max is common to all waves and moves lazily: a tile whose
// logits exceed it by more than 2^SLACK raises a flag and every wave takes a
// rare exact rescale path (second barrier).  Row LDS layout: 16-byte granule
// c of row r sits at c ^ swz(r), swz(r) = 2*(r & 7) + ((r >> 3) & 1), which
// keeps both the row writes and the transposed reads free of bank conflicts.
constexpr int AR_TR = 64;  // rows per tile

__device__ __forceinline__ int ar_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__global__ __launch_bounds__(256) void attn_rows16_kernel(AttnArgs a, int n_hg, int total_items) {
  __shared__ __attribute__((aligned(16))) uint8_t tbuf[2][AR_TR * AT_ROWB];
  __shared__ __attribute__((aligned(16))) __bf16 pbuf[2][16][AR_TR];
  __shared__ float mbuf[2][4][64];
  __shared__ uint32_t fbuf[2][4];
  __shared__ float lbuf[4][64];
  __shared__ __attribute__((aligned(16))) int32_t s_rows[AT_LIST];
  __shared__ uint64_t s_mask[AT_LIST / AR_TR];
  __shared__ float2 rope_cs[AT_D / 2];

  const int item = xcd_remap(blockIdx.x, total_items);
  const int qi = item / n_hg, hgi = item % n_hg;
  const int b = qi / a.S, s = qi % a.S;
  const int t = a.q_pos[b] + s;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int h0 = hgi * 16;
  const int d0 = wave * 128;  // P.V dim slice of this wave
  const int nwin = max(0, min(t + 1, a.window));
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const int ncand = nwin + ncmp;
  const int ntiles = (ncand + AR_TR - 1) / AR_TR;
  const char* winb = (const char*)a.win + (size_t)b * a.W_cap * AT_ROWB;
  const char* cmpb = (const char*)a.cmp + (size_t)b * a.N_cap * AT_ROWB;

  // q fragments for QK^T (B operand): head h0 + n, dims 32*kk + 8*g .. +8
  bf16x8_t qf[16];
  {
    const bf16* qrow = (const bf16*)a.q + ((size_t)qi * a.H + h0 + n) * AT_D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
  }
  const float sink = a.sink[h0 + n];

  // candidate slots -> row ids (>= 0: compressed entry, < 0: window row -1-id)
  // and per-tile validity masks (bit j of s_mask[tile]: slot tile*64 + j)
  const int nlist = min(ntiles * AR_TR, AT_LIST);
  for (int j0 = wave * 64; j0 < nlist; j0 += 256) {
    const int j = j0 + lane;
    int id = -1;
    bool ok = false;
    if (j < nwin) {
      const int u = t - nwin + 1 + j;
      const int rw = a.win_pos0 ? u - a.win_pos0[b] : u % a.W_cap;
      ok = rw >= 0 && rw < a.W_cap;
      id = ok ? -1 - rw : -1;
    } else if (j < ncand) {
      const int e = a.dense ? j - nwin : a.topk_idx[(size_t)qi * a.k + (j - nwin)];
      ok = e >= 0 && e < a.N_cap;
      id = ok ? e : -1;
    }
    if (j < nlist) s_rows[j] = id;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
    if (lane == 0) s_mask[j0 / AR_TR] = bal;
  }
  __syncthreads();

  // this lane's row of tile ti: slot ti*64 + 16*wave + n; 16 bytes per 32-dim step
  auto row_base = [&](int ti) -> const char* {
    const int j = ti * AR_TR + 16 * wave + n;
    int id;
    if (j < nlist)
      id = s_rows[j];
    else
      id = (j < ncand) ? j - nwin : 0;  // dense candidates past the table (or masked tail)
    const char* p = id >= 0 ? cmpb + (size_t)id * AT_ROWB : winb + (size_t)(-1 - id) * AT_ROWB;
    return p + 16 * g;
  };
  auto load_rows = [&](int ti, bf16x8_t (&R)[16]) {
    const char* p = row_base(ti);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) R[kk] = *(const bf16x8_t*)(p + 64 * kk);
  };
  auto tile_mask = [&](int ti) -> uint64_t {
    if (ti * AR_TR < nlist) return s_mask[ti];
    const int left = ncand - ti * AR_TR;  // dense tail past the table
    return left >= 64 ? ~0ull : ((1ull << left) - 1ull);
  };

  // de-rotation table (visible after the first tile barrier)
  for (int p = threadIdx.x; p < a.rope_dim / 2; p += 256) {
    float c, sn;
    rope_cos_sin((double)t, p, a.rope_dim, a.base, &c, &sn);
    rope_cs[p] = make_float2(c, sn);
  }

  const float sc2 = a.scale * LOG2E;
  // running max shared by all lanes of a head in all waves; partial sums per
  // lane (the sink's exp2(0) = 1 counted once: wave 0, lane group 0)
  float m_run = sink * LOG2E;
  float l_run = (sink == -INFINITY || wave != 0 || g != 0) ? 0.f : 1.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int myrow = 16 * wave + n;           // row this lane loads (within a tile)
  const int wswz = ar_swz(myrow);
  const int trow = 8 * g + (n >> 2);         // transposed-read row for k-chunk 0 (add 32c, +4)
  bf16x8_t Ra[16], Rb[16];

  auto tile_step = [&](int i, bf16x8_t (&R)[16], bf16x8_t (&Rn)[16]) {
    const int buf = i & 1;
    if (i + 1 < ntiles) load_rows(i + 1, Rn);  // prefetch into registers
    // 1. logits of this wave's 16 rows for the 16 heads (two MFMA chains)
    f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int kk = 0; kk < 16; kk += 2) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(R[kk], qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(R[kk + 1], qf[kk + 1], s1, 0, 0, 0);
    }
    // 2. rows -> LDS for the transposed P.V reads
    uint8_t* tb = tbuf[buf];
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      *(bf16x8_t*)(tb + myrow * AT_ROWB + 16 * ((4 * kk + g) ^ wswz)) = R[kk];
    // 3. P with the current running max; lane (head n, group g): rows 16w+4g+ii
    const f32x4_t S = s0 + s1;
    const uint32_t vb = (uint32_t)(tile_mask(i) >> (16 * wave + 4 * g)) & 0xFu;
    float sv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sv[ii] = ((vb >> ii) & 1u) ? S[ii] * sc2 : -INFINITY;
    const float lm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    const bool moved = __builtin_amdgcn_ballot_w64(lm > m_run + AT_SLACK) != 0;
    float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
    float pv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) pv[ii] = __builtin_amdgcn_exp2f(sv[ii] - m_ref);
    {
      __attribute__((ext_vector_type(4))) __bf16 pk;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) pk[ii] = (__bf16)pv[ii];
      *(decltype(pk)*)&pbuf[buf][n][16 * wave + 4 * g] = pk;
    }
    mbuf[buf][wave][lane] = lm;
    if (lane == 0) fbuf[buf][wave] = moved ? 1u : 0u;
    __syncthreads();  // rows, P and flags of all waves visible; stage buf^1 no longer read
    if (fbuf[buf][0] | fbuf[buf][1] | fbuf[buf][2] | fbuf[buf][3]) {
      // rare: some logit left the running max's headroom -> exact rescale
      float mt = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
        for (int g2 = 0; g2 < 4; ++g2) mt = fmaxf(mt, mbuf[buf][w2][16 * g2 + n]);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run == -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      m_run = m_new;
      m_ref = (m_run == -INFINITY) ? 0.f : m_run;
      __attribute__((ext_vector_type(4))) __bf16 pk;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        pv[ii] = __builtin_amdgcn_exp2f(sv[ii] - m_ref);
        pk[ii] = (__bf16)pv[ii];
      }
      *(decltype(pk)*)&pbuf[buf][n][16 * wave + 4 * g] = pk;
      __syncthreads();
    }
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    // 4. O^T[128 dims x 16 heads] += R^T[128 x 64 rows] P^T[64 rows x 16 heads]
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8_t pf = *(const bf16x8_t*)&pbuf[buf][n][32 * c + 8 * g];
      const int ra = 32 * c + trow, rb = ra + 4;
      const uint8_t* pa = tb + ra * AT_ROWB;
      const uint8_t* pb = tb + rb * AT_ROWB;
      const int sa = ar_swz(ra), sb = ar_swz(rb);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int dim = d0 + 16 * dt + 4 * (n & 3);
        const int gr = dim >> 3, half = (dim >> 2) & 1;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4_t*)(pa + 16 * (gr ^ sa) + 8 * half));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4_t*)(pb + 16 * (gr ^ sb) + 8 * half));
        const bf16x8_t afr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, pf, o[dt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) load_rows(0, Ra);
  for (int i = 0; i < ntiles; i += 2) {
    tile_step(i, Ra, Rb);
    if (i + 1 < ntiles) tile_step(i + 1, Rb, Ra);
  }

  // epilogue: total sum per head (lane groups, then waves), normalise, de-rotate, store
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  lbuf[wave][lane] = l_run;
  __syncthreads();
  const float l_tot = lbuf[0][n] + lbuf[1][n] + lbuf[2][n] + lbuf[3][n];
  const float inv_l = 1.f / l_tot;
  const int tail0 = AT_D - a.rope_dim;
  bf16* outp = (bf16*)a.out + ((size_t)qi * a.H + h0 + n) * AT_D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int dim = d0 + 16 * dt + 4 * g;
    float v[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) v[ii] = o[dt][ii] * inv_l;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      if (dim + 2 * pp >= tail0) {
        const float2 cs = rope_cs[(dim + 2 * pp - tail0) / 2];
        const float x0 = v[2 * pp], x1 = v[2 * pp + 1];
        v[2 * pp] = x0 * cs.x + x1 * cs.y;
        v[2 * pp + 1] = -x0 * cs.y + x1 * cs.x;
      }
    }
    uint2 pk;
    pk.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    pk.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *(uint2*)(outp + dim) = pk;
  }
  if (a.lse && wave == 0 && g == 0) a.lse[(size_t)qi * a.H + h0 + n] = (m_run + log2f(l_tot)) / LOG2E;
}

}  // namespace csa

namespace csa_host {
using namespace csa;

size_t attn_workspace_size(int, int, int, int, int) { return 0; }

hipError_t launch_attn(const void* q, const void* cmp, const int32_t* topk_idx, int k, int dense, int ratio,
                       const void* win,
                       const int32_t* win_pos0, const float* sink, const int32_t* q_pos, void* out, float* lse,
                       void* ws, int B, int S, int H, int D, int rope_dim, int N_cap, int W_cap, int window,
                       float scale, float base, int dtype, hipStream_t st) {
  (void)ws;
  AttnArgs a{q, cmp, topk_idx, win, win_pos0, sink, q_pos, out, lse, dense, S, H, D, rope_dim, N_cap, k, ratio,
             W_cap, window, scale, base};
  const long Q = (long)B * S;
  if (dtype == CSA_BF16 && D == AT_D && H % 16 == 0 && (dense || k <= AT_MAXK) && window <= AT_MAXWIN) {
    // widest head group that still gives >= 256 work items (one per CU)
    int HG = (H % 64 == 0) ? 64 : (H % 32 == 0) ? 32 : 16;
    while (HG > 16 && Q * (H / HG) < 256) HG /= 2;
    const int n_hg = H / HG;
    const int total = (int)(Q * n_hg);
    if (HG == 64)
      hipLaunchKernelGGL((attn_mfma_kernel<64>), dim3(total), dim3(256), 0, st, a, n_hg, total);
    else if (HG == 32)
      hipLaunchKernelGGL((attn_mfma_kernel<32>), dim3(total), dim3(256), 0, st, a, n_hg, total);
    else
      hipLaunchKernelGGL(attn_rows16_kernel, dim3(total), dim3(256), 0, st, a, n_hg, total);
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
