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
// Work item = (query, group of HG heads); the item -> block map is
// XCD-aware so all head groups of one query share an L2 and its gathered rows
// come from HBM once.  Workgroup = 4 waves; wave w owns heads
// [16*(w % NHW), +16) of the group and the dim slice [DS*(w / NHW), +DS),
// NHW = HG/16, DS = 512*NHW/4.
//
// Candidates stream in tiles of 32 rows (32 KiB) through an NSTAGE-deep LDS
// ring filled by direct global->LDS loads (one 1 KiB row per wave
// instruction; each wave loads 8 rows per tile).  Per tile and wave:
//   S^T[32 rows x 16 heads] = R . Q^T over the wave's dims (MFMA 16x16x32, A =
//     rows from LDS, B = q fragments held in VGPRs); partial sums of the waves
//     sharing a head group are added through LDS, so every wave sees the same
//     logits and keeps identical softmax statistics;
//   online softmax in the exp2 domain; the sink seeds the running max/sum;
//   O^T[DS dims x 16 heads] += R^T . P^T (A = rows read transposed with
//     ds_read_b64_tr_b16, B = P^T straight from the S^T accumulator lanes).
// Rows are XOR-swizzled in LDS (16 B granule c of row r at c ^ (r & 15)).
// The epilogue divides by the sum, de-rotates the RoPE tail at the query
// position and stores bf16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n)&15) | (((n) >> 4) << 14)) | 0x0F70)

constexpr int AT_D = 512;
constexpr int AT_ROWS = 32;
constexpr int AT_ROWB = AT_D * 2;
constexpr int AT_TILE_B = AT_ROWS * AT_ROWB;
constexpr int AT_MAXK = 2048;
constexpr float LOG2E = 1.4426950408889634f;

template <int HG, int NSTAGE>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnArgs a, int n_hg, int total_items) {
  constexpr int NHW = HG / 16;
  constexpr int NDQ = 4 / NHW;
  constexpr int DS = AT_D / NDQ;
  constexpr int KSTEPS = DS / 32;
  constexpr int DTILES = DS / 16;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NSTAGE][AT_TILE_B];
  __shared__ __attribute__((aligned(16))) float xch[2][4][2][256];
  __shared__ __attribute__((aligned(16))) int32_t s_idx[AT_MAXK];
  __shared__ float2 rope_cs[AT_D / 2];
  __shared__ __attribute__((aligned(4))) uint8_t tmask[NSTAGE][4];

  const int item = xcd_remap(blockIdx.x, total_items);
  const int qi = item / n_hg, hgi = item % n_hg;
  const int b = qi / a.S, s = qi % a.S;
  const long t = (long)a.q_pos[b] + s;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int hw = wave % NHW, dq = wave / NHW;
  const int h0 = hgi * HG + hw * 16;
  const int d0 = dq * DS;
  const int nwin = (int)(t + 1 < a.window ? t + 1 : a.window);
  const int ncmp = a.dense ? (int)visible_entries(t, a.ratio, a.N_cap) : a.k;
  const int ncand = (nwin > 0 ? nwin : 0) + ncmp;
  const int ntiles = (ncand + AT_ROWS - 1) / AT_ROWS;
  const bf16* win = (const bf16*)a.win + (size_t)b * a.W_cap * AT_D;
  const bf16* cmp = (const bf16*)a.cmp + (size_t)b * a.N_cap * AT_D;
  const long wp0 = a.win_pos0 ? (long)a.win_pos0[b] : 0;

  // candidate list and RoPE table into LDS
  if (!a.dense)
    for (int j = threadIdx.x; j < a.k; j += 256) s_idx[j] = a.topk_idx[(size_t)qi * a.k + j];
  for (int p = threadIdx.x; p < a.rope_dim / 2; p += 256) {
    float c, sn;
    rope_cos_sin((double)t, p, a.rope_dim, a.base, &c, &sn);
    rope_cs[p] = make_float2(c, sn);
  }
  // q fragments: head h0 + n, dims d0 + 32*kk + 8*g .. +8
  bf16x8_t qf[KSTEPS];
  {
    const bf16* qrow = (const bf16*)a.q + ((size_t)qi * a.H + h0 + n) * AT_D + d0 + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = *(const bf16x8_t*)(qrow + 32 * kk);
  }
  __syncthreads();

  // this wave loads rows 8*wave .. 8*wave+7 of tile ti into stage st
  auto issue = [&](int ti, int st) {
    uint32_t vm = 0;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 8 * wave + rr;
      const int j = ti * AT_ROWS + r;
      const bf16* row = win;  // placeholder row (masked) for empty slots
      bool valid = false;
      if (j < nwin) {
        const long u = t - nwin + 1 + j;
        const long rw = a.win_pos0 ? u - wp0 : u % a.W_cap;
        if (rw >= 0 && rw < a.W_cap) {
          row = win + rw * AT_D;
          valid = true;
        }
      } else if (j < ncand) {
        const int jj = j - nwin;
        const long e = a.dense ? (long)jj : (long)s_idx[jj];
        if (e >= 0 && e < a.N_cap) {
          row = cmp + e * AT_D;
          valid = true;
        }
      }
      vm |= (valid ? 1u : 0u) << rr;
      const int c = lane ^ (r & 15);
      __builtin_amdgcn_global_load_lds((const void*)(row + 8 * c), LDS_PTR(&tiles[st][r * AT_ROWB]), 16, 0, 0);
    }
    if (lane == 0) tmask[st][wave] = (uint8_t)vm;
  };

#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p)
    if (p < ntiles) issue(p, p);

  const float sink = a.sink[h0 + n];
  const float sc2 = a.scale * LOG2E;
  float m_run = sink * LOG2E;  // running max, log2 domain
  float l_run = (sink == -INFINITY) ? 0.f : 1.f;
  f32x4_t o[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < ntiles; ++i) {
    const int st = i % NSTAGE;
    const int ahead = min(NSTAGE - 2, ntiles - 1 - i);
    if (ahead >= 2)
      WAIT_VMCNT(16);
    else if (ahead == 1)
      WAIT_VMCNT(8);
    else
      WAIT_VMCNT(0);
    __syncthreads();  // tile i is in LDS for everyone; stage (i-1) % NSTAGE is free
    if (i + NSTAGE - 1 < ntiles) issue(i + NSTAGE - 1, (i + NSTAGE - 1) % NSTAGE);
    const uint8_t* tile = tiles[st];

    // logits over this wave's dims
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint8_t* rowp = tile + (16 * rt + n) * AT_ROWB;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int c = (d0 + 32 * kk) / 8 + g;
        const bf16x8_t afr = *(const bf16x8_t*)(rowp + 16 * (c ^ n));
        sacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, qf[kk], sacc[rt], 0, 0, 0);
      }
    }
    if constexpr (NDQ > 1) {
      float* xw = &xch[i & 1][wave][0][0];
      *(f32x4_t*)(xw + lane * 4) = sacc[0];
      *(f32x4_t*)(xw + 256 + lane * 4) = sacc[1];
      __syncthreads();
      sacc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q2 = 0; q2 < NDQ; ++q2) {
        const float* xo = &xch[i & 1][hw + NHW * q2][0][0];
        sacc[0] += *(const f32x4_t*)(xo + lane * 4);
        sacc[1] += *(const f32x4_t*)(xo + 256 + lane * 4);
      }
    }

    // online softmax (lane: head n; rows 4g+ii and 16+4g+ii of the tile)
    const uint32_t vmask = *(const uint32_t*)tmask[st];
    float sv[8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 16 * rt + 4 * g + ii;
        sv[4 * rt + ii] = ((vmask >> r) & 1u) ? sacc[rt][ii] * sc2 : -INFINITY;
      }
    float mt = sv[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, sv[j]);
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float ps = 0.f;
    bf16x8_t pf;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(sv[j] - m_use);
      ps += p;
      pf[j] = (__bf16)p;
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;

    // O^T += R^T P^T over this wave's dims
    const int trow = 4 * g + (n >> 2);
    const uint8_t* trp = tile + trow * AT_ROWB;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) {
      const int dim = d0 + 16 * dt + 4 * (n & 3);
      const int c = dim >> 3, half = (dim >> 2) & 1;
      const uint8_t* p1 = trp + 16 * (c ^ (trow & 15)) + 8 * half;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(p1));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)(p1 + 16 * AT_ROWB));
      const bf16x8_t afr = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] *= alpha;
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, pf, o[dt], 0, 0, 0);
    }
  }

  // epilogue: normalise, de-rotate the RoPE tail at position t, store
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
  if (dtype == CSA_BF16 && D == AT_D && H % 16 == 0 && (dense || k <= AT_MAXK)) {
    // widest head group that still gives >= 256 work items (one per CU)
    int HG = (H % 64 == 0) ? 64 : (H % 32 == 0) ? 32 : 16;
    while (HG > 16 && Q * (H / HG) < 256) HG /= 2;
    const int n_hg = H / HG;
    const int total = (int)(Q * n_hg);
    if (HG == 64)
      hipLaunchKernelGGL((attn_mfma_kernel<64, 4>), dim3(total), dim3(256), 0, st, a, n_hg, total);
    else if (HG == 32)
      hipLaunchKernelGGL((attn_mfma_kernel<32, 4>), dim3(total), dim3(256), 0, st, a, n_hg, total);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<16, 4>), dim3(total), dim3(256), 0, st, a, n_hg, total);
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
