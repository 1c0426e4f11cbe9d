// proj.hip -- the projections around the attention: low-rank Q and the
// grouped output projection.
//
// "DeepSeek-V4-Pro 架构：一个 token 的旅程", section "低秩 Q：两次矩阵乘法接起来":
//   qr = RMSNorm(X Wq_a^T) (gain gamma_q)   X [M, d_model], Wq_a [q_rank, d_model]
//   q  = (qr Wq_b^T) as [M, H, D]           Wq_b [H*D, q_rank]
//   each head divided by sqrt(mean(q^2 over D) + eps), then RoPE on its last
//   rope_dim dims at the token's position.
// Section "输出投影也分组，并且降低中间维度":
//   o (attention output, inverse RoPE already applied) as [M, groups, H*D/groups]
//   r[:, g] = o[:, g] Wo_a[g]^T             Wo_a [groups, o_rank, H*D/groups]
//   y = r (flattened, group-major) Wo_b^T   Wo_b [d_model, groups*o_rank]
// M = B*S rows.  Operands bf16, accumulation fp32, qr / q / r / y stored bf16.
//
// Weights are used in a packed layout (csa_pack_weights): a matrix W [N][K]
// becomes blocks of 16 columns x 512 dims, block (c, h) at element offset
// (c * K/512 + h) * 8192, holding for k-step j (32 dims) and lane (g, n) the
// eight values W[16c + n][512h + 32j + 8g .. +8] at (j * 64 + 16g + n) * 8:
// exactly the MFMA B-operand order of v_mfma_f32_16x16x32_bf16.  A wave that
// owns 16 columns and a K split then reads one contiguous run, 1 KiB per
// load instruction.  (HBM3E on this part streams fastest as a few long
// contiguous runs per CU; rows read 64 bytes at a time across 16 rows of a
// row-major weight run measurably slower.)
//
// gemm_nt_kernel computes split-K partials C[g][ks][m][n] = sum over k in
// split ks of A_g[m][k] W_g[n][k].  At decode M is a few dozen rows and every
// weight is read once, so the kernel is an HBM stream of the weights:
//   * about one workgroup per CU; a workgroup owns rows [m0, m0+TM), one K
//     split of KC dims and a contiguous range of 64-column tiles;
//   * it copies its A slab (TM x KC bf16, up to 128 KiB) into LDS once, with
//     direct global->LDS copies, and reuses it for all of its tiles;
//   * each of its 4 waves streams the packed run of its 16 columns into MFMA
//     B fragments, PF k-steps of loads in flight, the ring running on across
//     tile boundaries so the stream never drains between tiles.
// The host picks KC and the tiles per workgroup from a small cost model
// (busiest CU's weight bytes + partial traffic + A slab copies).  Split-K
// partials are fp32 and summed in split order by rows_finish_kernel, so
// results do not depend on scheduling.
//
// rows_finish_kernel: per output row and segment of `seg` columns, the sum of
// the splits, then optionally an RMS normalisation over the segment (times a
// gain when given), optionally RoPE on the segment's last rope_dim dims at the
// row's position, and the bf16 store.  The finishing pass reads the fp32
// partials once, coalesced, with a batch of splits in flight per thread.
#include "common.hpp"

#include <atomic>
#include <cmath>

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int PJ_NW = 4;           // waves per workgroup
constexpr int PJ_TN = 16 * PJ_NW;  // columns per tile (16 per wave)
constexpr int PJ_CUS = 256;        // workgroups the plan aims for (one per CU)
constexpr int PJ_PF = 16;  // k-steps (32 dims each) of weight loads in flight per wave
// Every split holds whole 512-dim chunks (16 k-steps); the loop runs in
// blocks of PJ_PF steps and its loads run PJ_PF steps ahead, so PJ_PF must
// divide 16 or the last block would read past the split (and, in the last
// split of the last weight row, past the weights).
static_assert(PJ_PF >= 1 && 16 % PJ_PF == 0, "PJ_PF must divide the 16 k-steps of a 512-dim chunk");

struct GemmArgs {
  const bf16* A;   // [groups] x [M][lda]
  const bf16* Bp;  // [groups] x packed W [N][K]
  float* C;        // [groups][ksplit][M][N]
  int M, N, K, lda;
  long sa, sb;     // group strides (elements) of A and of the packed weights
  int kc, ksplit, ntiles, tpw, gx, mtiles, groups;
};

// LDS bytes per A row: 16 bytes of padding puts rows n and n+1 four banks
// apart, so the 16 lanes of a ds_read_b128 phase hit 64 distinct banks.
__host__ __device__ constexpr int pj_row_bytes(int kc) { return 2 * kc + 16; }

template <int TM>
__global__ __launch_bounds__(64 * PJ_NW) void gemm_nt_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_a[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, gq = lane >> 4, n = lane & 15;
  // 1-D grid, remapped so that the workgroups sharing an A slab (same split,
  // row tile and group; consecutive bx) run on one XCD and share its L2
  const int rows = g.ksplit * g.mtiles;
  const int L = xcd_remap((int)blockIdx.x, g.gx * rows * g.groups);
  const int bx = L % g.gx, by = (L / g.gx) % rows, grp = L / (g.gx * rows);
  const int ks = by % g.ksplit, mt = by / g.ksplit;
  const int m0 = mt * TM, k0 = ks * g.kc;
  const int kn = min(g.kc, g.K - k0);  // a multiple of 512 (K and kc are)
  const int nstep = kn >> 5;           // a multiple of 16, so of PJ_PF
  const int AS = pj_row_bytes(g.kc);
  const bf16* A = g.A + grp * g.sa;
  const bf16* Bp = g.Bp + grp * g.sb;
  const int t0 = bx * g.tpw, t1 = min(t0 + g.tpw, g.ntiles);

  // A slab -> LDS, 1 KiB (512 dims) per copy; rows past M are zero
  const int chunks = kn >> 9;
  for (int idx = wave; idx < TM * chunks; idx += PJ_NW) {
    const int r = idx / chunks, c = idx - r * chunks;
    uint8_t* dst = lds_a + r * AS + 1024 * c;
    if (m0 + r < g.M)
      dma16_sbase((const char*)(A + (size_t)(m0 + r) * g.lda + k0 + 512 * c), 16u * (uint32_t)lane, dst);
    else
      *(uint4*)(dst + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  }

  // the packed run of this wave's 16 columns of tile t over this split:
  // nstep KiB, k-step j at +512 j elements
  const int kch = g.K >> 9;
  auto run_ptr = [&](int t) -> const bf16* {
    return Bp + ((size_t)(4 * t + wave) * kch + (k0 >> 9)) * 8192 + 8 * lane;
  };
  const bf16* cur = run_ptr(t0);
  bf16x8_t bfrag[PJ_PF];
#pragma unroll
  for (int j = 0; j < PJ_PF; ++j) bfrag[j] = *(const bf16x8_t*)(cur + 512 * j);
  WAIT_VMCNT(PJ_PF);  // this wave's A copies (issued first) are in LDS
  lds_barrier();      // ... and every wave's; the weight loads stay in flight

  for (int t = t0; t < t1; ++t) {
    // the last tile's ring re-reads its own run's start (in bounds, unused)
    const bf16* nxt = run_ptr(t + 1 < t1 ? t + 1 : t);
    f32x4_t acc[TM / 16];
#pragma unroll
    for (int mb = 0; mb < TM / 16; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < nstep; j0 += PJ_PF) {
      // the loads issued in this block are PF steps ahead: further along this
      // run, or the start of the next tile's run in the last block
      const bf16* lb = (j0 + PJ_PF < nstep) ? cur + 512 * (j0 + PJ_PF) : nxt;
#pragma unroll
      for (int j = 0; j < PJ_PF; ++j) {
        const uint8_t* ap = lds_a + n * AS + 2 * (32 * (j0 + j) + 8 * gq);
#pragma unroll
        for (int mb = 0; mb < TM / 16; ++mb) {
          const bf16x8_t afr = *(const bf16x8_t*)(ap + 16 * mb * AS);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfrag[j], acc[mb], 0, 0, 0);
        }
        // refill the slot just consumed, into the same registers (a separate
        // destination would need a copy, i.e. a wait, at the loop's back edge)
        bfrag[j] = *(const bf16x8_t*)(lb + 512 * j);
        // keep each step's load here: the scheduler would otherwise sink all
        // PF loads to the end of the block and drain the ring
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur = nxt;
    // C lane (gq, n): rows 16mb + 4gq + i of the tile, column 64t + 16 wave + n (< N: N % 64 == 0)
    float* C = g.C + ((size_t)grp * g.ksplit + ks) * (size_t)g.M * g.N + t * PJ_TN + 16 * wave + n;
#pragma unroll
    for (int mb = 0; mb < TM / 16; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * mb + 4 * gq + i;
        if (m < g.M) C[(size_t)m * g.N] = acc[mb][i];
      }
  }
  WAIT_VMCNT(0);  // the last ring of loads before exit
}

// Packing: one thread per 16-byte group of eight k-consecutive values.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16* W, bf16* P, int N, int K, size_t total) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;  // packed 16-byte group
  if (i >= total) return;
  const int kch = K >> 9;
  const int lane = (int)(i & 63), j = (int)((i >> 6) & 15);
  const size_t blk = i >> 10;  // (g, c, h) block
  const int h = (int)(blk % kch);
  const size_t gc = blk / kch;  // g * N/16 + c
  const size_t g = gc / (N >> 4);
  const int c = (int)(gc - g * (N >> 4));
  const int col = 16 * c + (lane & 15), k = 512 * h + 32 * j + 8 * (lane >> 4);
  *(uint4*)(P + 8 * i) = *(const uint4*)(W + (g * N + col) * (size_t)K + k);
}

struct FinishArgs {
  const float* part;   // [groups][ksplit][M][gcols]
  bf16* out;           // [M][ncols], ncols = groups * gcols
  const float* gamma;  // [seg] or NULL
  const int32_t* pos;  // [B] (row m sits at pos[m / S] + m % S) or NULL
  int M, ncols, gcols, seg, spw, ksplit, norm, rope_dim, S;
  float eps;
  double log2_base;
};

constexpr int FN_THREADS = 256;
constexpr int FN_PASS = 2;   // 1024-column passes per workgroup: seg <= 2048
constexpr int FN_BATCH = 8;  // splits whose loads are in flight together

// Workgroup = one row m and `spw` consecutive segments of `seg` columns
// (seg a multiple of 256, spw * seg <= 2048).  Thread j of pass p owns the
// four columns 4j + 1024p of the workgroup's range: every wave reads 1 KiB
// contiguous runs of each split and each wave's 256 columns lie in one
// segment.  The split sum runs in split order (loads of FN_BATCH splits are
// issued before the adds).  RoPE pairs (2i, 2i+1) never straddle a thread's
// four columns, so the rotation needs no data exchange.
__global__ __launch_bounds__(FN_THREADS) void rows_finish_kernel(FinishArgs f) {
  __shared__ float red[FN_PASS][FN_THREADS / 64];
  const int m = blockIdx.y;
  const int c0 = blockIdx.x * f.spw * f.seg;  // first column of this workgroup
  const int width = f.spw * f.seg;
  const int wave = threadIdx.x >> 6;
  float4 v[FN_PASS];
  const float* src[FN_PASS];
  bool on[FN_PASS];
#pragma unroll
  for (int p = 0; p < FN_PASS; ++p) {
    const int c = 1024 * p + 4 * threadIdx.x;
    on[p] = c < width;
    const int cc = c0 + (on[p] ? c : 0), gi = cc / f.gcols, ci = cc - gi * f.gcols;
    src[p] = f.part + (((size_t)gi * f.ksplit) * f.M + m) * f.gcols + ci;
    v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const size_t sstride = (size_t)f.M * f.gcols;
  for (int k0 = 0; k0 < f.ksplit; k0 += FN_BATCH) {
    float4 t[FN_BATCH][FN_PASS];
#pragma unroll
    for (int u = 0; u < FN_BATCH; ++u)
#pragma unroll
      for (int p = 0; p < FN_PASS; ++p)
        t[u][p] = (k0 + u < f.ksplit && on[p]) ? *(const float4*)(src[p] + (size_t)(k0 + u) * sstride)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < FN_BATCH; ++u)
#pragma unroll
      for (int p = 0; p < FN_PASS; ++p) {
        v[p].x += t[u][p].x;
        v[p].y += t[u][p].y;
        v[p].z += t[u][p].z;
        v[p].w += t[u][p].w;
      }
  }
  if (f.norm) {
    // sum of squares per (pass, wave) chunk; each chunk lies in one segment
#pragma unroll
    for (int p = 0; p < FN_PASS; ++p) {
      const float ss = wave_sum(v[p].x * v[p].x + v[p].y * v[p].y + v[p].z * v[p].z + v[p].w * v[p].w);
      if ((threadIdx.x & 63) == 0) red[p][wave] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < FN_PASS; ++p) {
      if (!on[p]) continue;
      const int c = 1024 * p + 4 * threadIdx.x;
      const int sg = c / f.seg;  // segment within the workgroup
      float tot = 0.f;
      for (int q = 0; q < FN_PASS * FN_THREADS / 64; ++q) {
        const int cq = 1024 * (q / (FN_THREADS / 64)) + 256 * (q % (FN_THREADS / 64));
        if (cq < width && cq / f.seg == sg) tot += red[q / (FN_THREADS / 64)][q % (FN_THREADS / 64)];
      }
      const float inv = 1.0f / sqrtf(tot / (float)f.seg + f.eps);
      v[p].x *= inv;
      v[p].y *= inv;
      v[p].z *= inv;
      v[p].w *= inv;
      if (f.gamma != nullptr) {
        const float4 g = *(const float4*)(f.gamma + (c - sg * f.seg));
        v[p].x *= g.x;
        v[p].y *= g.y;
        v[p].z *= g.z;
        v[p].w *= g.w;
      }
    }
  }
  const double t = f.pos != nullptr ? (double)((long)f.pos[m / f.S] + m % f.S) : 0.0;
#pragma unroll
  for (int p = 0; p < FN_PASS; ++p) {
    if (!on[p]) continue;
    const int c = 1024 * p + 4 * threadIdx.x;
    const int cs = c % f.seg;  // column within its segment
    float a[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
    if (f.rope_dim > 0) {
      const int tail0 = f.seg - f.rope_dim;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cp = cs + 2 * h;
        if (cp >= tail0) {
          float co, sn;
          rope_cos_sin(t, (cp - tail0) >> 1, f.rope_dim, f.log2_base, &co, &sn);
          const float x = a[2 * h], y = a[2 * h + 1];
          a[2 * h] = x * co - y * sn;
          a[2 * h + 1] = x * sn + y * co;
        }
      }
    }
    uint2 o;
    o.x = (uint32_t)f2bf(a[0]) | ((uint32_t)f2bf(a[1]) << 16);
    o.y = (uint32_t)f2bf(a[2]) | ((uint32_t)f2bf(a[3]) << 16);
    *(uint2*)(f.out + (size_t)m * f.ncols + c0 + c) = o;
  }
}

}  // namespace csa

namespace csa_host {
using namespace csa;

struct GemmPlan {
  int tm, kc, ksplit, mtiles, ntiles, tpw, gx;
};

// Tile plan of one (grouped) product, shared by the workspace-size query and
// the launch.  TM = 32 rows when M <= 32 (decode), else 64.  For each K split
// width KC in {512, 1024, 1536, 2048} (A slab <= 128 KiB of LDS) the column
// tiles of every (split, row tile, group) are dealt out in contiguous ranges
// of tpw tiles so that at most one workgroup per CU is needed; the KC with
// the least estimated per-CU traffic (busiest CU's weight bytes, fp32
// partials written and read, A slab copies at half weight) wins, the larger
// KC on ties.  N % 64 == 0 and K % 512 == 0.
GemmPlan gemm_plan(int groups, int M, int N, int K) {
  GemmPlan best{};
  double best_cost = 0;
  const int tm = M <= 32 ? 32 : 64;
  const int mtiles = (M + tm - 1) / tm, ntiles = N / PJ_TN;
  const int kc_max = tm == 32 ? 2048 : 1024;
  for (int kc = 512; kc <= kc_max; kc += 512) {
    const int kce = kc < K ? kc : K;
    const int ksplit = (K + kce - 1) / kce;
    const long upc = (long)ksplit * mtiles * groups;  // workgroup rows
    long cols = PJ_CUS / upc;                          // workgroups per row within one CU round
    if (cols < 1) cols = 1;
    int tpw = (int)((ntiles + cols - 1) / cols);
    const int gx = (ntiles + tpw - 1) / tpw;
    const long wgs = (long)gx * upc;
    const long rounds = (wgs + PJ_CUS - 1) / PJ_CUS;
    const double stream = (double)rounds * tpw * PJ_TN * kce * 2;
    const double part = (double)groups * ksplit * M * N * 8 / PJ_CUS;
    const double aslab = (double)rounds * tm * kce;
    const double cost = stream + part + aslab;
    if (kc == 512 || cost <= best_cost) {
      best = GemmPlan{tm, kce, ksplit, mtiles, ntiles, tpw, gx};
      best_cost = cost;
    }
    if (kce == K) break;
  }
  return best;
}

size_t gemm_partial_bytes(int groups, int M, int N, int K) {
  const GemmPlan p = gemm_plan(groups, M, N, K);
  return (size_t)groups * p.ksplit * M * N * sizeof(float);
}

// Bp: packed weights (pack_weights); N % 64 == 0, K % 512 == 0.
hipError_t launch_gemm_nt(const void* A, const void* Bp, float* C, int groups, int M, int N, int K, int lda, long sa,
                          long sb, int* ksplit_out, hipStream_t st) {
  const GemmPlan p = gemm_plan(groups, M, N, K);
  GemmArgs g{(const bf16*)A, (const bf16*)Bp, C, M, N, K, lda, sa, sb, p.kc, p.ksplit, p.ntiles, p.tpw, p.gx, p.mtiles,
             groups};
  const dim3 grid((unsigned)(p.gx * p.ksplit * p.mtiles * groups));
  const size_t lds = (size_t)p.tm * pj_row_bytes(p.kc);
  if (ksplit_out) *ksplit_out = p.ksplit;
  // A slabs above 64 KiB need the dynamic-LDS limit raised, once per device
  static std::atomic<unsigned long long> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = 1ull << (dev & 63);
  if (!(raised.load() & bit)) {
    e = hipFuncSetAttribute((const void*)gemm_nt_kernel<32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(32 * pj_row_bytes(2048)));
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)gemm_nt_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(64 * pj_row_bytes(1024)));
    if (e != hipSuccess) return e;
    raised.fetch_or(bit);
  }
  if (p.tm == 32)
    hipLaunchKernelGGL(gemm_nt_kernel<32>, grid, dim3(64 * PJ_NW), lds, st, g);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<64>, grid, dim3(64 * PJ_NW), lds, st, g);
  return hipGetLastError();
}

// groups x [N][K] -> packed; N % 16 == 0, K % 512 == 0.
hipError_t launch_pack_weights(const void* W, void* P, int groups, int N, int K, hipStream_t st) {
  const size_t total = (size_t)groups * N * (size_t)K / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const bf16*)W,
                     (bf16*)P, N, K, total);
  return hipGetLastError();
}

// seg divides ncols and is a multiple of 256, <= 2048; with rope_dim > 0,
// rope_dim is even and <= seg.  gcols is a multiple of 4.
hipError_t launch_rows_finish(const float* part, void* out, const float* gamma, const int32_t* pos, int M, int ncols,
                              int gcols, int seg, int ksplit, int norm, int rope_dim, int S, float eps, float base,
                              hipStream_t st) {
  int spw = 1;  // segments per workgroup: up to 2048 columns (FN_PASS passes)
  while (2 * spw * seg <= 1024 * FN_PASS && (ncols / seg) % (2 * spw) == 0) spw *= 2;
  FinishArgs f{part, (bf16*)out, gamma, pos, M, ncols, gcols, seg, spw, ksplit, norm, rope_dim, S, eps,
               std::log2((double)base)};
  hipLaunchKernelGGL(rows_finish_kernel, dim3((unsigned)(ncols / (seg * spw)), (unsigned)M), dim3(FN_THREADS), 0, st,
                     f);
  return hipGetLastError();
}

}  // namespace csa_host
