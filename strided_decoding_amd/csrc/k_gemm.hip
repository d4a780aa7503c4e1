// Projection GEMMs of the decode step: Y[M, N] = X[M, K] W[N, K]^T with fused epilogues
// (bf16 store, fp32 store, fp32 residual add, SwiGLU of a gate/up pair) and the MASK-row
// LoRA delta.
//
// bf16 path: the weights are in a packed operand layout (the B operand of one 32x32x16 MFMA
// is one contiguous kilobyte), so every weight load is a full-rate contiguous 1 KB access.
// Tiled kernel (the automatic choice above 32 rows): one 224 x 64 WV output tile per
// workgroup of WV = 4, 3 or 2 waves, one wave per SIMD, each 224 x 64 = 7 x 2 MFMA tiles (224
// accumulators in AGPRs).  224 = 448 / 2 makes the decode row count (64 slots x 7 rows)
// exactly two row tiles; a product of more than 128 rows has at least two row tiles, its rows
// split evenly in 32-row blocks.  The activation tile is streamed in 32-wide k stages through
// an 8-deep LDS ring filled by direct global->LDS loads and shared by the waves; each wave
// loads its own weight operands straight into a 4-stage register ring.  Each 64-byte LDS row
// keeps its four 16-byte k-chunks XOR-swizzled by (row/4)%4 so that the 16 rows an MFMA
// operand read touches fall in distinct banks.
// Skinny kernel (at most 128 rows; the automatic choice up to 32): workgroups of two waves (one
// for very wide products), each wave streaming 64 weight columns while the pair shares the
// activation stages.
// Split-K: split s covers k-stages [s kt, (s+1) kt) and writes fp32 partials that
// splitk_reduce_kernel sums in split order - no atomics - so every output element has a fixed
// accumulation order that depends only on K and the split count, never on the number of rows.
// Workgroup ids are ordered so that the row tiles sharing a weight tile differ by a multiple
// of 8 and run on the same XCD (one L2).
// fp32 path: LDS-tiled FMA, same epilogues.
#include <algorithm>
#include <type_traits>

#include "gemm_tile.h"

namespace isd {
namespace {

// LDS ring depth of the skinny kernel for one / two / four 32-row tiles
#ifndef ISD_SK_SD1
#define ISD_SK_SD1 8
#endif
#ifndef ISD_SK_SD2
#define ISD_SK_SD2 8
#endif
#ifndef ISD_SK_SD4
#define ISD_SK_SD4 4
#endif
// waves per skinny workgroup for one / two / four row tiles, and the ring depth of the
// two-wave form
#ifndef ISD_SK_WV1
#define ISD_SK_WV1 2
#endif
#ifndef ISD_SK_WV2
#define ISD_SK_WV2 2
#endif
#ifndef ISD_SK_WV4
#define ISD_SK_WV4 2
#endif
#ifndef ISD_SK_SD1W
#define ISD_SK_SD1W 8
#endif
#ifndef ISD_SK_SD2W
#define ISD_SK_SD2W 6
#endif
#ifndef ISD_SK_SD4W
#define ISD_SK_SD4W 4
#endif


// Skinny path for at most 128 rows (decode at small batch, where a projection is bound by
// streaming its weights from HBM).  One workgroup of WV waves per (output-column group, K
// split).  Each wave streams its packed weight operands (one contiguous 1 KB direct load per
// block and k-step) and the (L2-resident) activation rows through an SD-stage LDS ring filled
// by direct global->LDS loads, with the loads of the next stages in flight under explicit
// vmcnt waits while one stage is multiplied.  WV = 1 needs no barrier at all.  The MFMA (32x32x16), the k-chunk
// held by each lane, the k-step order, the split rule and the partial layout are those of the
// tiled kernel, so every output element is accumulated in exactly the same order and the two
// paths give bit-identical results.
//
// WV = 2: two waves share the activation stages (each loads half of the row groups) and each
// streams its own 64 output columns; a barrier per stage then orders the ring's refills.  The
// activation traffic per output column halves; the accumulation order is unchanged.
template <int EPI, bool PARTIAL, int MT, int SD, int WV>
__global__ __launch_bounds__(64 * WV) void gemm_bf16_skinny_kernel(GemmArgs a, int n_nt, int S, float* part) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int NB = 2;                     // 32-column MFMA tiles per wave (gate + up for SwiGLU)
  constexpr int TNO = DUAL ? 32 : 64;       // output columns per wave
  constexpr int XG = 2 * MT / WV;           // activation row groups each wave loads per stage
  constexpr int STAGE = (MT + NB * WV) * 2048;   // bytes per 32-k stage: activation tiles, then each wave's weight operands
  constexpr int PER_STAGE = XG + 2 * NB;    // direct loads per stage and wave
  static_assert(WV == 1 || WV == 2, "one or two waves");
  static_assert((SD - 1) * PER_STAGE < 64, "vmcnt counts at most 63 outstanding loads");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SD * STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = WV > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
  const int unit = blockIdx.x;
  const int sp = unit / n_nt, nt = unit - sp * n_nt;
  const int kt_per = (a.K / BK) / S;
  const int kbase = sp * kt_per * BK;
  const int nw0 = nt * TNO * WV;            // the workgroup's first column (segments never split a workgroup)
  const int n0 = nw0 + wave * TNO;          // this wave's
  const int r32 = lane & 31, khi = lane >> 5;
  const uint16_t* zero = kZeroOperand + lane * 8;
  // stages kt_per .. kt_end-1: the fused LoRA expand (last split only)
  const LoraPlan lp = lora_plan(a, nw0, DUAL, sp == S - 1);
  const int kt_end = kt_per + lp.n;

  // Activation loader (the tiled kernel's 16-row group layout): one direct load per 16-row
  // group and stage; lane l fills LDS bytes [16 l, 16 l + 16) of the group with row l/4,
  // k-chunk (l%4) ^ ((row/4)%4), so the operand reads below are free of bank conflicts.
  const int lrow = lane >> 2;
  const int chunk = (lane & 3) ^ ((lrow >> 2) & 3);
  const int aoff = gemm_seg_aoff(a, nw0);
  // this wave's row groups: q * WV + wave, i.e. 16-row group g = gq % 2 of row tile gq / 2
  const uint16_t* xsrc[XG];
  const uint16_t* lsrc[XG];                 // fused LoRA: the row's lora_a row (null: zeros)
  {
    // every row-index load is issued before any is used (one wait, not one per row group)
    int sr[XG], lr[XG];
#pragma unroll
    for (int q = 0; q < XG; ++q) {
      const int mc = min(16 * (q * WV + wave) + lrow, a.M - 1);
      sr[q] = a.a_rows ? a.a_rows[mc] : mc;
      lr[q] = lp.n ? a.lora_rows[mc] : -1;
    }
#pragma unroll
    for (int q = 0; q < XG; ++q) {
      const bool valid = 16 * (q * WV + wave) + lrow < a.M;
      const int srow = valid ? max(sr[q], 0) : 0;   // unused rows: their outputs are never consumed
      const int l = valid ? lr[q] : -1;
      xsrc[q] = (const uint16_t*)a.A + (size_t)srow * a.lda + aoff + kbase + chunk * 8;
      lsrc[q] = l >= 0 ? (const uint16_t*)a.lora_a + (size_t)l * a.ld_la + lp.seg_off + chunk * 8 : nullptr;
    }
  }
  // weight operand blocks: columns n0 + 32 j .. (SwiGLU: gate j = 0 and up j = 1 of n0 ..)
  const uint16_t* wsrc[NB];
  const uint16_t* lwsrc[NB];                // fused LoRA: the packed lora_b blocks of the same columns
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int nb = min(DUAL ? (n0 >> 5) : (n0 >> 5) + j, ((a.N + 31) >> 5) - 1);
    wsrc[j] = packed_operand((const uint16_t*)((DUAL && j) ? a.B1 : a.B0), nb, a.K, kbase / 16, lane);
    lwsrc[j] = packed_operand((const uint16_t*)((DUAL && j) ? a.lora_b1 : a.lora_b0), nb, a.lora_r, 0, lane);
  }

  // stage kt -> ring slot kt % SD: activation tile t, row group g at + (2 t + g) KB, then the
  // weight operand of block j and k-step kk at + (2 MT + 2 j + kk) KB.  Stages past the last
  // one load zeros.
  // (stages kt_per .. kt_end-1 are the LoRA stages: SwiGLU per gate of the up group, with the
  // other block's operand zero; later stages load zeros)
  // MODE: a stage inside the product (plain addresses), or any stage without (kZeroTail) or
  // with (kLoraTail) fused LoRA stages
  auto issue = [&](auto mode, int kt) {
    constexpr int MODE = decltype(mode)::value;
    uint8_t* st = smem + (kt % SD) * STAGE;
    const bool live = MODE == kPlainStages || kt < kt_per;
    const int ls = kt - kt_per;                 // LoRA stage offsets as in the tiled kernel
    const bool lora = ls >= 0 && ls < lp.n;
#pragma unroll
    for (int q = 0; q < XG; ++q) {
      const uint16_t* l = (MODE == kLoraTail && lora && lsrc[q]) ? lsrc[q] + ls * BK : zero;
      __builtin_amdgcn_global_load_lds((const void*)(live ? xsrc[q] + kt * BK : l),
                                       (lds_void*)(st + (q * WV + wave) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int lk = ls - (DUAL ? j * lp.per : 0);
        const uint16_t* l = (MODE == kLoraTail && lk >= 0 && lk < (DUAL ? lp.per : lp.n)) ? lwsrc[j] + (2 * lk + kk) * 512 : zero;
        // weights non-temporal (streamed once; measured -6 % per decode pass at 1 slot)
        __builtin_amdgcn_global_load_lds((const void*)(live ? wsrc[j] + (2 * kt + kk) * 512 : l),
                                         (lds_void*)(st + (2 * MT + 2 * NB * wave + 2 * j + kk) * 1024), 16, 0,
                                         kCachePolicyNT);
      }
  };
  f32x16_t acc[MT][NB];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // activation operand of lane L: row r32 (group r32/16, row r32%16), k-chunk 2 kk + khi, swizzled
  const int rig = r32 & 15;
  const int rd0 = (r32 >> 4) * 1024 + rig * 64;
  const int sw = (rig >> 2) & 3;
  auto mul = [&](int kt) {
    const uint8_t* st = smem + (kt % SD) * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int off = ((2 * kk + khi) ^ sw) * 16;
      bf16x8_t x[MT], w[NB];
#pragma unroll
      for (int t = 0; t < MT; ++t) x[t] = as_bf16x8(*(const u32x4_t*)(st + rd0 + 2 * t * 1024 + off));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        w[j] = as_bf16x8(*(const u32x4_t*)(st + (2 * MT + 2 * NB * wave + 2 * j + kk) * 1024 + lane * 16));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32x32x16(x[i], w[j], acc[i][j]);
    }
  };

  // Stage kt is issued SD-1 steps before it is multiplied.  One wave: issue, then wait until
  // only the loads of the stages issued after stage kt are outstanding.  Two waves: wait for
  // this wave's loads of stage kt, then a barrier (every wave's loads of stage kt have landed
  // and every wave is done with stage kt-1, whose slot the next issue refills).
  auto step = [&](auto mode, int kt) {
    if constexpr (WV == 1) {
      issue(mode, kt + SD - 1);
      wait_vmcnt<(SD - 1) * PER_STAGE>();
    } else {
      wait_vmcnt<(SD - 2) * PER_STAGE>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(mode, kt + SD - 1);
    }
    mul(kt);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int kt = 0; kt < SD - 1; ++kt) issue(StageMode<kLoraTail>{}, kt);
  const int fast_end = max(0, kt_per - (SD - 1));   // steps whose issued stage is a product stage
  int kt = 0;
  for (; kt < fast_end; ++kt) step(StageMode<kPlainStages>{}, kt);
  auto tail = [&](auto mode) {
    for (; kt < kt_end; ++kt) step(mode, kt);
  };
  if (lp.n == 0)
    tail(StageMode<kZeroTail>{});
  else
    tail(StageMode<kLoraTail>{});
  wait_vmcnt<0>();                               // the loads past the last stage

  // The MASK-row LoRA delta of a row tile is loaded before any of its stores, so that the
  // loads are issued together rather than one round trip per output.
  GemmArgs b = a;
  b.delta_row = nullptr;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    float dl[16][NB];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < NB; ++j) dl[r][j] = -0.f;   // x + (-0) == x for every x
    if (!PARTIAL && a.delta_row) {
      int dr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * khi + (r & 3);
        dr[r] = row < a.M ? a.delta_row[row] : -1;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = DUAL ? n0 + r32 : n0 + 32 * j + r32;
          if (dr[r] >= 0 && col < a.N)
            dl[r][j] = a.delta[(size_t)dr[r] * a.ldd + (DUAL && j ? a.delta_off2 : 0) + col];
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * i + 8 * (r >> 2) + 4 * khi + (r & 3);
      if (row >= a.M) continue;
      if (DUAL) {
        const int col = n0 + r32;
        if (PARTIAL) {
          if (col < a.N) {
            float* pr = part + ((size_t)sp * a.M + row) * (2 * (size_t)a.N);
            pr[col] = acc[i][0][r];
            pr[a.N + col] = acc[i][1][r];
          }
        } else {
          epilogue_store_t<bf16, EPI>(b, row, col, acc[i][0][r] + dl[r][0], acc[i][1][r] + dl[r][1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = n0 + 32 * j + r32;
          if (PARTIAL) {
            if (col < a.N) part[((size_t)sp * a.M + row) * (size_t)a.N + col] = acc[i][j][r];
          } else {
            epilogue_store_t<bf16, EPI>(b, row, col, acc[i][j][r] + dl[r][j], 0.f);
          }
        }
      }
    }
  }
}

constexpr int kMaxSplits = 16;

// Sum the split-K partials in split order and apply the epilogue (MAXS: the split bucket).
template <int EPI, int MAXS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, int S, const float* part) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  const size_t ld = DUAL ? 2 * (size_t)a.N : (size_t)a.N;
  const int m_lim = a.m_live ? min(*a.m_live, a.M) : a.M;       // live rows of a packed pass
  const size_t n4 = (size_t)m_lim * a.N / 4;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e * 4 / a.N), col = (int)(e * 4 % a.N);
    f32x4_t v, u;
    sum_split_partials<MAXS, DUAL>(part + (size_t)row * ld + col, (size_t)a.M * ld, S, a.N, v, u);
#pragma unroll
    for (int j = 0; j < 4; ++j) epilogue_store_t<bf16, EPI>(a, row, col + j, v[j], u[j]);
  }
}

// Split-K reduction fused with the residual update and the RMSNorm of the updated row: one
// block of 1024 threads per row; thread t owns the 4-column groups t + 1024 k.  Each group is
// summed over the splits in order (all split loads issued together), added to the residual,
// and its squares accumulated in the same order and tree as the standalone RMSNorm kernel, so
// both paths give the same normalized row for the same residual row.
constexpr int kNormThreads = 1024;
constexpr int kNormMaxGroups = 2;         // rows up to 8192 wide
template <int MAXS>
__global__ __launch_bounds__(kNormThreads) void splitk_resid_norm_kernel(GemmArgs a, int S, const float* part) {
  __shared__ float sh[kNormThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  // the live-row count, the row's delta index and this thread's norm weights are loaded
  // together, ahead of the row's data (one memory round trip before the partials, none after
  // the reduction)
  const int live = a.m_live ? *a.m_live : a.M;
  const int dr = a.delta_row ? a.delta_row[row] : -1;
  const bf16* g = (const bf16*)a.norm_g;
  float gv[kNormMaxGroups][4];
#pragma unroll
  for (int k = 0; k < kNormMaxGroups; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j)   // (clamped, not branched: every load goes out at once)
      gv[k][j] = to_f(g[min(4 * (tid + kNormThreads * k) + j, a.N - 1)]);
  if (row >= live) return;                          // a dead row of a packed pass
  float* R = a.R + (size_t)row * a.ldr;
  const size_t split_stride = (size_t)a.M * a.N;
  const float* prow = part + (size_t)row * a.N;
  f32x4_t rv[kNormMaxGroups];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormMaxGroups; ++k) {
    const int c = 4 * (tid + kNormThreads * k);
    rv[k] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if (c < a.N) {
      const f32x4_t rin = *(const f32x4_t*)(R + c);
      f32x4_t dv = {0.f, 0.f, 0.f, 0.f};
      if (dr >= 0) dv = *(const f32x4_t*)(a.delta + (size_t)dr * a.ldd + c);
      f32x4_t v, unused;
      sum_split_partials<MAXS, false>(prow + c, split_stride, S, 0, v, unused);
      if (dr >= 0) v += dv;
      const f32x4_t r = rin + v;
      *(f32x4_t*)(R + c) = r;
      rv[k] = r;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(r[j], r[j], ss);
    }
  }
  const float tot = block_sum_1024(ss, sh);
  const float denom = sqrtf(tot / (float)a.N + a.norm_eps);
  bf16* y = (bf16*)a.norm_out + (size_t)row * a.N;
#pragma unroll
  for (int k = 0; k < kNormMaxGroups; ++k) {
    const int c = 4 * (tid + kNormThreads * k);
    if (c < a.N) {
#pragma unroll
      for (int j = 0; j < 4; ++j) y[c + j] = from_f<bf16>((rv[k][j] / denom) * gv[k][j]);
    }
  }
}

// fp32 reference-precision path: 64 x 64 tile, 256 threads with 4 x 4 outputs each.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 1];
  __shared__ float Bs[TK][T + 1];
  __shared__ float Us[DUAL ? TK : 1][T + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * T, m0 = blockIdx.y * T;
  const float* A = (const float*)a.A;
  const float* B0 = (const float*)a.B0;
  const float* B1 = (const float*)a.B1;
  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += TK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e, r = idx >> 4, k = idx & 15;
      const int m = m0 + r, n = n0 + r, kk = k0 + k;
      float av = 0.f, bv = 0.f, uv = 0.f;
      if (m < a.M && kk < a.K) {
        const int src = a.a_rows ? a.a_rows[m] : m;
        if (src >= 0) av = A[(size_t)src * a.lda + kk];
      }
      if (n < a.N && kk < a.K) {
        bv = B0[(size_t)n * a.ldb + kk];
        if (DUAL) uv = B1[(size_t)n * a.ldb + kk];
      }
      As[k][r] = av;
      Bs[k][r] = bv;
      if (DUAL) Us[k][r] = uv;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float av[4], bv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[k][ty * 4 + i];
        bv[i] = Bs[k][tx * 4 + i];
        if (DUAL) uv[i] = Us[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
          if (DUAL) accu[i][j] = fmaf(av[i], uv[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      epilogue_store_t<float, EPI>(a, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j], accu[i][j]);
}

// After the main kernel: the ordered split-K reduction (fused with the residual update and the
// next RMSNorm when asked), or the standalone RMSNorm when there is no split.
template <int EPI>
hipError_t finish(const GemmArgs& a, int S, hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (S > 1 && a.keep_part) return hipSuccess;       // the consumer reduces the partials
  const bool norm = EPI == EPI_RESID && a.norm_out;
  if (S > 1) {
    const size_t n4 = (size_t)a.M * a.N / 4;
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    const float* part = (const float*)a.part;
#define ISD_REDUCE(B)                                                                                   \
  if (norm)                                                                                             \
    hipLaunchKernelGGL(splitk_resid_norm_kernel<B>, dim3(a.M), dim3(kNormThreads), 0, s, a, S, part); \
  else                                                                                                  \
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI, B>), dim3(blocks), dim3(256), 0, s, a, S, part);
    switch (split_bucket(S)) {
      case 2: ISD_REDUCE(2) break;
      case 4: ISD_REDUCE(4) break;
      case 8: ISD_REDUCE(8) break;
      default: ISD_REDUCE(16) break;
    }
#undef ISD_REDUCE
    return hipGetLastError();
  }
  if (norm) return launch_rmsnorm<bf16>(a.R, (const bf16*)a.norm_g, (bf16*)a.norm_out, a.M, a.N, a.norm_eps, s);
  return hipSuccess;
}

// CUs of the current device (queried once).
int num_cus() {
  static const int n = [] {
    int dev = 0, v = 0;
    return (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
  }();
  return n;
}

// Waves per workgroup of the tiled kernel.  Every workgroup of a decode-size grid runs at
// once (one per CU), and its stage time follows the data its CU streams per stage: the
// activation tile (14 row-group loads, padded to a multiple of the wave count) plus 4 KB of
// weight operands per wave.  Fewer waves per workgroup mean more workgroups over the same
// columns; the choice minimises (grid rounds over the CUs) x (loads per stage and CU), among
// the wave counts whose column tiles do not straddle a segment boundary.
template <int EPI>
int big_waves(const GemmArgs& a, int n_mt, int S) {
  const int tnw = EPI == EPI_SWIGLU ? 32 : 64;   // output columns per wave
  auto fits = [&](int wv) {                       // no column tile straddles a segment boundary
    bool ok = true;
    for (int j = 0; j + 1 < a.nseg; ++j) ok = ok && a.seg_end[j] % (wv * tnw) == 0;
    if (a.lora_r > 0)
      for (int j = 0; j + 1 < a.lora_nseg; ++j) ok = ok && a.lora_seg_end[j] % (wv * tnw) == 0;
    return ok;
  };
  if (a.path >= GEMM_PATH_TILED4) {
    const int wv = 4 - (a.path - GEMM_PATH_TILED4);
    return fits(wv) ? wv : 4;
  }
#ifdef ISD_BIG_WAVES
  return ISD_BIG_WAVES;   // build-time override of the automatic choice (tuning)
#endif
  const int n_cu = num_cus();
  int best = 4;
  long best_cost = -1;
  for (int wv = 4; wv >= 2; --wv) {
    if (!fits(wv)) continue;
    const long wgs = (long)n_mt * ((a.N + wv * tnw - 1) / (wv * tnw)) * S;
    const long cost = (wgs + n_cu - 1) / n_cu * (wv * ((AG + wv - 1) / wv) + 4 * wv);
    if (best_cost < 0 || cost < best_cost) best = wv, best_cost = cost;
  }
  return best;
}

template <int EPI>
hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
  // at least two row tiles above 128 rows: at 224 rows two tiles of 128 + 96 rows (a smaller
  // activation stage per CU, twice the workgroups) were 20-30 % faster than one of 224.  Not for
  // very wide products (the LM head), whose column tiles alone fill the CUs several times over:
  // there a second row tile only reads the weights twice (+12 % at 224 rows, measured).
  const int n_mt = std::max((a.M + TM2 - 1) / TM2, a.M > 128 && a.N <= 65536 ? 2 : 1);
  const int S = (a.splits > 1 && a.part) ? a.splits : 1;
  const int WV = big_waves<EPI>(a, n_mt, S);
  const int tno = (EPI == EPI_SWIGLU ? 32 : 64) * WV;
  const int n_nt = (a.N + tno - 1) / tno;
  const int units = n_nt * S;
  dim3 grid(((units + 7) / 8) * 8 * n_mt);
  const hipError_t e = launch_big_kernel<EPI>(a, grid, WV, n_mt, units, S, s);
  if (e != hipSuccess) return e;
  return finish<EPI>(a, S, s);
}

template <int EPI>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
  const int tno = EPI == EPI_SWIGLU ? 32 : 64;
  const int MT = a.M <= 32 ? 1 : (a.M <= 64 ? 2 : 4);
  int WV = MT == 1 ? ISD_SK_WV1 : (MT == 2 ? ISD_SK_WV2 : ISD_SK_WV4);
  // very wide products (the LM head) keep one wave per workgroup: their activation traffic is
  // small next to the weights, and twice the workgroups spread better (measured)
  if (a.N > 65536) WV = 1;
  // a two-wave workgroup shares one activation stage: no (LoRA) segment boundary inside it
  for (int j = 0; j + 1 < a.nseg; ++j)
    if (a.seg_end[j] % (WV * tno)) WV = 1;
  if (a.lora_r > 0)
    for (int j = 0; j + 1 < a.lora_nseg; ++j)
      if (a.lora_seg_end[j] % (WV * tno)) WV = 1;
  const int n_nt = (a.N + WV * tno - 1) / (WV * tno);
  const int S = (a.splits > 1 && a.part) ? a.splits : 1;
  dim3 grid(n_nt * S);
  float* part = S > 1 ? a.part : nullptr;
#define ISD_SKINNY(P, MT, SD, W) \
  hipLaunchKernelGGL((gemm_bf16_skinny_kernel<EPI, P, MT, SD, W>), grid, dim3(64 * W), 0, s, a, n_nt, S, part)
#define ISD_SKINNY_WV(MT, SD, SDW)                         \
  if (WV == 1) {                                           \
    if (S > 1) ISD_SKINNY(true, MT, SD, 1);                \
    else ISD_SKINNY(false, MT, SD, 1);                     \
  } else {                                                 \
    if (S > 1) ISD_SKINNY(true, MT, SDW, 2);               \
    else ISD_SKINNY(false, MT, SDW, 2);                    \
  }
  if (MT == 1) {
    ISD_SKINNY_WV(1, ISD_SK_SD1, ISD_SK_SD1W)
  } else if (MT == 2) {
    ISD_SKINNY_WV(2, ISD_SK_SD2, ISD_SK_SD2W)
  } else {
    ISD_SKINNY_WV(4, ISD_SK_SD4, ISD_SK_SD4W)
  }
#undef ISD_SKINNY_WV
#undef ISD_SKINNY
  return finish<EPI>(a, S, s);
}

template <int EPI>
hipError_t launch_path(const GemmArgs& a, hipStream_t s) {
  // automatic: the skinny kernel up to 32 rows (64 for very wide products, the LM head), the
  // tiled kernel above (measured per decode pass: 16 slots, 112 rows, 7.28 -> 6.49 ms; 8 slots,
  // 56 rows, 5.59 -> 5.52 ms; at 7 rows the skinny kernel stays ahead)
  const bool skinny = a.path == GEMM_PATH_SKINNY ||
                      (a.path == GEMM_PATH_AUTO && (a.M <= 32 || (a.M <= 64 && a.N > 65536)));
  return skinny ? launch_skinny<EPI>(a, s) : launch_big<EPI>(a, s);
}

}  // namespace
}  // namespace isd

int gemm_splits(int n_out, int K, bool dual) {
  const int tno = dual ? isd::TN2 / 2 : isd::TN2;
  const int tiles = (n_out + tno - 1) / tno;
  int S = 1;
  // split while there are fewer than 256 workgroups of 256 columns (x2 row tiles) and every
  // split keeps at least 4 k-stages
  while (S < isd::kMaxSplits && 2 * tiles * (2 * S) <= 256 && (K / isd::BK) % (2 * S) == 0 && K / (2 * S) >= 128)
    S *= 2;
  return S;
}

namespace isd {

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % BK != 0 || a.N % 4 != 0) return hipErrorInvalidValue;
  if (a.norm_out && (a.epi != EPI_RESID || a.N > 4 * kNormThreads * kNormMaxGroups)) return hipErrorInvalidValue;
  if ((a.splits > 1 && a.part) && a.splits > kMaxSplits) return hipErrorInvalidValue;
  const int S = (a.splits > 1 && a.part) ? a.splits : 1;
  if ((a.K / BK) % S != 0) return hipErrorInvalidValue;
  if (a.path == GEMM_PATH_SKINNY && a.M > kSkinnyMaxRows) return hipErrorInvalidValue;
  if (a.nseg < 0 || a.nseg > 3 || (a.nseg > 1 && (S > 1 || a.epi == EPI_SWIGLU))) return hipErrorInvalidValue;
  for (int j = 0; j + 1 < a.nseg; ++j)
    if (a.seg_end[j] % TN2) return hipErrorInvalidValue;
  if (a.lora_r > 0) {
    if (a.lora_r % BK || !a.lora_rows || !a.lora_a || !a.lora_b0 || (a.epi == EPI_SWIGLU && !a.lora_b1))
      return hipErrorInvalidValue;
    if (a.lora_nseg < 1 || a.lora_nseg > 3 || (a.epi == EPI_SWIGLU && a.lora_nseg != 1)) return hipErrorInvalidValue;
    for (int j = 0; j + 1 < a.lora_nseg; ++j)
      if (a.lora_seg_end[j] % TN2) return hipErrorInvalidValue;
  }
  switch (a.epi) {
    case EPI_STORE: return launch_path<EPI_STORE>(a, s);
    case EPI_STORE_F32: return launch_path<EPI_STORE_F32>(a, s);
    case EPI_RESID: return launch_path<EPI_RESID>(a, s);
    case EPI_SWIGLU: return launch_path<EPI_SWIGLU>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Row-major bf16 W [rows, cols] -> the packed operand layout (rows padded with zeros to a
// multiple of 32): thread e writes the 16 bytes of lane e%64 of operand block e/64.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* src, uint16_t* dst, int rows, int cols,
                                                           size_t n16) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n16) return;
  const int lane = (int)(e & 63);
  const size_t blk = e >> 6;
  const int kbn = cols / 16;
  const int kb = (int)(blk % kbn);
  const size_t nb = blk / kbn;
  const size_t row = nb * 32 + (lane & 31);
  const int k0 = kb * 16 + 8 * (lane >> 5);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < (size_t)rows) v = *(const u32x4_t*)(src + row * cols + k0);
  *(u32x4_t*)(dst + e * 8) = v;
}

size_t packed_weight_elems(int rows, int cols) { return (size_t)((rows + 31) / 32) * 32 * cols; }

hipError_t launch_pack_weights(const void* src, void* dst, int rows, int cols, hipStream_t s) {
  if (rows < 1 || cols < 16 || cols % 16) return hipErrorInvalidValue;
  const size_t n16 = packed_weight_elems(rows, cols) / 8;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, (const uint16_t*)src,
                     (uint16_t*)dst, rows, cols, n16);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, dim3(256), 0, s, a); break;
    case EPI_STORE_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE_F32>, grid, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_kernel<EPI_RESID>, grid, dim3(256), 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.norm_out) return e;
  return launch_rmsnorm<float>(a.R, (const float*)a.norm_g, (float*)a.norm_out, a.M, a.N, a.norm_eps, s);
}

}  // namespace isd
