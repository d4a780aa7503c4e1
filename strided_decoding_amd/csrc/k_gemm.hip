// Projection GEMMs of the decode step: Y[M, N] = X[M, K] W[N, K]^T with fused epilogues
// (bf16 store, fp32 store, fp32 residual add, SwiGLU of a gate/up pair) and the MASK-row
// LoRA delta.
//
// bf16 path: the weights are in a packed operand layout (the B operand of one 32x32x16 MFMA
// is one contiguous kilobyte), so every weight load is a full-rate contiguous 1 KB access.
// Tiled kernel (more than 128 rows): one 224 x 64 WV output tile per workgroup of WV = 4, 3
// or 2 waves, one wave per SIMD, each 224 x 64 = 7 x 2 MFMA tiles (224 accumulators in AGPRs).  224 = 448 / 2
// makes the decode row count (64 slots x 7 rows) exactly two row tiles.  The activation tile
// is streamed in 32-wide k stages through a 10-deep LDS ring filled by direct global->LDS
// loads and shared by the waves; each wave loads its own weight operands straight into a
// 4-stage register ring.  Each 64-byte LDS row keeps its four 16-byte k-chunks XOR-swizzled by
// (row/4)%4 so that the 16 rows an MFMA operand read touches fall in distinct banks.
// Skinny kernel (at most 128 rows): workgroups of two waves (one for very wide products), each
// wave streaming 64 weight columns while the pair shares the activation stages.
// Split-K: split s covers k-stages [s kt, (s+1) kt) and writes fp32 partials that
// splitk_reduce_kernel sums in split order - no atomics - so every output element has a fixed
// accumulation order that depends only on K and the split count, never on the number of rows.
// Workgroup ids are ordered so that the row tiles sharing a weight tile differ by a multiple
// of 8 and run on the same XCD (one L2).
// fp32 path: LDS-tiled FMA, same epilogues.
#include <algorithm>
#include <type_traits>

#include "isd_common.h"

namespace isd {
namespace {

constexpr int BK = 32;            // k per pipeline stage (one MFMA k-step)
constexpr int TM2 = 224, TN2 = 256;
constexpr int GROUP_BYTES = 16 * BK * 2;                 // 16 rows x 64 B
constexpr int AG = TM2 / 16;              // A row groups of 16 rows per tile
constexpr int kNsA = 10;                  // A ring depth (10 x 14 KB)
constexpr int kAStage = AG * GROUP_BYTES;
constexpr int kBRing = 4;                 // B operands: a register ring of this many stages,
constexpr int kBDepth = kBRing - 1;       // loaded this many stages ahead
constexpr int kEpiLds = 4 * 128 * 68 * 4; // epilogue staging: 4 waves x 128 rows x 68 floats
constexpr int kBigLds = kNsA * kAStage > kEpiLds ? kNsA * kAStage : kEpiLds;
static_assert(kBDepth <= kNsA - 2, "the B wait must cover the A wait");
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

// Packed weight layout of the bf16 path: the B operand of one 32x32x16 MFMA is 1 KB contiguous.
// Block (nb, kb) holds rows 32 nb .. 32 nb + 31 and k = 16 kb .. 16 kb + 15; its lane l part
// (16 bytes) is row 32 nb + l%32, k = 16 kb + 8 (l/32) .. + 7, at element
// ((nb (K/16) + kb) 64 + l) 8.  Rows are padded with zeros to a multiple of 32.
__device__ __forceinline__ const uint16_t* packed_operand(const uint16_t* p, int nb, int K, int kb, int lane) {
  return p + ((size_t)nb * (K / 16) + kb) * 512 + lane * 8;
}
// (a global-memory load: p points into device memory, never LDS or scratch)
__device__ __forceinline__ bf16x8_t ld_operand(const uint16_t* p) {
  return as_bf16x8(*(const __attribute__((address_space(1))) u32x4_t*)p);
}

// 1 KB of zeros: the operands of the padding stages that round a split's stage count up to a
// whole number of operand-ring rounds (0 x 0 products leave every accumulator unchanged).
__device__ __attribute__((aligned(1024))) uint16_t kZeroOperand[512] = {};

// How a pipeline step picks its load sources: every stage inside the product (plain
// addresses), or product / zero stages, or product / fused LoRA / zero stages.
constexpr int kPlainStages = 0, kZeroTail = 1, kLoraTail = 2;
template <int M> using StageMode = std::integral_constant<int, M>;

template <typename T, int EPI>
__device__ __forceinline__ void epilogue_store_t(const GemmArgs& a, int row, int col, float v, float v_up) {
  if (row >= a.M || col >= a.N) return;
  if (a.delta_row) {
    const int dr = a.delta_row[row];
    if (dr >= 0) {
      v += a.delta[(size_t)dr * a.ldd + col];
      if (EPI == EPI_SWIGLU) v_up += a.delta[(size_t)dr * a.ldd + a.delta_off2 + col];
    }
  }
  if (EPI == EPI_STORE) {
    ((T*)a.C)[(size_t)row * a.ldc + col] = from_f<T>(v);
  } else if (EPI == EPI_STORE_F32) {
    ((float*)a.C)[(size_t)row * a.ldc + col] = v;
  } else if (EPI == EPI_RESID) {
    a.R[(size_t)row * a.ldr + col] += v;
  } else {
    const float s = v / (1.0f + expf(-v));
    ((T*)a.C)[(size_t)row * a.ldc + col] = from_f<T>(s * v_up);
  }
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// D = A * B + C for one 32x32x16 bf16 tile: lane l holds A row (l%32) and B column (l%32)
// with k-values 8*(l/32) .. 8*(l/32)+7; D register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.  (On gfx950 this tile sustains about 1.5x the rate of 16x16x32.)
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LORA: the instance that can run fused LoRA stages (a separate instance, so that each one
// holds only two versions of the pipeline loop: a third does not fit the registers).
// WV: waves per workgroup (4, 3 or 2), i.e. a 224 x 64 WV output tile.  The per-wave work and
// the k order are the same for every WV; fewer waves per workgroup give more workgroups for a
// product whose 4-wave grid leaves CUs idle, each CU then streaming less data per stage.
template <int EPI, bool PARTIAL, bool LORA, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_big_kernel(GemmArgs a, int n_mt, int n_units, int S, float* part) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int TNO = DUAL ? 32 * WV : 64 * WV;   // output columns per workgroup
  constexpr int kALoads = (AG + WV - 1) / WV;     // A loads per wave and stage (the 14 groups over WV waves)
  constexpr int PER = kALoads + 4;                // loads per wave and pipeline step
  static_assert(WV >= 2 && WV <= 4 && kALoads <= 13, "2 to 4 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBigLds];

  const int id = blockIdx.x;
  const int grp = id / (8 * n_mt), rem = id % (8 * n_mt);
  const int mt = rem / 8, unit = grp * 8 + (rem % 8);
  if (unit >= n_units) return;
  const int nt = unit / S, sp = unit % S;
  const int kt_per = (a.K / BK) / S;
  const int kbase = sp * kt_per * BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // This workgroup's rows: row tile mt of TM2 rows, or, with a live-row count on the device
  // (a packed decode pass), the live rows split evenly over the n_mt tiles in whole 32-row
  // blocks.  Only the nblk blocks holding this tile's live rows are multiplied and stored.
  int th = TM2, m_lim = a.M;
  if (a.m_live) {
    m_lim = min(__builtin_amdgcn_readfirstlane(*a.m_live), a.M);
    th = min(TM2, ((m_lim + n_mt - 1) / n_mt + 31) / 32 * 32);
  }
  const int n0 = nt * TNO, m0 = mt * th;
  if (m0 >= m_lim) return;
  const int row_lim = min(m_lim, m0 + th);
  const int nblk = min(7, (row_lim - m0 + 31) / 32);
  const uint16_t* zero = kZeroOperand + lane * 8;
  // stages kt_per .. kt_end-1: the fused LoRA expand (last split only); the stage count is
  // rounded up to whole ring rounds with zero stages (kZeroOperand)
  const LoraPlan lp = LORA ? lora_plan(a, n0, DUAL, sp == S - 1) : LoraPlan{};
  const int kt_end = kt_per + lp.n;
  const int kt_loop = (kt_end + kBRing - 1) / kBRing * kBRing;

  // A loader: wave w fills row groups min(w + WV i, 13), i < kALoads, of the 14 (with 4 or 3
  // waves some refill group 13 with the same bytes, so every wave issues kALoads loads per
  // stage).  Lane l writes LDS
  // bytes [16 l, 16 l + 16) of its group: row l/4, slot l%4, which holds k-chunk
  // (l%4) ^ ((row/4)%4) of that row.
  const int lrow = lane >> 2;
  const int chunk = (lane & 3) ^ ((lrow >> 2) & 3);
  const int aoff = gemm_seg_aoff(a, n0);
  const uint16_t* asrc[kALoads];
  const uint16_t* lsrc[kALoads];         // fused LoRA: the row's lora_a row (null: zeros)
  {
    // every row-index load is issued before any is used (one wait, not one per row group)
    int sr[kALoads], lr[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int mc = min(m0 + min(wave + WV * i, AG - 1) * 16 + lrow, a.M - 1);
      sr[i] = a.a_rows ? a.a_rows[mc] : mc;
      lr[i] = (LORA && lp.n) ? a.lora_rows[mc] : -1;
    }
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const bool valid = m0 + min(wave + WV * i, AG - 1) * 16 + lrow < row_lim;
      const int srow = valid ? max(sr[i], 0) : 0;   // unused rows: their outputs are never consumed
      const int l = valid ? lr[i] : -1;
      asrc[i] = (const uint16_t*)a.A + (size_t)srow * a.lda + aoff + kbase + chunk * 8;
      lsrc[i] = l >= 0 ? (const uint16_t*)a.lora_a + (size_t)l * a.ld_la + lp.seg_off + chunk * 8 : nullptr;
    }
  }
  // B: this wave's two 32-row operand blocks, straight from the packed weights into registers
  // (one contiguous 1 KB operand per k-step and block).  Block j is output columns
  // n0 + 64 w + 32 j .. (SwiGLU: gate block j = 0 and up block j = 1 of columns n0 + 32 w ..).
  const uint16_t* bsrc[2];
  const uint16_t* lbsrc[2];              // fused LoRA: the packed lora_b blocks of the same columns
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int nb = DUAL ? (n0 >> 5) + wave : (n0 >> 5) + 2 * wave + j;
    nb = min(nb, ((a.N + 31) >> 5) - 1);        // past the last block: outputs are discarded
    bsrc[j] = packed_operand((const uint16_t*)(DUAL && j ? a.B1 : a.B0), nb, a.K, kbase / 16, lane);
    lbsrc[j] = packed_operand((const uint16_t*)(DUAL && j ? a.lora_b1 : a.lora_b0), nb, a.lora_r, 0, lane);
  }
  // stage kt's sources: the product, then the LoRA stages, then zeros.  LoRA stage ls reads
  // k-step ls of the row's lora_a segment (SwiGLU: the gate and up halves follow each other, so
  // the offset is ls BK for both) and, per weight block j, its own k-step ls - j per (SwiGLU:
  // gate stages 0 .. per-1, up stages per .. 2 per-1; the other block's operand is zero).
  auto a_src = [&](int i, int kt) {
    const int ls = kt - kt_per;
    const uint16_t* l = (ls >= 0 && ls < lp.n && lsrc[i]) ? lsrc[i] + ls * BK : zero;
    return kt < kt_per ? asrc[i] + kt * BK : l;
  };
  auto b_src = [&](int j, int kt, int kk) {
    const int lk = kt - kt_per - (DUAL ? j * lp.per : 0);
    const uint16_t* l = (lk >= 0 && lk < (DUAL ? lp.per : lp.n)) ? lbsrc[j] + (2 * lk + kk) * 512 : zero;
    return kt < kt_per ? bsrc[j] + (2 * kt + kk) * 512 : l;
  };
  auto a_dma = [&](int i, uint8_t* st, int kt) {
    __builtin_amdgcn_global_load_lds((const void*)a_src(i, kt),
                                     (lds_void*)(st + min(wave + WV * i, AG - 1) * GROUP_BYTES), 16, 0, 0);
  };
  // operand ring: stage kt's B fragments in slot kt % kBRing, loaded kBDepth stages ahead
  bf16x8_t bq[kBRing][2][2];
  auto b_load = [&](int slot, int kt) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) bq[slot][j][kk] = ld_operand(b_src(j, kt, kk));
  };
  f32x16_t acc[7][2];
#pragma unroll
  for (int i = 0; i < 7; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // The loads follow a fixed pattern: pipeline step i issues kALoads A loads (stage
  // i + kNsA - 1) and 4 B loads (stage i + kBDepth), the last of them a B load, and the
  // prologue is the same pattern for the steps i = 1 - kNsA .. -1 without the B loads of
  // negative stages.  Stages past the last one load zeros, so the pattern never changes:
  // before step kt reads B stage kt exactly PER (kBDepth - 1) loads were issued after it, and
  // at least as many after A stage kt+1 because kBDepth <= kNsA - 2.
#pragma unroll
  for (int i = 1 - kNsA; i < 0; ++i) {
    const int sa = i + kNsA - 1, sb = i + kBDepth;
#pragma unroll
    for (int q = 0; q < kALoads; ++q) a_dma(q, smem + sa * kAStage, sa);
    if (sb >= 0) b_load(sb, sb);
  }

  // A operand read: row (lane%32) of a 32-row block, k-chunk 2 kk + lane/32 (swizzled)
  const int rig = lane & 15, half = (lane >> 4) & 1, khi = lane >> 5;
  const int rd0 = rig * (BK * 2) + half * GROUP_BYTES;
  const int sw = (rig >> 2) & 3;
  auto frag = [&](int kt, int kk, int i) {
    const uint8_t* st = smem + (kt % kNsA) * kAStage;
    return as_bf16x8(*(const u32x4_t*)(st + 2 * i * GROUP_BYTES + rd0 + (((2 * kk + khi) ^ sw) * 16)));
  };

  bf16x8_t x0[7], x1[7];
  wait_vmcnt<PER * (kBDepth - 1)>();                 // A stage 0 and B stage 0 have landed
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 7; ++i)
    if (i < nblk) x0[i] = frag(0, 0, i);
  wait_lgkm0();
  // One pipeline step per 32-k stage kt: make A stage kt+1 visible, then two halves of 14
  // MFMAs.  One wave per SIMD keeps the matrix unit fed by itself: the MFMAs are interleaved
  // with the LDS reads of the next k-step's A operands, the refill of the A slot of stage kt-1
  // (every wave finished it before the barrier) and the B loads of stage kt+kBDepth into the
  // ring slot of stage kt-1; a half ends by waiting for its LDS reads.
  // The rounds whose loads all fall inside the product run with plain addresses; the last
  // rounds select zero stages (no fused LoRA) or the LoRA and zero stages.
  auto round = [&](auto mode, int kt0) {
    constexpr int MODE = decltype(mode)::value;
#pragma unroll
    for (int d = 0; d < kBRing; ++d) {
      const int kt = kt0 + d;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<PER * (kBDepth - 1)>();   // B stage kt and A stage kt+1 have landed
      __builtin_amdgcn_s_barrier();      // no fence: the later stages' loads stay in flight
      __builtin_amdgcn_sched_barrier(0);
      {
        uint8_t* dst = smem + ((kt + kNsA - 1) % kNsA) * kAStage;
        const int ka = kt + kNsA - 1, kb = kt + kBDepth;
        const int nslot = (d + kBDepth) % kBRing;     // a constant once the loop is unrolled
#pragma unroll
        for (int m = 0; m < 14; ++m) {
          if ((m >> 1) < nblk) acc[m >> 1][m & 1] = mfma32x32x16(x0[m >> 1], bq[d][m & 1][0], acc[m >> 1][m & 1]);
          __builtin_amdgcn_sched_barrier(0);
          if (m < nblk) x1[m] = frag(kt, 1, m);
          if (m >= 1 && m <= kALoads) {
            const int q = m - 1;
            const uint16_t* src = MODE == kPlainStages ? asrc[q] + ka * BK
                                : MODE == kZeroTail   ? (ka < kt_per ? asrc[q] + ka * BK : zero)
                                                      : a_src(q, ka);
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             (lds_void*)(dst + min(wave + WV * q, AG - 1) * GROUP_BYTES), 16, 0, 0);
          }
          if (m >= 6 && m < 10) {
            const int j = (m - 6) >> 1, kk = (m - 6) & 1;
            const uint16_t* src = MODE == kPlainStages ? bsrc[j] + (2 * kb + kk) * 512
                                : MODE == kZeroTail   ? (kb < kt_per ? bsrc[j] + (2 * kb + kk) * 512 : zero)
                                                      : b_src(j, kb, kk);
            bq[nslot][j][kk] = ld_operand(src);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lgkm0();
      {
        const int kn = kt + 1;                            // past the end: a slot of zeros
#pragma unroll
        for (int m = 0; m < 14; ++m) {
          if ((m >> 1) < nblk) acc[m >> 1][m & 1] = mfma32x32x16(x1[m >> 1], bq[d][m & 1][1], acc[m >> 1][m & 1]);
          __builtin_amdgcn_sched_barrier(0);
          if (m < nblk) x0[m] = frag(kn, 0, m);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wait_lgkm0();
    }
  };
  const int fast_end = max(0, (kt_per - (kNsA - 1)) / kBRing * kBRing);
  int kt0 = 0;
  for (; kt0 < fast_end; kt0 += kBRing) round(StageMode<kPlainStages>{}, kt0);
  for (; kt0 < kt_loop; kt0 += kBRing) round(StageMode<LORA ? kLoraTail : kZeroTail>{}, kt0);
  wait_vmcnt<0>();                                 // the loads past the last stage

  // Epilogue through LDS: each wave's 224 x 64 fp32 tile is staged row-major (rows padded to
  // 68 floats) in two halves (row blocks 0-3, then 4-6), then written out in 16-byte chunks.
  // Accumulator register r of block (i, j) in lane l is tile row 32 i + 8 (r/4) + 4 (l/32) + r%4,
  // column 32 j + l%32.  For SwiGLU columns 0-31 are the gate and 32-63 the up product.
  __syncthreads();                                 // every wave is done with the ring
  constexpr int LD = 68;
  float* tile = (float*)smem + (size_t)wave * (128 * LD);
  const int cl = lane & 31;
  const int wcol = n0 + (DUAL ? 32 : 64) * wave;   // first output column of this wave
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i0 = 4 * h, nb = h ? min(3, nblk - 4) : min(4, nblk), r0 = m0 + 128 * h;
    if (nb <= 0) break;                            // no live block in this half (uniform)
    if (h) __syncthreads();                        // the first half has been written out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nb) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          tile[(32 * i + 8 * (r >> 2) + 4 * khi + (r & 3)) * LD + 32 * j + cl] = acc[i0 + i][j][r];
    }
    __syncthreads();
    if (DUAL && !PARTIAL) {
      for (int q = lane; q < nb * 32 * 4; q += 64) {
        const int tr = q >> 2, c8 = (q & 3) * 8, row = r0 + tr, col = wcol + c8;
        if (row >= row_lim || col >= a.N) continue;
        float g[8], u[8];
        *(f32x4_t*)&g[0] = *(const f32x4_t*)&tile[tr * LD + c8];
        *(f32x4_t*)&g[4] = *(const f32x4_t*)&tile[tr * LD + c8 + 4];
        *(f32x4_t*)&u[0] = *(const f32x4_t*)&tile[tr * LD + 32 + c8];
        *(f32x4_t*)&u[4] = *(const f32x4_t*)&tile[tr * LD + 32 + c8 + 4];
        const int dr = a.delta_row ? a.delta_row[row] : -1;
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          float v0 = g[j], v1 = g[j + 1], w0 = u[j], w1 = u[j + 1];
          if (dr >= 0) {
            const float* dl = a.delta + (size_t)dr * a.ldd + col + j;
            v0 += dl[0];
            v1 += dl[1];
            w0 += dl[a.delta_off2];
            w1 += dl[a.delta_off2 + 1];
          }
          pk[j >> 1] = pack_bf16x2(v0 / (1.0f + expf(-v0)) * w0, v1 / (1.0f + expf(-v1)) * w1);
        }
        uint16_t* dst = (uint16_t*)a.C + (size_t)row * a.ldc + col;
        if (col + 8 <= a.N) {
          *(u32x4_t*)dst = (u32x4_t){pk[0], pk[1], pk[2], pk[3]};
        } else {
          for (int j = 0; j < 8 && col + j < a.N; ++j) dst[j] = (uint16_t)(pk[j >> 1] >> (16 * (j & 1)));
        }
      }
    } else if (!PARTIAL && EPI == EPI_STORE) {
      for (int q = lane; q < nb * 32 * 8; q += 64) {
        const int tr = q >> 3, c8 = (q & 7) * 8, row = r0 + tr, col = wcol + c8;
        if (row >= row_lim || col >= a.N) continue;
        float v[8];
        *(f32x4_t*)&v[0] = *(const f32x4_t*)&tile[tr * LD + c8];
        *(f32x4_t*)&v[4] = *(const f32x4_t*)&tile[tr * LD + c8 + 4];
        const int dr = a.delta_row ? a.delta_row[row] : -1;
        if (dr >= 0) {
          const float* dl = a.delta + (size_t)dr * a.ldd + col;
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += dl[j];
        }
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        uint16_t* dst = (uint16_t*)a.C + (size_t)row * a.ldc + col;
        if (col + 8 <= a.N) {
          *(u32x4_t*)dst = (u32x4_t){pk[0], pk[1], pk[2], pk[3]};
        } else {
          for (int j = 0; j < 8 && col + j < a.N; ++j) dst[j] = (uint16_t)(pk[j >> 1] >> (16 * (j & 1)));
        }
      }
    } else {
      // fp32 outputs: split-K partials (raw sums), fp32 store or residual add (with delta)
      for (int q = lane; q < nb * 32 * 16; q += 64) {
        const int tr = q >> 4, c4 = (q & 15) * 4, row = r0 + tr;
        // SwiGLU partials: columns 0-31 of the tile are gate sums, 32-63 up sums
        const int col = DUAL ? wcol + (c4 & 31) : wcol + c4;
        if (row >= row_lim || col >= a.N) continue;
        f32x4_t v = *(const f32x4_t*)&tile[tr * LD + c4];
        if (PARTIAL) {
          float* dst = DUAL ? part + ((size_t)sp * a.M + row) * (2 * (size_t)a.N) + (c4 >> 5) * a.N + col
                            : part + ((size_t)sp * a.M + row) * (size_t)a.N + col;
          *(f32x4_t*)dst = v;
        } else {
          const int dr = a.delta_row ? a.delta_row[row] : -1;
          if (dr >= 0) v += *(const f32x4_t*)(a.delta + (size_t)dr * a.ldd + col);
          if (EPI == EPI_RESID) {
            f32x4_t* dst = (f32x4_t*)(a.R + (size_t)row * a.ldr + col);
            *dst = *dst + v;
          } else {
            *(f32x4_t*)((float*)a.C + (size_t)row * a.ldc + col) = v;
          }
        }
      }
    }
  }
}

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
        __builtin_amdgcn_global_load_lds((const void*)(live ? wsrc[j] + (2 * kt + kk) * 512 : l),
                                         (lds_void*)(st + (2 * MT + 2 * NB * wave + 2 * j + kk) * 1024), 16, 0, 0);
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

// Sum the split-K partials in split order and apply the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, int S, const float* part) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  const size_t ld = DUAL ? 2 * (size_t)a.N : (size_t)a.N;
  const int m_lim = a.m_live ? min(*a.m_live, a.M) : a.M;       // live rows of a packed pass
  const size_t n4 = (size_t)m_lim * a.N / 4;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e * 4 / a.N), col = (int)(e * 4 % a.N);
    f32x4_t v = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float* pr = part + ((size_t)s * a.M + row) * ld;
      v += *(const f32x4_t*)(pr + col);
      if (DUAL) u += *(const f32x4_t*)(pr + a.N + col);
    }
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
constexpr int kMaxSplits = 16;
__global__ __launch_bounds__(kNormThreads) void splitk_resid_norm_kernel(GemmArgs a, int S, const float* part) {
  __shared__ float sh[kNormThreads / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (a.m_live && row >= *a.m_live) return;        // a dead row of a packed pass
  const int dr = a.delta_row ? a.delta_row[row] : -1;
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
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < S; ++s) v += *(const f32x4_t*)(prow + s * split_stride + c);
      if (dr >= 0) v += *(const f32x4_t*)(a.delta + (size_t)dr * a.ldd + c);
      const f32x4_t r = *(const f32x4_t*)(R + c) + v;
      *(f32x4_t*)(R + c) = r;
      rv[k] = r;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(r[j], r[j], ss);
    }
  }
  const float tot = block_sum_1024(ss, sh);
  const float denom = sqrtf(tot / (float)a.N + a.norm_eps);
  const bf16* g = (const bf16*)a.norm_g;
  bf16* y = (bf16*)a.norm_out + (size_t)row * a.N;
#pragma unroll
  for (int k = 0; k < kNormMaxGroups; ++k) {
    const int c = 4 * (tid + kNormThreads * k);
    if (c < a.N) {
#pragma unroll
      for (int j = 0; j < 4; ++j) y[c + j] = from_f<bf16>((rv[k][j] / denom) * to_f(g[c + j]));
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
    if (norm) {
      hipLaunchKernelGGL(splitk_resid_norm_kernel, dim3(a.M), dim3(kNormThreads), 0, s, a, S, (const float*)a.part);
      return hipGetLastError();
    }
    const size_t n4 = (size_t)a.M * a.N / 4;
    const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel<EPI>, dim3(blocks), dim3(256), 0, s, a, S, (const float*)a.part);
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
  const int n_mt = (a.M + TM2 - 1) / TM2;
  const int S = (a.splits > 1 && a.part) ? a.splits : 1;
  const int WV = big_waves<EPI>(a, n_mt, S);
  const int tno = (EPI == EPI_SWIGLU ? 32 : 64) * WV;
  const int n_nt = (a.N + tno - 1) / tno;
  const int units = n_nt * S;
  dim3 grid(((units + 7) / 8) * 8 * n_mt);
#define ISD_BIG(P, L, W) \
  hipLaunchKernelGGL((gemm_bf16_big_kernel<EPI, P, L, W>), grid, dim3(64 * W), 0, s, a, n_mt, units, S, P ? a.part : nullptr)
#define ISD_BIG_W(P, L) \
  if (WV == 4) ISD_BIG(P, L, 4); \
  else if (WV == 3) ISD_BIG(P, L, 3); \
  else ISD_BIG(P, L, 2);
  const bool lora = a.lora_r > 0;
  if (S > 1) {
    if (lora) { ISD_BIG_W(true, true) }
    else { ISD_BIG_W(true, false) }
  } else {
    if (lora) { ISD_BIG_W(false, true) }
    else { ISD_BIG_W(false, false) }
  }
#undef ISD_BIG_W
#undef ISD_BIG
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
  // automatic: the skinny kernel up to 64 rows, and up to 128 rows unless the product is so
  // wide (the LM head) that the tiled kernel's 224-row tiles have work for every CU
  const bool skinny = a.path == GEMM_PATH_SKINNY ||
                      (a.path == GEMM_PATH_AUTO && (a.M <= 64 || (a.M <= kSkinnyMaxRows && a.N <= 65536)));
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
