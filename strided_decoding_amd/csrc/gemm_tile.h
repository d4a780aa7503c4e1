// Shared pieces of the bf16 projection GEMMs (the packed weight operands, the 32x32x16 MFMA
// tile, the epilogues) and the tiled kernel.
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
#pragma once
#include <algorithm>
#include <type_traits>

#include "isd_common.h"

namespace isd {
namespace {

constexpr int BK = 32;            // k per pipeline stage (one MFMA k-step)
constexpr int TM2 = 224, TN2 = 256;
constexpr int GROUP_BYTES = 16 * BK * 2;                 // 16 rows x 64 B
constexpr int AG = TM2 / 16;              // A row groups of 16 rows per tile
constexpr int kNsA = 8;                   // A ring depth (8 x 14 KB; 6, 7, 9 and 10 measured slower)
constexpr int kAStage = AG * GROUP_BYTES;
constexpr int kBRing = 4;                 // B operands: a register ring of this many stages,
constexpr int kBDepth = kBRing - 1;       // loaded this many stages ahead
constexpr int kEpiLds = 4 * 128 * 68 * 4; // epilogue staging: 4 waves x 128 rows x 68 floats
constexpr int kBigLds = kNsA * kAStage > kEpiLds ? kNsA * kAStage : kEpiLds;
static_assert(kBDepth <= kNsA - 2, "the B wait must cover the A wait");

// Packed weight layout of the bf16 path: the B operand of one 32x32x16 MFMA is 1 KB contiguous.
// Block (nb, kb) holds rows 32 nb .. 32 nb + 31 and k = 16 kb .. 16 kb + 15; its lane l part
// (16 bytes) is row 32 nb + l%32, k = 16 kb + 8 (l/32) .. + 7, at element
// ((nb (K/16) + kb) 64 + l) 8.  Rows are padded with zeros to a multiple of 32.
__device__ __forceinline__ const uint16_t* packed_operand(const uint16_t* p, int nb, int K, int kb, int lane) {
  return p + ((size_t)nb * (K / 16) + kb) * 512 + lane * 8;
}
// (a global-memory load: p points into device memory, never LDS or scratch; non-temporal, as
// a weight streamed once per product should not displace cached activation rows: measured
// -2 % per decode pass at 64 slots)
__device__ __forceinline__ bf16x8_t ld_operand(const uint16_t* p) {
  return as_bf16x8(__builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)p));
}

// 1 KB of zeros: the operands of the padding stages that round a split's stage count up to a
// whole number of operand-ring rounds (0 x 0 products leave every accumulator unchanged).
__device__ __attribute__((aligned(1024))) uint16_t kZeroOperand[512] = {};

// How a pipeline step picks its load sources: every stage inside the product (plain
// addresses), or product / zero stages, or product / fused LoRA / zero stages.
constexpr int kPlainStages = 0, kZeroTail = 1, kLoraTail = 2;
template <int M> using StageMode = std::integral_constant<int, M>;

// SwiGLU of one output: silu(g) u = g u / (1 + e^-g), with e^-g = 2^(-g log2 e) and the
// reciprocal taken by the hardware's exp2 and reciprocal instructions (about 1 ulp each: the
// result is rounded to bf16 where it is stored, and every kernel uses this one formula).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g)) * u;
}

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
    ((T*)a.C)[(size_t)row * a.ldc + col] = from_f<T>(silu_mul(v, v_up));
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
// NB: the number of live 32-row blocks of the tile (1 to 7), a compile-time constant.
template <int EPI, bool PARTIAL, bool LORA, int WV, int NB>
__device__ __forceinline__ void big_tile(const GemmArgs& a, uint8_t* smem, int unit, int S, float* part, int m0,
                                         int row_lim) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int TNO = DUAL ? 32 * WV : 64 * WV;   // output columns per workgroup
  constexpr int kALoads = (AG + WV - 1) / WV;     // A loads per wave and stage (the 14 groups over WV waves)
  constexpr int PER = kALoads + 4;                // loads per wave and pipeline step
  static_assert(WV >= 2 && WV <= 4 && kALoads <= 13, "2 to 4 waves");
  static_assert(NB >= 1 && NB <= 7, "1 to 7 row blocks");
  constexpr int nblk = NB;
  const int nt = unit / S, sp = unit % S;
  const int kt_per = (a.K / BK) / S;
  const int kbase = sp * kt_per * BK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = nt * TNO;
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
  const int cl = lane & 31;
  const int wcol = n0 + (DUAL ? 32 : 64) * wave;   // first output column of this wave
  __syncthreads();                                 // every wave is done with the ring
  if (DUAL && !PARTIAL && !a.delta_row) {
    // SwiGLU without a delta: the gate and up sums of an output share a lane and a register
    // index, so the outputs are formed in registers.  Adjacent lanes trade one value so that each
    // holds two adjacent columns of one row (rows r and r + 1 of a register pair: the even lane
    // keeps row r, the odd lane row r + 1), the bf16 pairs are staged row-major in this wave's
    // LDS rows (40 bf16 per row: 16-byte aligned), and each row's 64 bytes leave in 16-byte stores.
    constexpr int LDW = 20;                        // 32-bit words per staged row
    uint32_t* st = (uint32_t*)smem + wave * (TM2 * LDW);
    const bool odd = cl & 1;
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float x0 = silu_mul(acc[i][0][r], acc[i][1][r]);          // row t, column cl
        const float x1 = silu_mul(acc[i][0][r + 1], acc[i][1][r + 1]);  // row t + 1, column cl
        const float give = odd ? x0 : x1;
        const float got = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, give), 0xB1, 0xF, 0xF, false));  // lane ^ 1
        const uint32_t w = odd ? pack_bf16x2(got, x1) : pack_bf16x2(x0, got);
        const int t = 32 * i + 8 * (r >> 2) + 4 * khi + (r & 3) + (odd ? 1 : 0);
        st[t * LDW + (cl >> 1)] = w;
      }
    // (one wave's LDS accesses are processed in order: its reads see its writes)
    for (int q = lane; q < NB * 32 * 4; q += 64) {
      const int t = q >> 2, c8 = (q & 3) * 8, row = m0 + t, col = wcol + c8;
      if (row >= row_lim || col >= a.N) continue;
      const u32x4_t v = *(const u32x4_t*)(st + t * LDW + c8 / 2);
      uint16_t* dst = (uint16_t*)a.C + (size_t)row * a.ldc + col;
      if (col + 8 <= a.N) {
        *(u32x4_t*)dst = v;
      } else {
        for (int j = 0; j < 8 && col + j < a.N; ++j) dst[j] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
      }
    }
    return;
  }
  constexpr int LD = 68;
  float* tile = (float*)smem + (size_t)wave * (128 * LD);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i0 = 4 * h, nb = h ? min(3, NB - 4) : min(4, NB), r0 = m0 + 128 * h;
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
          pk[j >> 1] = pack_bf16x2(silu_mul(v0, w0), silu_mul(v1, w1));
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

// One workgroup: row tile mt of the rows (with a live-row count on the device, a packed decode
// pass, the live ones) split evenly over the n_mt tiles in whole 32-row blocks.  The
// tile body is instantiated for every count of live 32-row blocks, so that the blocks past the
// live rows cost neither an MFMA nor a branch in the pipeline loop (a uniform branch around
// each MFMA and operand read made the decode launches 10-25 % slower).
template <int EPI, bool PARTIAL, bool LORA, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_big_kernel(GemmArgs a, int n_mt, int n_units, int S, float* part) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kBigLds];
  const int id = blockIdx.x;
  const int grp = id / (8 * n_mt), rem = id % (8 * n_mt);
  const int mt = rem / 8, unit = grp * 8 + (rem % 8);
  if (unit >= n_units) return;
  const int m_lim = a.m_live ? min(__builtin_amdgcn_readfirstlane(*a.m_live), a.M) : a.M;
  const int th = min(TM2, ((m_lim + n_mt - 1) / n_mt + 31) / 32 * 32);
  const int m0 = mt * th;
  if (m0 >= m_lim) return;
  const int row_lim = min(m_lim, m0 + th);
  switch (min(7, (row_lim - m0 + 31) / 32)) {
    case 1: big_tile<EPI, PARTIAL, LORA, WV, 1>(a, smem, unit, S, part, m0, row_lim); break;
    case 2: big_tile<EPI, PARTIAL, LORA, WV, 2>(a, smem, unit, S, part, m0, row_lim); break;
    case 3: big_tile<EPI, PARTIAL, LORA, WV, 3>(a, smem, unit, S, part, m0, row_lim); break;
    case 4: big_tile<EPI, PARTIAL, LORA, WV, 4>(a, smem, unit, S, part, m0, row_lim); break;
    case 5: big_tile<EPI, PARTIAL, LORA, WV, 5>(a, smem, unit, S, part, m0, row_lim); break;
    case 6: big_tile<EPI, PARTIAL, LORA, WV, 6>(a, smem, unit, S, part, m0, row_lim); break;
    default: big_tile<EPI, PARTIAL, LORA, WV, 7>(a, smem, unit, S, part, m0, row_lim); break;
  }
}

// Launch of the tiled kernel for one epilogue.
template <int EPI>
hipError_t launch_big_impl(const GemmArgs& a, dim3 grid, int WV, int n_mt, int units, int S, hipStream_t s) {
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
  return hipGetLastError();
}

}  // namespace

// Tiled-kernel launch for epilogue EPI (each epilogue's instances compile in a translation
// unit of their own, k_gemm_big_*.hip).
template <int EPI>
hipError_t launch_big_kernel(const GemmArgs& a, dim3 grid, int WV, int n_mt, int units, int S, hipStream_t s);

}  // namespace isd
