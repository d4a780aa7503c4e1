// Shared device helpers and internal structures of libisd (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/isd.h"

#define ISD_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------
// bfloat16 stored as raw bits.  Conversion to float is exact; float -> bf16 rounds to
// nearest-even (NaN kept quiet).
struct bf16 {
  uint16_t u;
};

ISD_DEV float to_f(float x) { return x; }
ISD_DEV float to_f(bf16 x) { return __uint_as_float((uint32_t)x.u << 16); }

template <typename T>
ISD_DEV T from_f(float f);
template <>
ISD_DEV float from_f<float>(float f) { return f; }
template <>
ISD_DEV bf16 from_f<bf16>(float f) {   // v_cvt_pk_bf16_f32: round to nearest even
  bf16 r;
  r.u = __builtin_bit_cast(uint16_t, (__bf16)f);
  return r;
}
// Two floats rounded to bf16 (nearest even) and packed, lo in the low half.
ISD_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Cache-policy operand of a direct global->LDS load with the nt (non-temporal) bit: data read
// once per pass, which should not displace cached lines.
constexpr int kCachePolicyNT = 2;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA operand (8 bf16)
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16-byte load unit

ISD_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// D = A * B + C for one 16x16x32 bf16 tile.  Lane l holds A row (l%16), B column (l%16),
// each with 8 k-values in slots 8*(l/16) .. 8*(l/16)+7 (any fixed k permutation shared by
// A and B gives the same product); D lane l, register r is row 4*(l/16)+r, column l%16.
ISD_DEV f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split-K reduction of fp32 4-vectors: a = sum over s = 0 .. S-1 (1 <= S <= MAXS) of
// p[s * stride] and, with PAIR, b = the same at p + off, each added in split order starting from
// zero.  Every load is issued before the first add (one memory round trip instead of S dependent
// ones); the loads are unconditional, s > S - 1 re-reading split S - 1 (callers choose MAXS as
// the smallest power of two >= S, so that happens only for other S), and the adds past S are
// selected away.
template <int MAXS, bool PAIR>
ISD_DEV void sum_split_partials(const float* p, size_t stride, int S, size_t off, f32x4_t& a, f32x4_t& b) {
  f32x4_t ta[MAXS], tb[PAIR ? MAXS : 1];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const size_t o = (size_t)min(s, S - 1) * stride;
    ta[s] = *(const f32x4_t*)(p + o);
    if (PAIR) tb[s] = *(const f32x4_t*)(p + off + o);
  }
  a = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  b = a;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const bool in = s < S;
    const f32x4_t na = a + ta[s];
    a = in ? na : a;
    if (PAIR) {
      const f32x4_t nb = b + tb[s];
      b = in ? nb : b;
    }
  }
}
// The MAXS bucket of a split count: the smallest power of two >= S (S <= 16).
inline int split_bucket(int S) { return S <= 1 ? 1 : S <= 2 ? 2 : S <= 4 ? 4 : S <= 8 ? 8 : 16; }

// ---------------------------------------------------------------------------------------
// Wave (64-lane) reductions.
ISD_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
ISD_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over a 1024-thread block: wave trees, then the 16 wave sums in a fixed pairwise order.
// sh must hold 16 floats.  Every thread receives the total.
ISD_DEV float block_sum_1024(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = sh[2 * i] + sh[2 * i + 1];
  return ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
}
ISD_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): one round maps (c0,c1,c2,c3) under key
// (k0,k1) to (hi(M1 c2)^c1^k0, lo(M1 c2), hi(M0 c0)^c3^k1, lo(M0 c0)); the key is bumped by
// the Weyl constants between rounds.
ISD_DEV void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// u(slot, t, position, purpose) = ((word0 >> 8) + 1/2) * 2^-24, an odd multiple of 2^-25 in
// (0, 1), exact in double.  purpose 0 = acceptance test, 1 = categorical draw.
ISD_DEV double philox_uniform(uint64_t seed, uint32_t slot, uint32_t t, uint32_t pos, uint32_t purpose) {
  uint32_t c[4] = {slot, t, pos, purpose};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return ((double)(c[0] >> 8) + 0.5) * 0x1p-24;
}

// ---------------------------------------------------------------------------------------
// Internal structures shared by the runtime and the kernels.

// One attention work item: nq consecutive query positions pos0 .. pos0+nq-1 of `slot`,
// stored in activation rows row0 .. row0+nq-1.
typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N vector-memory operations of this wave are outstanding (direct
// global->LDS loads included: their data is in LDS once they are no longer counted).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Wait until every LDS read (and scalar load) of this wave has returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); }

struct AttnItem {              // query rows row0 .. row0+nq-1 of one slot at positions pos0 ..
  int32_t slot, row0, nq, pos0;
};

// Per-row, per-chunk statistics of a logits row: max m_c, lowest argmax, the second largest
// logit m2_c (equal to m_c when the maximum occurs twice), and s_c = sum_j exp((l_j - m_c)/T)
// over the chunk (double).
struct ChunkStat {
  float m;
  float m2;
  int32_t arg;
  int32_t pad;
  double s;
};

constexpr int kStatChunk = 4096;        // logits per statistics chunk

enum EpiMode : int { EPI_STORE = 0, EPI_STORE_F32 = 1, EPI_RESID = 2, EPI_SWIGLU = 3 };

struct GemmArgs {
  const void* A;             // [*, lda] act; row of output row m is a_rows ? a_rows[m] : m
  const int32_t* a_rows;     // optional gather (entries < 0 read as zero rows)
  int lda;
  const void* B0;            // [N, ldb] act (out x in)
  const void* B1;            // second operand for EPI_SWIGLU (up projection)
  int ldb;
  int M, N, K;
  int epi;
  void* C;                   // EPI_STORE / EPI_SWIGLU: act [M, ldc]; EPI_STORE_F32: float
  int ldc;
  float* R;                  // EPI_RESID: float residual [M, ldr], R += A B^T
  int ldr;
  const float* delta;        // optional LoRA delta rows [*, ldd] added before the epilogue
  const int32_t* delta_row;  // [M] delta row of output row m or -1
  int ldd;
  int delta_off2;            // EPI_SWIGLU: column offset of the up-projection delta
  int splits;                // split-K factor (bf16 path; 1 = none)
  float* part;               // split-K partials [splits, M, N (x2 for SwiGLU)] fp32
  // EPI_RESID only, optional: after R += X W^T, norm_out[row] = RMSNorm(R[row]) * norm_g
  // (act type), fused into the split-K reduction when there is one
  const void* norm_g;
  void* norm_out;
  float norm_eps;
  int path;                  // bf16 kernel choice: GEMM_PATH_AUTO / _TILED / _SKINNY / _TILED4..2
  // Segmented A (0 = off): output columns [seg_end[j-1], seg_end[j]) read A columns starting at
  // seg_aoff[j], i.e. several products X_j W_j^T with stacked W_j in one launch.  Segment ends
  // must be multiples of 256 (no column tile straddles two segments).
  int nseg;
  int seg_end[3];
  int seg_aoff[3];
  // Split-K (splits > 1) only: leave the fp32 partials for the consumer (the fused QKV reduce
  // in rope_append) instead of reducing them into C.
  int keep_part;
  // Fused LoRA expand (bf16 kernels; lora_r = 0: off).  For an output row m with
  // lora_rows[m] >= 0 the product runs over lora_r more k values: row lora_rows[m] of lora_a
  // (bf16, row stride ld_la) times the packed lora_b0 [N, lora_r]; rows with lora_rows[m] < 0
  // add exact zeros.  Column segment i ([lora_seg_end[i-1], lora_seg_end[i])) reads lora_a
  // columns i*lora_r ..; SwiGLU: the gate block reads columns 0 .. with lora_b0, then the up
  // block columns lora_r .. with lora_b1.  The extra k-stages belong to the last split.
  const int32_t* lora_rows;
  const void* lora_a;
  int ld_la;
  const void* lora_b0;
  const void* lora_b1;
  int lora_r;
  int lora_nseg;
  int lora_seg_end[3];
  // Optional (tiled kernel, decode): the number of live rows, read on the device.  The live
  // rows are the first *m_live of the M (the pass's packed rows); the row tiles shrink to
  // them (the grid still covers M) and rows past them are neither computed nor stored.
  const int32_t* m_live;
};
// TILED4 / TILED3 / TILED2: the tiled kernel with that many waves per workgroup (TILED and
// AUTO choose it by the grid's fill of the CUs)
enum { GEMM_PATH_AUTO = 0, GEMM_PATH_TILED = 1, GEMM_PATH_SKINNY = 2, GEMM_PATH_TILED4 = 3, GEMM_PATH_TILED3 = 4,
       GEMM_PATH_TILED2 = 5 };

// Fused-LoRA stage plan of a workgroup: its number of extra k-stages (32 k each) and, for
// extra stage ls, the lora_a column offset and the group (SwiGLU: 0 gate, 1 up; else 0).
struct LoraPlan {
  int n = 0, per = 0, seg_off = 0;
};
ISD_DEV LoraPlan lora_plan(const GemmArgs& a, int n0, bool dual, bool last_split) {
  LoraPlan p;
  if (a.lora_r <= 0 || !last_split) return p;
  p.per = a.lora_r / 32;
  p.n = dual ? 2 * p.per : p.per;
  int seg = 0;
  for (int j = 0; j + 1 < a.lora_nseg; ++j)
    if (n0 >= a.lora_seg_end[j]) seg = j + 1;
  p.seg_off = seg * a.lora_r;
  return p;
}
constexpr int kSkinnyMaxRows = 128;  // the skinny kernel holds at most four 32-row MFMA tiles

// A column offset of the output columns starting at n0 (segmented products; 0 otherwise).
ISD_DEV int gemm_seg_aoff(const GemmArgs& a, int n0) {
  int off = 0;
  for (int j = a.nseg - 1; j >= 0; --j)
    if (j == 0 || n0 >= a.seg_end[j - 1]) {
      off = a.seg_aoff[j];
      break;
    }
  return off;
}

// Split-K factor of a bf16 projection: a function of the output width and K only (never of
// the row count), so that a row's result is the same whatever the batch composition.
int gemm_splits(int n_out, int K, bool dual);

// ---------------------------------------------------------------------------------------
// Kernel launchers (defined in the .hip files).
namespace isd {

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s);
// bf16 weights of the GEMMs are in the packed operand layout (k_gemm.hip): elements of a
// packed [rows, cols] matrix, and the conversion from row-major
// MASK-row LoRA shrink: out[m, 0:N] = X[rows[m], 0:K] A^T in bf16 (A packed bf16 [N, K],
// N % 32 == 0, K % 128 == 0, K <= 32768; rows[m] < 0: the output row is unused).  One launch; with
// lora_shrink_splits(K) > 1 k-splits it needs part (>= splits * M * N floats) and cnt
// (>= ceil(M / 64) * N / 32 counters, zero before the first call and left zero by every call).
struct ShrinkArgs {
  const void* X;
  int ldx;
  const int32_t* rows;
  int M;
  const void* A;
  int N, K;
  void* out;
  int ldo;
  float* part;
  size_t part_floats;
  int32_t* cnt;
  int n_cnt;
};
int lora_shrink_splits(int K);
hipError_t launch_lora_shrink(const ShrinkArgs& a, hipStream_t s);
size_t packed_weight_elems(int rows, int cols);
hipError_t launch_pack_weights(const void* src, void* dst, int rows, int cols, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

struct AttnArgs {
  const void* q;             // [rows, Hq*hd] act (after RoPE)
  const void* k_pool;        // layer base: [n_pages, Hkv, P, hd]
  const void* v_pool;        // layer base: [n_pages, Hkv, hd, P]
  const int32_t* page_table; // [slots, max_pages]
  int max_pages;
  const AttnItem* items;
  int n_items;               // grid size (items beyond the live count have nq = 0)
  const int32_t* ctx_len;    // [slots] keys in the pages
  int Hq, Hkv, hd, P;
  int ncb;                   // 16-column query blocks per item (2 or 4): nq * Hq/Hkv <= 16 * ncb
  int split;                 // keys per split (0: one pass writes `out` directly)
  int max_splits;
  float* part_o;             // [max_splits, part_rows, Hq, hd]
  float* part_ml;            // [max_splits, part_rows, Hq, 2]
  int part_rows;
  void* out;                 // [rows, Hq*hd] act
  const int32_t* row_pos;    // [rows] position or -1 (combine, f32 path)
  const int32_t* row_slot;   // [rows] slot (f32 path)
  int n_rows;
};
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_combine_bf16(const AttnArgs& a, hipStream_t s);
// Keys per context split of a decode pass, from the slots, KV heads and longest context the
// context serves: 2048 when the (slot, KV head) pairs alone fill the chip, else about 2048
// workgroups at the longest context (short splits when few slots must still fill the chip).
// Fixed per context, so a row's attention never depends on the other rows of a pass.
int attn_split_len(int batch, int n_kv_heads, int max_ctx);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* table, float* X, int rows, int d, int mask_id, hipStream_t s);
template <typename T>
hipError_t launch_rmsnorm(const float* X, const T* g, T* Y, int rows, int d, float eps, hipStream_t s);

struct RopeAppendArgs {
  const float* qkv;          // [rows, (Hq+2Hkv)*hd] fp32 (the projection, unrounded)
  void* q_out;               // [rows, Hq*hd] act
  void* k_pool;              // layer base
  void* v_pool;
  const int32_t* page_table;
  int max_pages;
  const int32_t* row_pos;    // -1: dead row (no cache write, zero q)
  const int32_t* row_slot;
  const float* cos_t;        // [max_pos, hd/2]
  const float* sin_t;
  int rows, Hq, Hkv, hd, P;
  // Optional: read the projection from its split-K partials (part != null: fp32
  // [splits, rows, (Hq+2Hkv)*hd], summed in split order, plus the LoRA delta of MASK rows)
  // instead of qkv.  Either way q, k and v are rounded to act once, after RoPE.
  const float* part;
  int splits;
  const int32_t* delta_row;  // -1 / null: no delta
  const float* delta;
  int ldd;
};
template <typename T>
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s);
hipError_t launch_rope_tables(float* cos_t, float* sin_t, int max_pos, int hd, float base, hipStream_t s);

struct StepMeta {            // device buffers of the block / page machinery
  isd_slot* slots;
  int32_t* page_table;
  int max_pages;
  int32_t* free_stack;
  int32_t* n_free;
  int32_t* row_tok;
  int32_t* row_pos;
  int32_t* row_slot;
  int32_t* delta_row;        // [rows] LoRA delta row or -1
  int32_t* mask_rows;        // [max_batch*(N-1)] row of each MASK row or -1
  int32_t* ctx_len;          // [max_batch]
  AttnItem* items;
  int items_per_slot, q_max;   // decode: attention items per slot, query positions per item
  int max_batch, N, P, mask_id;
  int n_active;               // decode: the pass covers slots 0 .. n_active-1 (isd_step_active)
  int32_t* last_rows;        // prefill: last row of each prompt
  int32_t* zero_words;       // cleared once at init (arrival counters)
  int n_zero_words;
  int32_t* sticky_host;      // pinned host word: the first non-zero slot status (0 = none), or null
  // decode: slot b's live rows are rows row_off[b] .. row_off[b] + row_len[b] - 1 of the pass
  // (slots packed in order, B-state slots N rows, A-state 2N-1, others none); *m_live rows in all
  int32_t* row_off;
  int32_t* row_len;
  int32_t* m_live;
};
hipError_t launch_init_state(const StepMeta& m, int n_pages, hipStream_t s);
hipError_t launch_assemble(const StepMeta& m, hipStream_t s);
hipError_t launch_attn_setup(AttnItem* items, int32_t* row_pos, int32_t* row_slot, const int32_t* ctx_len,
                             const int32_t* q_len, int batch, int rows, hipStream_t s);
hipError_t launch_truncate(const StepMeta& m, const int32_t* order, int n, hipStream_t s);

constexpr int kMaxPrefillSlots = 256;
struct PrefillCall {
  int n;
  int32_t slot[kMaxPrefillSlots];
  int32_t off[kMaxPrefillSlots + 1];
  int32_t max_new[kMaxPrefillSlots];
  int32_t item_off[kMaxPrefillSlots + 1];   // first attention item of each prompt
};
hipError_t launch_prefill_setup(const StepMeta& m, const PrefillCall& c, const int32_t* prompt_ids,
                                int q_tile, int32_t* order_out, hipStream_t s);

static_assert(sizeof(isd_slot) == 128, "slot record layout is part of the ABI");

struct SampleArgs {
  isd_slot* slots;
  int n_slots;
  const int32_t* slot_ids;   // optional: slot index of work item i (prefill); NULL = i
  int N, V, propose;
  float T;
  uint64_t seed;
  const float* logits;       // current rows
  int rows_per_slot;         // R (decode) or 1 (prefill)
  const ChunkStat* stats;    // [rows, n_chunks]
  const float* q_logits;     // previous pass rows
  const ChunkStat* q_stats;
  int q_rows;
  int n_chunks;
  int32_t* tokens;           // [n_slots, N]
  int32_t* n_commit;
  int32_t* n_accept;
  int prefill;               // 1: draw the first token only (t = 0, position L)
  int32_t* first_tok;        // prefill output [n_slots]
  int meter;                 // 1: commit pending tokens untested, accumulate their acceptance
  double* margins;           // optional [n_slots, 2N]: margin of each decision (-1 past the last)
  int32_t* kinds;            // optional [n_slots, 2N]: ISD_DEC_* of each decision (-1 past the last)
  const int32_t* row_off;    // optional: first row of slot b (packed pass); null: b * rows_per_slot
};
// rows past *m_live (when given) are skipped
hipError_t launch_row_stats(const float* logits, int rows, int V, float T, ChunkStat* stats, hipStream_t s,
                            const int32_t* m_live = nullptr);
// Debug record: dst[r, 0:width] = src[row of rows[r], 0:width] for r < n, zeros when that row is
// outside [0, n_src) (ld and width in elements of elem_bytes; both multiples of 16 bytes).
// With row_off / row_len, rows[r] = b R + i names block row i of slot b, which is packed row
// row_off[b] + i (none when i >= row_len[b]); without, rows[r] is the row itself.
hipError_t launch_debug_gather(const void* src, size_t ld, const int32_t* rows, int n, int n_src, int width,
                               int elem_bytes, void* dst, hipStream_t s, const int32_t* row_off = nullptr,
                               const int32_t* row_len = nullptr, int R = 1);
hipError_t launch_decide(const SampleArgs& a, hipStream_t s);

}  // namespace isd
