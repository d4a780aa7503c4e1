// MASK-row LoRA shrink of R-ISD: S[m, :] = X[rows[m], :] A^T, rank-r bottleneck inputs of the
// gated adapter (it acts on the MASK rows only, the clean rows pass through the base weights).
//
// The product is tiny (tens of rows, N = r .. 3r columns, K = d or d_ffn), so its cost is the
// chain of memory round trips, not bandwidth or MFMA rate.  One launch does it all: workgroup
// (n-block, k-split, row block) has 8 waves, each wave takes one 128-wide k chunk and issues all
// of its operand loads at once (8 k-steps x (row tiles + 1) 16-byte loads per lane, straight
// into registers), multiplies them with 32x32x16 MFMAs, and the 8 per-wave results are summed
// in wave order through LDS.  With more than one k-split each workgroup writes its fp32 partial,
// and the last workgroup of the tile to arrive (an arrival counter per tile, no spinning) sums
// all partials in split order and stores the bf16 result, then clears the counter for the
// next launch.  Every output has the same accumulation order whatever the arrival order.
#include "isd_common.h"

namespace isd {
namespace {

constexpr int kShrinkWaves = 8;     // waves per workgroup, one 128-wide k chunk each
constexpr int kChunk = 128;
constexpr int kMaxShrinkSplits = 32;  // K <= 32768

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// A row (l%32) and B column (l%32) hold k = 8 (l/32) .. + 7; D register r of lane l is row
// 8 (r/4) + 4 (l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16_t mma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) {
  return as_bf16x8(*(const __attribute__((address_space(1))) u32x4_t*)p);
}

template <int MT>
__global__ __launch_bounds__(64 * kShrinkWaves) void lora_shrink_kernel(ShrinkArgs a) {
  __shared__ float red[kShrinkWaves * MT * 1024];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.x, sp = blockIdx.y, S = gridDim.y;
  const int m0 = blockIdx.z * 32 * MT;
  const int chunk = sp * kShrinkWaves + wave;

  f32x16_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  if (chunk < a.K / kChunk) {
    const uint16_t* xp[MT];
    int src[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = min(m0 + 32 * t + (lane & 31), a.M - 1);
      src[t] = a.rows ? a.rows[m] : m;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)   // rows past M or without a source: any row (never stored)
      xp[t] = (const uint16_t*)a.X + (size_t)max(src[t], 0) * a.ldx + chunk * kChunk + 8 * (lane >> 5);
    // packed operand block (nb, kb): lane l holds row 32 nb + l%32, k = 16 kb + 8 (l/32) .. + 7
    const uint16_t* ap = (const uint16_t*)a.A + ((size_t)nb * (a.K / 16) + chunk * 8) * 512 + lane * 8;
    bf16x8_t xv[8][MT], av[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[ks][t] = ld16(xp[t] + 16 * ks);
      av[ks] = ld16(ap + ks * 512);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load in flight before the first product
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mma32(xv[ks][t], av[ks], acc[t]);
  }
  // element e = (t 16 + r) 64 + lane of every wave's tile, summed over the waves in order
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * MT * 16 + t * 16 + r) * 64 + lane] = acc[t][r];
  __syncthreads();
  constexpr int kPer = MT * 1024 / (64 * kShrinkWaves);   // elements per thread
  float v[kPer];
  int row[kPer], col[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * 64 * kShrinkWaves;
    float s = red[e];
#pragma unroll
    for (int w = 1; w < kShrinkWaves; ++w) s += red[w * MT * 1024 + e];
    v[i] = s;
    const int t = e >> 10, r = (e >> 6) & 15, l = e & 63;
    row[i] = m0 + 32 * t + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    col[i] = 32 * nb + (l & 31);
  }
  if (S > 1) {
    // The partials go out as device-scope relaxed atomic stores, which write through to the
    // point where every XCD sees them, and are read back the same way: no cache-wide
    // write-back or invalidation (a device-scope fence costs several microseconds here).
    // Each thread waits for its own stores before the barrier that precedes the arrival.
    // Why the last workgroup sees every partial (an argument about the ISA's ordering, not the
    // source-level memory model, in which relaxed atomics alone would not order the data):
    //  1. a device-scope atomic store is performed at the memory side shared by all XCDs (it
    //     bypasses the XCD's L2), and s_waitcnt(0) returns only once every store of the
    //     thread has been acknowledged there, i.e. is visible to any later device-scope load;
    //  2. the barrier after that wait means thread 0's counter increment (a device-scope atomic
    //     performed at the same memory side) is issued after all 512 threads' partials are
    //     visible; the counter's value orders the workgroups of a tile;
    //  3. the workgroup that reads S - 1 from the counter knows every other workgroup's
    //     increment happened, hence (2) every other partial is visible; its loads of the
    //     partials are device-scope atomic loads (no stale L2 or L1 line can serve them) and are
    //     issued only after the counter's value has returned (s_last through LDS and a barrier).
    //  The counter is reset by that last workgroup with a device-scope store; the next launch
    //  of the kernel starts after this one has ended (stream order), so it sees zero.
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (row[i] < a.M)
        __hip_atomic_store(a.part + ((size_t)sp * a.M + row[i]) * a.N + col[i], v[i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(&a.cnt[blockIdx.z * gridDim.x + nb], 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (!s_last) return;
    // every split's partial is loaded before the first add (one round trip), then summed in
    // split order
    float p[kPer][kMaxShrinkSplits];
#pragma unroll
    for (int j = 0; j < kMaxShrinkSplits; ++j)
      if (j < S && j != sp)
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          p[i][j] = __hip_atomic_load(a.part + ((size_t)j * a.M + min(row[i], a.M - 1)) * a.N + col[i],
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxShrinkSplits; ++j)
        if (j < S) {
          const float q = j == sp ? v[i] : p[i][j];
          s = j == 0 ? q : s + q;
        }
      v[i] = s;
    }
    if (tid == 0) __hip_atomic_store(&a.cnt[blockIdx.z * gridDim.x + nb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (row[i] < a.M) ((bf16*)a.out)[(size_t)row[i] * a.ldo + col[i]] = from_f<bf16>(v[i]);
}

}  // namespace

int lora_shrink_splits(int K) { return (K / kChunk + kShrinkWaves - 1) / kShrinkWaves; }

hipError_t launch_lora_shrink(const ShrinkArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (!a.X || !a.A || !a.out || a.N <= 0 || a.N % 32 || a.K <= 0 || a.K % kChunk || a.ldx < a.K || a.ldo < a.N)
    return hipErrorInvalidValue;
  const int S = lora_shrink_splits(a.K);
  if (S > kMaxShrinkSplits) return hipErrorInvalidValue;
  const int MT = a.M <= 32 ? 1 : 2;
  const int rb = (a.M + 32 * MT - 1) / (32 * MT);
  if (S > 1 && (!a.part || !a.cnt || (size_t)rb * (a.N / 32) > (size_t)a.n_cnt ||
                (size_t)S * a.M * a.N > a.part_floats))
    return hipErrorInvalidValue;
  dim3 grid(a.N / 32, S, rb);
  if (MT == 1)
    hipLaunchKernelGGL(lora_shrink_kernel<1>, grid, dim3(64 * kShrinkWaves), 0, s, a);
  else
    hipLaunchKernelGGL(lora_shrink_kernel<2>, grid, dim3(64 * kShrinkWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace isd
