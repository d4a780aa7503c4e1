// Projection GEMMs of the decode step: Y[M, N] = X[M, K] W[N, K]^T with fused epilogues
// (bf16 store, fp32 store, fp32 residual add, SwiGLU of a gate/up pair) and the MASK-row
// LoRA delta.  bf16 path: MFMA 16x16x32 tiles, LDS double buffering; fp32 path: LDS-tiled
// FMA.  Per output element the K order is fixed (k = 0, 32, 64, ...), independent of M and
// of which other rows share the tile, so a row's result does not depend on the batch.
#include "isd_common.h"

namespace isd {
namespace {

constexpr int BM = 128;        // rows per tile
constexpr int BK = 64;         // k per LDS stage (two MFMA k-steps)
constexpr int LDSS = BK + 8;   // LDS row stride in bf16 (144 B; breaks bank aliasing)

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

// 256 threads = 4 waves in a 2 x 2 arrangement, each wave a 64 x 64 sub-tile of 4 x 4 MFMA
// tiles.  EPI_SWIGLU interleaves gate and up in 16-column blocks of the B tile so that a
// lane holds gate and up of the same output element.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU);
  constexpr int BNO = DUAL ? 64 : 128;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDSS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * LDSS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BNO, m0 = blockIdx.y * BM;
  const uint16_t* A = (const uint16_t*)a.A;
  const uint16_t* B0 = (const uint16_t*)a.B0;
  const uint16_t* B1 = (const uint16_t*)a.B1;

  // global -> register staging: 4 chunks of 16 B per thread for each operand
  const uint16_t* pa[4];
  const uint16_t* pb[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, kc = (c & 7) * 8;
    soff[i] = row * LDSS + kc;
    const int m = m0 + row;
    int src = -1;
    if (m < a.M) src = a.a_rows ? a.a_rows[m] : m;
    pa[i] = src >= 0 ? A + (size_t)src * a.lda + kc : nullptr;
    int n;
    const uint16_t* Bp;
    if (DUAL) {
      const int blk = row >> 4;
      Bp = (blk & 1) ? B1 : B0;
      n = n0 + (blk >> 1) * 16 + (row & 15);
    } else {
      Bp = B0;
      n = n0 + row;
    }
    pb[i] = n < a.N ? Bp + (size_t)n * a.ldb + kc : nullptr;
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = pa[i] ? *(const u32x4_t*)(pa[i] + k0) : zero;
      rb[i] = pb[i] ? *(const u32x4_t*)(pb[i] + k0) : zero;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4_t*)&As[buf][soff[i]] = ra[i];
      *(u32x4_t*)&Bs[buf][soff[i]] = rb[i];
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 15, lg = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = as_bf16x8(*(const u32x4_t*)&As[buf][(wm * 64 + t * 16 + lr) * LDSS + kk * 32 + lg]);
        bfr[t] = as_bf16x8(*(const u32x4_t*)&Bs[buf][(wn * 64 + t * 16 + lr) * LDSS + kk * 32 + lg]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + i * 16 + rq + r;
      if (DUAL) {
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const int col = n0 + (2 * wn + jp) * 16 + lr;
          epilogue_store_t<bf16, EPI>(a, row, col, acc[i][2 * jp][r], acc[i][2 * jp + 1][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 64 + j * 16 + lr;
          epilogue_store_t<bf16, EPI>(a, row, col, acc[i][j][r], 0.f);
        }
      }
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

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % BK != 0) return hipErrorInvalidValue;
  const int bno = a.epi == EPI_SWIGLU ? 64 : 128;
  dim3 grid((a.N + bno - 1) / bno, (a.M + BM - 1) / BM);
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE>, grid, dim3(256), 0, s, a); break;
    case EPI_STORE_F32: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE_F32>, grid, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_RESID>, grid, dim3(256), 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL(gemm_bf16_kernel<EPI_SWIGLU>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
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
  return hipGetLastError();
}

}  // namespace isd
