// Paged causal attention for blocks of query rows (decode: 2N-1 rows per slot; prefill: tiles
// of consecutive prompt positions).  Keys and values are read only from the KV pages, the
// block's own K/V having been appended first, and a row at position p sees keys 0 .. p.
//
// bf16 path (head_dim 128): one wave per (item, KV head, context split).  The up to 64 query
// rows of a KV-head group (positions x G query heads) are the columns of two MFMA products
//   S^T = K Q^T          (A = 16 keys x 32 dims per step, B = Q^T)
//   O^T += V^T P^T       (A = V^T rows = dims, k = 32 keys; B = P^T)
// so that every operand is a 16-byte contiguous load: K pages are [token][dim], V pages are
// stored transposed [dim][token] within a page.  The key order inside a 32-key step is
// permuted so that the S^T accumulator registers of a lane are exactly the P^T operand
// slots of the next product (no cross-lane traffic).  Online softmax in the log2 domain with
// wave reductions over the 4 lane groups sharing a column.  Context splits begin at
// multiples of the split length and 32-key steps at absolute positions, and masked keys
// contribute exact zeros, so a row's result does not depend on the other rows of its block.
#include "isd_common.h"

namespace isd {
namespace {

constexpr int HD = 128;
constexpr float kNegInf = -__builtin_huge_valf();

ISD_DEV u32x4_t ld16(const uint16_t* p) { return *(const u32x4_t*)p; }

template <int NCB>
__global__ __launch_bounds__(64) void attn_bf16_kernel(AttnArgs a) {
  const AttnItem it = a.items[blockIdx.x];
  if (it.nq <= 0) return;
  const int kvh = blockIdx.y, split = blockIdx.z;
  const int lane = threadIdx.x, lr = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const int ctx = a.ctx_len[it.slot];
  const int key_hi = min(ctx, it.pos0 + it.nq);
  int k_begin = 0, k_end = key_hi;
  if (a.split) {
    k_begin = split * a.split;
    if (k_begin >= key_hi) return;
    k_end = min(key_hi, k_begin + a.split);
  }
  const float scale = 1.4426950408889634f * rsqrtf((float)HD);
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* kp = (const uint16_t*)a.k_pool;
  const uint16_t* vp = (const uint16_t*)a.v_pool;
  const size_t q_stride = (size_t)a.Hq * HD;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  bf16x8_t qf[NCB][4];
  int qpos[NCB];
  bool qvalid[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int qr = c * 16 + lr, p = qr / G, h = qr % G;
    qvalid[c] = p < it.nq;
    qpos[c] = it.pos0 + p;
    const uint16_t* src = q + (size_t)(it.row0 + p) * q_stride + (size_t)(kvh * G + h) * HD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[c][ks] = as_bf16x8(qvalid[c] ? ld16(src + ks * 32) : zero);
  }

  float m_run[NCB], l_run[NCB];
  f32x4_t o[8][NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    m_run[c] = kNegInf;
    l_run[c] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d][c] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* pt = a.page_table + (size_t)it.slot * a.max_pages;
  const size_t page_elems = (size_t)a.Hkv * 16 * HD;

  for (int kb = k_begin; kb < k_end; kb += 32) {
    // K: MFMA row i of key block b holds key kb + 8*(i/4) + 4*b + i%4
    bf16x8_t kf[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int key = kb + 8 * (lr >> 2) + 4 * b + (lr & 3);
      if (key < k_end) {
        const uint16_t* base = kp + (size_t)pt[key >> 4] * page_elems + (size_t)(kvh * 16 + (key & 15)) * HD + g * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[b][ks] = as_bf16x8(ld16(base + ks * 32));
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[b][ks] = as_bf16x8(zero);
      }
    }
    // V^T: row d = dblk*16 + lr, keys kb + 8g .. kb + 8g + 7 (zero beyond k_end)
    bf16x8_t vf[8];
    {
      const int key0 = kb + 8 * g;
      if (key0 < k_end) {
        const uint16_t* base = vp + (size_t)pt[key0 >> 4] * page_elems + (size_t)kvh * HD * 16 + (key0 & 15);
        const int nvalid = k_end - key0;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          u32x4_t raw = ld16(base + (size_t)(d * 16 + lr) * 16);
          if (nvalid < 8) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int j0 = 2 * w;
              uint32_t m = 0u;
              if (j0 < nvalid) m |= 0x0000ffffu;
              if (j0 + 1 < nvalid) m |= 0xffff0000u;
              raw[w] &= m;
            }
          }
          vf[d] = as_bf16x8(raw);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 8; ++d) vf[d] = as_bf16x8(zero);
      }
    }

    bf16x8_t pf[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      f32x4_t s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma16x16x32(kf[b][ks], qf[c][ks], acc);
        s[b] = acc;
      }
      float sv[8];
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 8 * g + 4 * b + r;
          const bool vis = qvalid[c] && key < k_end && key <= qpos[c];
          const float v = vis ? s[b][r] * scale : kNegInf;
          sv[4 * b + r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[c], mx);
      float alpha = 1.f;
      uint16_t pb[8];
      float ps = 0.f;
      if (m_new == kNegInf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = 0;
      } else {
        alpha = exp2f(m_run[c] - m_new);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bf16 pbv = from_f<bf16>(exp2f(sv[j] - m_new));
          pb[j] = pbv.u;
          ps += to_f(pbv);
        }
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_run[c] = l_run[c] * alpha + ps;
      m_run[c] = m_new;
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d][c] *= alpha;
      u32x4_t pk;
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[w] = (uint32_t)pb[2 * w] | ((uint32_t)pb[2 * w + 1] << 16);
      pf[c] = as_bf16x8(pk);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int c = 0; c < NCB; ++c) o[d][c] = mfma16x16x32(vf[d], pf[c], o[d][c]);
  }

#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    if (!qvalid[c]) continue;
    const int qr = c * 16 + lr, p = qr / G, h = qr % G;
    const int row = it.row0 + p, head = kvh * G + h;
    if (a.split) {
      float* po = a.part_o + ((size_t)(split * a.part_rows + row) * a.Hq + head) * HD;
#pragma unroll
      for (int d = 0; d < 8; ++d) *(f32x4_t*)(po + d * 16 + 4 * g) = o[d][c];
      if (g == 0) {
        float* pml = a.part_ml + ((size_t)(split * a.part_rows + row) * a.Hq + head) * 2;
        pml[0] = m_run[c];
        pml[1] = l_run[c];
      }
    } else {
      const float inv = l_run[c] > 0.f ? 1.f / l_run[c] : 0.f;
      uint16_t* out = (uint16_t*)a.out + (size_t)row * q_stride + (size_t)head * HD;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint32_t lo = (uint32_t)from_f<bf16>(o[d][c][0] * inv).u | ((uint32_t)from_f<bf16>(o[d][c][1] * inv).u << 16);
        uint32_t hi = (uint32_t)from_f<bf16>(o[d][c][2] * inv).u | ((uint32_t)from_f<bf16>(o[d][c][3] * inv).u << 16);
        *(uint2*)(out + d * 16 + 4 * g) = make_uint2(lo, hi);
      }
    }
  }
}

// Combine the split partials of each row in ascending split order (row at position p uses
// splits 0 .. ceil((p+1)/split)-1).  Dead rows (position -1) are written as zeros.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int row = blockIdx.x;
  const int pos = a.row_pos[row];
  uint16_t* out = (uint16_t*)a.out + (size_t)row * a.Hq * HD;
  const int per_head = HD / 16;                    // threads per head (16 dims each)
  for (int t = threadIdx.x; t < a.Hq * per_head; t += blockDim.x) {
    const int head = t / per_head, d0 = (t % per_head) * 16;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (pos >= 0) {
      const int ns = (pos + 1 + a.split - 1) / a.split;
      float M = kNegInf;
      for (int s = 0; s < ns; ++s)
        M = fmaxf(M, a.part_ml[((size_t)(s * a.part_rows + row) * a.Hq + head) * 2]);
      float L = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float* ml = a.part_ml + ((size_t)(s * a.part_rows + row) * a.Hq + head) * 2;
        const float w = (ml[0] == kNegInf) ? 0.f : exp2f(ml[0] - M);
        L += w * ml[1];
        const float* po = a.part_o + ((size_t)(s * a.part_rows + row) * a.Hq + head) * HD + d0;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const f32x4_t v = *(const f32x4_t*)(po + i);
          acc[i] += w * v[0];
          acc[i + 1] += w * v[1];
          acc[i + 2] += w * v[2];
          acc[i + 3] += w * v[3];
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= inv;
    }
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pk[i] = (uint32_t)from_f<bf16>(acc[2 * i]).u | ((uint32_t)from_f<bf16>(acc[2 * i + 1]).u << 16);
    uint4* dst = (uint4*)(out + (size_t)head * HD + d0);
    dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
  }
}

// fp32 path: one wave per (row, query head); keys 0 .. pos streamed from the pages with a
// wave-reduced dot product and an online softmax.
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int row = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
  const int hd = a.hd, P = a.P, G = a.Hq / a.Hkv, kvh = head / G;
  float* out = (float*)a.out + (size_t)row * a.Hq * hd + (size_t)head * hd;
  const int pos = a.row_pos[row];
  if (pos < 0) {
    for (int d = lane; d < hd; d += 64) out[d] = 0.f;
    return;
  }
  const int slot = a.row_slot[row];
  const float* qv = (const float*)a.q + (size_t)row * a.Hq * hd + (size_t)head * hd;
  const float* kp = (const float*)a.k_pool;
  const float* vp = (const float*)a.v_pool;
  const int32_t* pt = a.page_table + (size_t)slot * a.max_pages;
  float qr[4], o[4];
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    qr[i] = d < hd ? qv[d] : 0.f;
    o[i] = 0.f;
  }
  const float scale = 1.0f / sqrtf((float)hd);
  float m = kNegInf, l = 0.f;
  for (int j = 0; j <= pos; ++j) {
    const int page = pt[j / P], tok = j % P;
    const float* kr = kp + ((size_t)page * a.Hkv + kvh) * P * hd + (size_t)tok * hd;
    float dot = 0.f;
    for (int i = 0; i < 4; ++i) {
      const int d = lane + 64 * i;
      if (d < hd) dot += qr[i] * kr[d];
    }
    const float s = wave_sum(dot) * scale;
    const float m_new = fmaxf(m, s);
    const float al = expf(m - m_new), p = expf(s - m_new);
    l = l * al + p;
    const float* vr = vp + ((size_t)page * a.Hkv + kvh) * hd * P + tok;
    for (int i = 0; i < 4; ++i) {
      const int d = lane + 64 * i;
      if (d < hd) o[i] = o[i] * al + p * vr[(size_t)d * P];
    }
    m = m_new;
  }
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d < hd) out[d] = o[i] / l;
  }
}

// Items and row metadata of the kernel-level attention entry: sequence b has q_len[b] rows
// at positions ctx_len[b] - q_len[b] .. ctx_len[b] - 1 in rows b*R ...
__global__ void attn_setup_kernel(AttnItem* items, int32_t* row_pos, int32_t* row_slot, const int32_t* ctx_len,
                                  const int32_t* q_len, int batch, int R) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  const int nq = max(0, min(R, q_len[b]));
  const int pos0 = ctx_len[b] - nq;
  AttnItem it;
  it.slot = b;
  it.row0 = b * R;
  it.nq = pos0 >= 0 ? nq : 0;
  it.pos0 = pos0;
  items[b] = it;
  for (int i = 0; i < R; ++i) {
    row_pos[b * R + i] = (i < it.nq) ? pos0 + i : -1;
    row_slot[b * R + i] = b;
  }
}

}  // namespace

hipError_t launch_attn_setup(AttnItem* items, int32_t* row_pos, int32_t* row_slot, const int32_t* ctx_len,
                             const int32_t* q_len, int batch, int rows, hipStream_t s) {
  hipLaunchKernelGGL(attn_setup_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, items, row_pos, row_slot, ctx_len,
                     q_len, batch, rows);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.hd != HD || a.P != 16) return hipErrorInvalidValue;
  if (a.n_items <= 0) return hipSuccess;
  dim3 grid(a.n_items, a.Hkv, a.split ? a.max_splits : 1);
  if (a.ncb == 2) {
    hipLaunchKernelGGL(attn_bf16_kernel<2>, grid, dim3(64), 0, s, a);
  } else if (a.ncb == 4) {
    hipLaunchKernelGGL(attn_bf16_kernel<4>, grid, dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.hd > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_rows, a.Hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace isd
