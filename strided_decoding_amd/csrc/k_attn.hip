// Paged causal attention for blocks of query rows (decode: 2N-1 rows per slot; prefill: tiles
// of consecutive prompt positions).  Keys and values are read only from the KV pages, the
// block's own K/V having been appended first, and a row at position p sees keys 0 .. p.
//
// bf16 path (head_dim 128): one workgroup of NCB waves per (item, KV head, context split);
// wave w owns 16 of the up to 16 NCB query columns of the KV-head group (positions x G query
// heads), which are the columns of two MFMA products
//   S^T = K Q^T          (A = 16 keys x 32 dims per step, B = Q^T)
//   O^T += V^T P^T       (A = V^T rows = dims, k = 32 keys; B = P^T)
// K pages are [token][dim] and V pages [dim][token] (transposed within a page), so both
// operands are 16-byte row chunks.  The workgroup streams its 32-key blocks (two 16-token
// pages of K and of V, 16 KB) through an NBUF-block LDS ring shared by its waves (each wave
// issues 16/NCB of a block's 16 direct global->LDS loads, one barrier per block), NBUF-1 blocks
// in flight under explicit vmcnt waits while one is multiplied; every load instruction reads
// 1 KB of one page contiguously, and the chunks are XOR-swizzled in LDS so the operand reads
// are free of bank conflicts.  The key order inside a block is permuted so
// that the S^T accumulator registers of a lane are exactly the P^T operand slots of the next
// product (no cross-lane traffic).  Online softmax in the log2 domain with wave reductions
// over the 4 lane groups sharing a column.  Context splits begin at multiples of the split
// length and blocks at absolute positions, and masked keys contribute exact zeros, so a
// row's result does not depend on the other rows of its pass.  With splits, each split
// writes fp32 partials (output, reference maximum, sum) and attn_combine_kernel merges them
// in split order.  (A workgroup's global-memory handoff to another workgroup would need a
// device-scope fence, which writes back the XCD's L2: a kernel boundary is cheaper.)
#include <algorithm>

#include "isd_common.h"

namespace isd {
namespace {

constexpr int HD = 128;
constexpr int kBlockBytes = 16384;         // one 32-key block: K and V, two pages each
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescale = 8.f;            // log2 headroom of the softmax reference maximum
#ifndef ISD_ATTN_NBUF
#define ISD_ATTN_NBUF 2
#endif
constexpr int kAttnBufs = ISD_ATTN_NBUF;

ISD_DEV u32x4_t ld16(const uint16_t* p) { return *(const u32x4_t*)p; }

// The maximum (sum) of x over lanes l and l ^ 16, and over l and l ^ 32: a register swapped with
// itself by gfx950's lane-swap instructions (rows of 16 lanes, halves of 32) leaves each lane
// holding its own value in one result and its partner's in the other (which is which depends on
// the lane; max and + are symmetric).  No LDS round trip, unlike a generic lane shuffle.
ISD_DEV float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
ISD_DEV float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
ISD_DEV float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
ISD_DEV float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
ISD_DEV u32x4_t lds16(const uint8_t* p) { return *(const u32x4_t*)p; }

// One workgroup per (item, KV head, context split); wave w handles the 16 query columns
// 16 w .. 16 w + 15 of the KV-head group and 16/NCB of the 16 loads of each KV block.
template <int NCB, int NBUF>
__global__ __launch_bounds__(64 * NCB) void attn_bf16_kernel(AttnArgs a) {
  constexpr int PW = 16 / NCB;                       // KV loads per block issued by each wave
  static_assert(NBUF >= 2 && NBUF <= 4 && (NBUF - 1) * PW + 4 < 64, "vmcnt counts at most 63 loads");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF * kBlockBytes];
  const AttnItem it = a.items[blockIdx.x];
  const int kvh = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  const size_t q_stride = (size_t)a.Hq * HD;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  if (it.nq <= 0) return;
  // Page ids of the key range, lane l holding logical pages win + l and win + 64 + l (a window
  // of 128 pages, 2048 keys: a whole context split; longer ranges reload it), read out with
  // readlane: no memory access inside the KV pipeline besides its own loads.  The first window
  // is loaded together with the context length (clamped to the table row, not to the context:
  // entries past the context are never read out).
  const int32_t* pt = a.page_table + (size_t)it.slot * a.max_pages;
  int win = a.split ? (split * a.split) >> 4 : 0;
  int pid0 = pt[min(win + lane, a.max_pages - 1)];
  int pid1 = pt[min(win + 64 + lane, a.max_pages - 1)];
  const int ctx = a.ctx_len[it.slot];
  const int key_hi = min(ctx, it.pos0 + it.nq);
  int k_begin = 0, k_end = key_hi;
  if (a.split) {
    k_begin = split * a.split;
    if (k_begin >= key_hi) return;
    k_end = min(key_hi, k_begin + a.split);
  }
  const float scale = 1.4426950408889634f * rsqrtf((float)HD);

  // Q^T operand of this wave: lane (lr, g) holds query column 16 w + lr (position (16 w + lr)/G,
  // head (16 w + lr) % G), dims 32 ks + 8 g .. +7, loaded by direct global->LDS loads into
  // the last ring slot ahead of the first KV blocks (lane l reads back its own 16 bytes).
  const int qcol = wave * 16 + lr, qp = qcol / G, qh = qcol % G;
  const bool qvalid = qp < it.nq;
  const int qpos = it.pos0 + qp;
  const uint16_t* qsrc =
      (const uint16_t*)a.q + (size_t)(it.row0 + (qvalid ? qp : 0)) * q_stride + (size_t)(kvh * G + qh) * HD + g * 8;

  const int last_page = (k_end - 1) >> 4;
  // this wave's Q goes out now (4 direct loads into the last ring slot), the page ids are
  // waited for with only those loads left in flight
  {
    uint8_t* qs = ring + (NBUF - 1) * kBlockBytes + wave * 4096;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      __builtin_amdgcn_global_load_lds((const void*)(qsrc + ks * 32), (lds_void*)(qs + ks * 1024), 16, 0, 0);
  }
  wait_vmcnt<4>();
  auto page_of = [&](int pg) -> int {
    if (pg >= win + 128) {
      wait_vmcnt<0>();
      win = pg;
      pid0 = pt[min(win + lane, last_page)];
      pid1 = pt[min(win + 64 + lane, last_page)];
      wait_vmcnt<0>();
    }
    const int o = pg - win;
    return o < 64 ? __builtin_amdgcn_readlane(pid0, o) : __builtin_amdgcn_readlane(pid1, o - 64);
  };
  const size_t page_elems = (size_t)a.Hkv * 16 * HD;
  const uint16_t* kbase = (const uint16_t*)a.k_pool + (size_t)kvh * 16 * HD;
  const uint16_t* vbase = (const uint16_t*)a.v_pool + (size_t)kvh * HD * 16;

  // Block blk (keys k_begin + 32 blk ..) -> ring slot blk % NBUF: K at +0 (token t: 256 bytes at
  // t * 256, dim chunk c in 16-byte slot c ^ h(t), h(t) = (t & 3) | ((t >> 1) & 12)); V at
  // +8192 (page j at + 4096 j, dim row d: 32 bytes at d * 32, key half e in slot e ^ (d/8 % 2)).
  // Load i < 8 of a block: K tokens 4i .. 4i+3; load 8 + i: V of page i/4, dims 32 (i%4) .. +31.
  auto issue = [&](int blk) {
    const int kb = k_begin + 32 * blk;
    uint8_t* st = ring + (blk % NBUF) * kBlockBytes;
    const int pg0 = page_of(kb >> 4);
    const int pg1 = kb + 16 < k_end ? page_of((kb >> 4) + 1) : pg0;   // past the context: any valid page
#pragma unroll
    for (int jj = 0; jj < PW; ++jj) {
      const int j = wave * PW + jj;
      const uint16_t* src;
      if (j < 8) {
        const int t = 4 * j + (lane >> 4);
        const int c = (lane & 15) ^ ((t & 3) | ((t >> 1) & 12));
        src = kbase + (size_t)(j < 4 ? pg0 : pg1) * page_elems + (size_t)(t & 15) * HD + c * 8;
      } else {
        const int i = j - 8;
        const int dim = 32 * (i & 3) + (lane >> 1);
        const int e = (lane & 1) ^ ((dim >> 3) & 1);
        src = vbase + (size_t)(i < 4 ? pg0 : pg1) * page_elems + (size_t)dim * 16 + e * 8;
      }
      // non-temporal: every K/V byte is read once per pass, so it should not displace cached
      // lines (measured 88.6 -> 80.4 us per launch at 64 slots, contexts ~2000)
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(st + j * 1024), 16, 0, kCachePolicyNT);
    }
  };

  bf16x8_t qf[4];
  float m_run = kNegInf, l_run = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) o[d] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  // One 32-key block.  Softmax in the log2 domain against a per-column reference maximum m
  // that is raised only when a block's maximum exceeds it by more than kRescale (so p <= 2^8
  // and the accumulators are rescaled rarely); the sum l and the output use the same m, so
  // the result is exact up to rounding.  Blocks whose keys are all visible to every row
  // (below the first query position and inside the range) skip all masking.
  auto compute = [&](int blk) {
    const int kb = k_begin + 32 * blk;
    const uint8_t* st = ring + (blk % NBUF) * kBlockBytes;
    const bool tail = kb + 32 > k_end;               // keys past the range in this block
    const bool clean = !tail && kb + 31 <= it.pos0;  // no causal or range mask
    // K: MFMA row i of key block b holds key kb + 8*(i/4) + 4*b + i%4, whose swizzle h is i
    f32x4_t s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int t = 8 * (lr >> 2) + 4 * b + (lr & 3);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16x16x32(as_bf16x8(lds16(st + t * 256 + (((4 * ks + g) ^ lr) * 16))), qf[ks], acc);
      s[b] = acc;
    }
    // V^T: row d = dblk*16 + lr, keys kb + 8g .. kb + 8g + 7 (zero past the range)
    bf16x8_t vf[8];
    {
      const uint8_t* vrow = st + 8192 + (g >> 1) * 4096 + lr * 32 + (((g & 1) ^ ((lr >> 3) & 1)) * 16);
      const int nvalid = k_end - (kb + 8 * g);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        u32x4_t raw = lds16(vrow + d * 16 * 32);
        if (tail) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t m = 0u;
            if (2 * w < nvalid) m |= 0x0000ffffu;
            if (2 * w + 1 < nvalid) m |= 0xffff0000u;
            raw[w] &= m;
          }
        }
        vf[d] = as_bf16x8(raw);
      }
    }
    float sv[8];
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[b][r] * scale;
        if (!clean) {
          const int key = kb + 8 * g + 4 * b + r;
          if (!(key < k_end && key <= qpos)) v = kNegInf;
        }
        sv[4 * b + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_xor32(max_xor16(mx));
    const bool raise = mx > m_run + kRescale;      // also the first visible key of the column
    const float m_new = raise ? mx : m_run;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    uint32_t pk[4];
    float ps = 0.f;
    if (m_new == kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[w] = 0u;
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pk[w] = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2 * w] - m_new), __builtin_amdgcn_exp2f(sv[2 * w + 1] - m_new));
        ps += __uint_as_float(pk[w] << 16) + __uint_as_float(pk[w] & 0xffff0000u);
      }
    }
    ps = sum_xor32(sum_xor16(ps));
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (__any(raise)) {
#pragma unroll
      for (int d = 0; d < 8; ++d) o[d] *= alpha;
    }
    const bf16x8_t pf = as_bf16x8((u32x4_t){pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = mfma16x16x32(vf[d], pf, o[d]);
  };

  // Pipeline: block blk is issued NBUF-1 blocks ahead into ring slot blk % NBUF.  Each wave
  // waits for its own loads of block blk, then one barrier makes the whole block visible and
  // also tells that every wave is done with block blk-1, whose slot is refilled next.
  const int nblk = (k_end - k_begin + 31) >> 5;
  const int pro = min(NBUF - 1, nblk);
  for (int blk = 0; blk < pro; ++blk) issue(blk);
  if (pro >= 3) wait_vmcnt<3 * PW>();                // this wave's Q has landed
  else if (pro == 2) wait_vmcnt<2 * PW>();
  else if (pro == 1) wait_vmcnt<PW>();
  else wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4_t v = lds16(ring + (NBUF - 1) * kBlockBytes + wave * 4096 + ks * 1024 + 16 * lane);
    qf[ks] = as_bf16x8(qvalid ? v : zero);
  }
  wait_lgkm0();                                      // Q is in registers before its slot is refilled
  for (int blk = 0; blk < nblk; ++blk) {
    const int later = min(NBUF - 2, nblk - 1 - blk);  // blocks issued after blk
    if (later >= 2) wait_vmcnt<2 * PW>();
    else if (later == 1) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (blk + NBUF - 1 < nblk) issue(blk + NBUF - 1);
    compute(blk);
    __builtin_amdgcn_sched_barrier(0);
  }

  // A row that only the first split covers (position below the split length) is final here:
  // it is written directly (the one-split merge would multiply by exp2(0) = 1) and the combine
  // kernel skips it.
  const bool final_here = !a.split || (split == 0 && qpos < a.split);
  if (final_here) {
    if (qvalid) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      uint16_t* out = (uint16_t*)a.out + (size_t)(it.row0 + qp) * q_stride + (size_t)(kvh * G + qh) * HD;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *(uint2*)(out + d * 16 + 4 * g) =
            make_uint2(pack_bf16x2(o[d][0] * inv, o[d][1] * inv), pack_bf16x2(o[d][2] * inv, o[d][3] * inv));
    }
  } else if (qvalid) {
    const int row = it.row0 + qp, head = kvh * G + qh;
    float* po = a.part_o + ((size_t)(split * a.part_rows + row) * a.Hq + head) * HD;
#pragma unroll
    for (int d = 0; d < 8; ++d) *(f32x4_t*)(po + d * 16 + 4 * g) = o[d];
    if (g == 0) *(float2*)(a.part_ml + ((size_t)(split * a.part_rows + row) * a.Hq + head) * 2) = make_float2(m_run, l_run);
  }
}

// Merge the split partials of each row in ascending split order (the row at position p uses
// splits 0 .. ceil((p+1)/split)-1; rows with p < split were written by the attention kernel);
// dead rows (position -1) are written as zeros.  Workgroup (row, y), thread x handles item
// t = 256 y + x of the row: dims 4 (t % 32) .. +3 of head t / 32.  Every split's (m, l) and
// output slice is loaded before the first use, in groups of G splits (G = 4, 8 or 16, the
// smallest that holds the row's splits, at most 16; a group's slots past the row's last split
// re-read it and are left out), so a row with up to 16 splits costs one memory round trip.
// The weights and sums follow the split order: M = max of the maxima, w_s = exp2(m_s - M)
// (zero for a split with no visible key), O = sum_s w_s O_s / sum_s w_s l_s.
constexpr int kMergeThreads = 256;
template <int G>
ISD_DEV f32x4_t merge_splits(const AttnArgs& a, size_t e0, size_t stride, int ns, int d4, float& inv) {
  float2 ml[G];
  f32x4_t po[G];
  auto load_group = [&](int s0, bool with_o) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const size_t e = e0 + (size_t)min(s0 + i, ns - 1) * stride;
      ml[i] = *(const float2*)(a.part_ml + e * 2);
      if (with_o) po[i] = *(const f32x4_t*)(a.part_o + e * HD + 4 * d4);
    }
  };
  float M = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += G) {
    load_group(s0, ns <= G);   // a single group: the outputs come with the maxima
#pragma unroll
    for (int i = 0; i < G; ++i) M = fmaxf(M, ml[i].x);   // repeats of the last split: same maximum
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int s0 = 0; s0 < ns; s0 += G) {
    if (ns > G) load_group(s0, true);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool in = s0 + i < ns;
      const float w = (ml[i].x == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ml[i].x - M);
      const float nl = L + w * ml[i].y;
      const f32x4_t na = acc + w * po[i];
      L = in ? nl : L;
      acc = in ? na : acc;
    }
  }
  inv = L > 0.f ? 1.f / L : 0.f;
  return acc;
}

__global__ __launch_bounds__(kMergeThreads) void attn_combine_kernel(AttnArgs a) {
  const int row = blockIdx.x;
  const int pos = a.row_pos[row];
  if (pos >= 0 && pos < a.split) return;                     // written by the attention kernel
  const int t = blockIdx.y * kMergeThreads + threadIdx.x;
  if (t >= a.Hq * (HD / 4)) return;
  const int head = t / (HD / 4), d4 = t % (HD / 4);
  const size_t stride = (size_t)a.part_rows * a.Hq;          // between splits
  const size_t e0 = (size_t)row * a.Hq + head;
  const int ns = pos >= 0 ? pos / a.split + 1 : 0;           // the same for the whole workgroup
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float inv = 0.f;
  if (ns > 8) acc = merge_splits<16>(a, e0, stride, ns, d4, inv);
  else if (ns > 4) acc = merge_splits<8>(a, e0, stride, ns, d4, inv);
  else if (ns > 0) acc = merge_splits<4>(a, e0, stride, ns, d4, inv);
  uint2* out = (uint2*)((uint16_t*)a.out + (size_t)row * a.Hq * HD + (size_t)head * HD + 4 * d4);
  *out = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
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

#ifndef ISD_ATTN_ITEMS
#define ISD_ATTN_ITEMS 2048
#endif
int attn_split_len(int batch, int n_kv_heads, int max_ctx) {
  // With at least two (slot, KV head) pairs per CU the pairs alone fill the chip: the longest
  // split, so that most rows are final in their first split and skip the merge (measured: the
  // 64-slot pass is 1.2 % faster than with 1024-key splits; 16 slots need the short splits).
  // Contexts a little past 2048 keys take one 2560-key split, so that no row needs the merge
  // (the pass then launches no combine kernel).
  if ((long long)batch * n_kv_heads >= 512) return max_ctx > 2048 && max_ctx <= 2560 ? 2560 : 2048;
  // else about kAttnItems (slot, KV head, split) workgroups at the longest context, 128 .. 2048
  // keys each
  constexpr long long kAttnItems = ISD_ATTN_ITEMS;
  const long long want = ((long long)max_ctx * batch * n_kv_heads + kAttnItems - 1) / kAttnItems;
  int split = 128;
  while (split < 2048 && split < want) split *= 2;
  return split;
}

hipError_t launch_attn_setup(AttnItem* items, int32_t* row_pos, int32_t* row_slot, const int32_t* ctx_len,
                             const int32_t* q_len, int batch, int rows, hipStream_t s) {
  hipLaunchKernelGGL(attn_setup_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, items, row_pos, row_slot, ctx_len,
                     q_len, batch, rows);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.hd != HD || a.P != 16) return hipErrorInvalidValue;
  if (a.n_items <= 0) return hipSuccess;
  if (a.split && a.split % 32) return hipErrorInvalidValue;
  dim3 grid(a.n_items, a.Hkv, a.split ? a.max_splits : 1);
  if (a.ncb == 2) {
    hipLaunchKernelGGL((attn_bf16_kernel<2, kAttnBufs>), grid, dim3(128), 0, s, a);
  } else if (a.ncb == 4) {
    hipLaunchKernelGGL((attn_bf16_kernel<4, kAttnBufs>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int per_row = (a.Hq * (HD / 4) + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.n_rows, per_row), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.hd > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_f32_kernel, dim3(a.n_rows, a.Hq), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace isd
