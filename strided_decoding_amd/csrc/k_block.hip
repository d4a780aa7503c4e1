// Block assembly, KV page reserve / append / truncate, and the elementwise glue of a pass
// (embedding gather, RMSNorm, RoPE).
//
// Block layout per slot (R = 2N-1 row slots, L cached tokens, c newest committed token):
//   state A: [c, v_1 .. v_{N-1}, MASK x (N-1)] at positions L .. L+2N-2
//   state B: [c, MASK x (N-1)]                 at positions L .. L+N-1
// Pages: a LIFO free stack (top = n_free-1).  A pass first reserves, slot by slot in
// ascending order, the pages positions L .. L+q_len-1 need; after the decisions every slot,
// in ascending order, frees the pages beyond ceil(L'/P), ascending logical order.  Both
// orders come from block-wide prefix sums, so the page tables are a deterministic function
// of the slot states.
#include <algorithm>
#include <type_traits>

#include "isd_common.h"

namespace isd {
namespace {

// Exclusive prefix sum over a 256-thread block; *total receives the block sum.
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int t = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void assemble_kernel(StepMeta m) {
  __shared__ int sh[256];
  __shared__ int s_nfree;
  const int tid = threadIdx.x;
  if (tid == 0) s_nfree = *m.n_free;
  __syncthreads();
  const int N = m.N, R = 2 * N - 1, P = m.P;
  int popped = 0, rows_base = 0;
  for (int g0 = 0; g0 < m.max_batch; g0 += 256) {
    const int b = g0 + tid;
    // slots at or past n_active sit this pass out; a live one there is an error of the caller
    if (b >= m.n_active && b < m.max_batch) {
      isd_slot* so = &m.slots[b];
      if (so->state == ISD_SLOT_A || so->state == ISD_SLOT_B) so->status = ISD_E_STATE;
    }
    const bool valid = b < m.n_active;
    isd_slot* st = valid ? &m.slots[b] : nullptr;
    int state = valid ? st->state : ISD_SLOT_EMPTY;
    const int L = valid ? st->L : 0;
    int q_len = state == ISD_SLOT_A ? R : (state == ISD_SLOT_B ? N : 0);
    const int have = valid ? st->n_pages : 0;
    int need = 0;
    if (q_len > 0) need = max(0, (L + q_len + P - 1) / P - have);
    int total;
    const int off = block_excl_scan(need, sh, &total);
    // A slot whose pages do not all fit on the stack after the slots before it (host admission
    // makes this unreachable; this is the device's own guard) takes none, is flagged
    // ISD_E_CAPACITY and finishes: no rows, no cache writes, its pages freed by truncate.
    // Slots are served in order, so the pages taken are one contiguous run from the top.
    const bool fits = popped + off + need <= s_nfree;
    const int grant = fits ? need : 0;
    int granted;
    block_excl_scan(grant, sh, &granted);
    if (valid && !fits) {
      st->status = ISD_E_CAPACITY;
      st->state = ISD_SLOT_DONE;
      state = ISD_SLOT_DONE;
      q_len = 0;
    }
    // packed rows: the slots' blocks back to back in slot order
    int n_rows;
    const int roff = rows_base + block_excl_scan(q_len, sh, &n_rows);
    if (b < m.max_batch) {
      m.row_off[b] = roff;
      m.row_len[b] = q_len;
    }
    if (valid) {
      int32_t* pt = m.page_table + (size_t)b * m.max_pages;
      for (int k = 0; k < grant; ++k) pt[have + k] = m.free_stack[s_nfree - 1 - (popped + off + k)];
      st->n_pages = have + grant;
      for (int i = 0; i < q_len; ++i) {
        const int r = roff + i;
        int tok = m.mask_id;
        if (i == 0) tok = st->c;
        else if (state == ISD_SLOT_A && i < N) tok = st->pending[i - 1];
        m.row_tok[r] = tok;
        m.row_pos[r] = L + i;
        m.row_slot[r] = b;
        m.delta_row[r] = -1;
      }
      for (int j = 0; j < N - 1; ++j) {
        int r = -1;
        if (state == ISD_SLOT_A) r = roff + N + j;
        else if (state == ISD_SLOT_B) r = roff + 1 + j;
        m.mask_rows[b * (N - 1) + j] = r;
        if (r >= 0) m.delta_row[r] = b * (N - 1) + j;
      }
      for (int k = 0; k < m.items_per_slot; ++k) {
        AttnItem it;
        it.slot = b;
        it.row0 = roff + k * m.q_max;
        it.nq = max(0, min(m.q_max, q_len - k * m.q_max));
        it.pos0 = L + k * m.q_max;
        m.items[b * m.items_per_slot + k] = it;
      }
      m.ctx_len[b] = L + q_len;
    }
    popped += granted;
    rows_base += n_rows;
  }
  // the rows past the live ones (up to the pass's n_active R) are dead: MASK token, no position
  for (int r = rows_base + tid; r < m.n_active * R; r += 256) {
    m.row_tok[r] = m.mask_id;
    m.row_pos[r] = -1;
    m.row_slot[r] = 0;
    m.delta_row[r] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    *m.n_free = s_nfree - popped;
    *m.m_live = rows_base;
  }
}

// Free the pages beyond ceil(L/P) (all pages of a finished or empty slot), slots taken in
// the given order (NULL = ascending), pushing in ascending logical page order.
__global__ __launch_bounds__(256) void truncate_kernel(StepMeta m, const int32_t* order, int n) {
  __shared__ int sh[256];
  __shared__ int s_nfree;
  __shared__ int s_bad;           // first slot (in processing order) with a non-zero status
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_nfree = *m.n_free;
    s_bad = INT_MAX;
  }
  __syncthreads();
  int pushed = 0;
  for (int g0 = 0; g0 < n; g0 += 256) {
    const int i = g0 + tid;
    const bool valid = i < n;
    const int b = valid ? (order ? order[i] : i) : 0;
    int frees = 0, keep = 0, have = 0;
    if (valid) {
      const isd_slot& st = m.slots[b];
      have = st.n_pages;
      keep = (st.state == ISD_SLOT_A || st.state == ISD_SLOT_B) ? (st.L + m.P - 1) / m.P : 0;
      frees = max(0, have - keep);
      if (st.status != 0) atomicMin(&s_bad, i);
    }
    int total;
    const int off = block_excl_scan(frees, sh, &total);
    if (valid && frees > 0) {
      int32_t* pt = m.page_table + (size_t)b * m.max_pages;
      for (int k = 0; k < frees; ++k) {
        m.free_stack[s_nfree + pushed + off + k] = pt[keep + k];
        pt[keep + k] = -1;
      }
      m.slots[b].n_pages = keep;
    }
    pushed += total;
  }
  __syncthreads();
  if (tid == 0) {
    *m.n_free = s_nfree + pushed;
    // the context's sticky status: the first slot status ever reported, kept in a pinned
    // host word so that the host reads it without a synchronization
    if (m.sticky_host && s_bad != INT_MAX) {
      volatile int32_t* h = m.sticky_host;
      if (*h == 0) *h = m.slots[order ? order[s_bad] : s_bad].status;
    }
  }
}

// Prefill set-up: slot by slot in call order, free the slot's old pages and take the
// prompt's pages; reset the slot; write row metadata and the attention items.
__global__ __launch_bounds__(256) void prefill_setup_kernel(StepMeta m, PrefillCall c, const int32_t* prompt_ids,
                                                            int q_tile, int32_t* order_out) {
  __shared__ int s_nfree;
  const int tid = threadIdx.x;
  if (tid == 0) s_nfree = *m.n_free;
  __syncthreads();
  for (int i = 0; i < c.n; ++i) {
    const int b = c.slot[i];
    const int len = c.off[i + 1] - c.off[i];
    isd_slot* st = &m.slots[b];
    int32_t* pt = m.page_table + (size_t)b * m.max_pages;
    const int old = st->n_pages;
    for (int k = tid; k < old; k += 256) m.free_stack[s_nfree + k] = pt[k];
    __syncthreads();
    if (tid == 0) s_nfree += old;
    __syncthreads();
    // a prompt whose pages are not all on the stack (host admission makes this unreachable)
    // takes none and finishes at once with ISD_E_CAPACITY: dead rows, empty attention items
    const int need = (len + m.P - 1) / m.P;
    const bool ok = need <= s_nfree;
    const int np = ok ? need : 0;
    for (int k = tid; k < np; k += 256) pt[k] = m.free_stack[s_nfree - 1 - k];
    for (int k = np + tid; k < m.max_pages; k += 256) pt[k] = -1;
    __syncthreads();
    if (tid == 0) {
      s_nfree -= np;
      st->state = ok ? ISD_SLOT_B : ISD_SLOT_DONE;
      st->L = len;
      st->c = 0;
      st->t = 0;
      st->n_gen = 0;
      st->max_new = c.max_new[i];
      st->n_pages = np;
      st->status = ok ? 0 : ISD_E_CAPACITY;
      for (int j = 0; j < ISD_MAX_STRIDE - 1; ++j) {
        st->pending[j] = -1;
        st->q_row[j] = -1;
      }
      st->passes = st->accepted = st->verified = st->committed = 0;
      st->meter_sum = 0.0;
      st->meter_n = 0;
      m.ctx_len[b] = len;
      m.last_rows[i] = c.off[i + 1] - 1;
      order_out[i] = b;
    }
    for (int r = c.off[i] + tid; r < c.off[i + 1]; r += 256) {
      m.row_tok[r] = prompt_ids[r];
      m.row_pos[r] = ok ? r - c.off[i] : -1;
      m.row_slot[r] = b;
      m.delta_row[r] = -1;
    }
    const int nit = (len + q_tile - 1) / q_tile;
    for (int k = tid; k < nit; k += 256) {
      AttnItem it;
      it.slot = b;
      it.row0 = c.off[i] + k * q_tile;
      it.nq = ok ? min(q_tile, len - k * q_tile) : 0;
      it.pos0 = k * q_tile;
      m.items[c.item_off[i] + k] = it;
    }
    __syncthreads();
  }
  if (tid == 0) *m.n_free = s_nfree;
}

// Token ids outside [0, vocab] (vocab = MASK) read the MASK row.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tok, const T* table, float* X, int d, int mask_id) {
  const int r = blockIdx.x;
  int id = tok[r];
  if (id < 0 || id > mask_id) id = mask_id;
  const T* src = table + (size_t)id * d;
  float* dst = X + (size_t)r * d;
  for (int i = threadIdx.x; i < d; i += 256) dst[i] = to_f(src[i]);
}

// y = g * x / sqrt(mean(x^2) + eps), one block of 1024 threads per row, fixed-order
// reduction: thread t owns the 4-column groups t + 1024 k (d is a multiple of 4), squares
// accumulated group by group, then a fixed tree (the same order the fused GEMM epilogue uses).
template <typename T>
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* X, const T* g, T* Y, int d, float eps) {
  __shared__ float sh[16];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* x = X + (size_t)r * d;
  // this thread's weights of the first 4096 columns, loaded ahead of the reduction (loaded
  // after it, each would wait behind the stores of the previous ones)
  float g0[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) g0[j] = to_f(g[min(4 * tid + j, d - 1)]);
  float ss = 0.f;
  for (int c = 4 * tid; c < d; c += 4096) {
    const f32x4_t v = *(const f32x4_t*)(x + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fmaf(v[j], v[j], ss);
  }
  const float tot = block_sum_1024(ss, sh);
  const float denom = sqrtf(tot / (float)d + eps);
  T* y = Y + (size_t)r * d;
  if (4 * tid < d) {
    const int c = 4 * tid;
    const f32x4_t v = *(const f32x4_t*)(x + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[c + j] = from_f<T>((v[j] / denom) * g0[j]);
  }
  for (int c = 4 * tid + 4096; c < d; c += 4096) {
    const f32x4_t v = *(const f32x4_t*)(x + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) y[c + j] = from_f<T>((v[j] / denom) * to_f(g[c + j]));
  }
}

// RoPE (rotate-half) on q and k, write q to q_out and k, v into the slot's pages at `pos`.
// K page layout [Hkv][P][hd]; V page layout [Hkv][hd][P].  One thread per group of 4 elements
// (a RoPE group is 4 elements and their 4 partners half a head away); with split-K partials
// the projection's reduction (in split order, plus the LoRA delta, rounded to act) happens
// here, so the QKV projection is never stored.
constexpr int kRopeMaxSplits = 16;   // split-K factor of the QKV projection

// MAXS: the split bucket of a.splits (1 without partials)
template <typename T, int MAXS>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  const int hd = a.hd, half = hd / 2, P = a.P, h4 = half / 4;
  const int qd = a.Hq * hd, kd = a.Hkv * hd, width = qd + 2 * kd;
  const int qi = a.Hq * h4, ki = a.Hkv * h4, vi = a.Hkv * (hd / 4);
  const int per_row = qi + ki + vi;
  const size_t total = (size_t)a.rows * per_row;
  const size_t split_stride = (size_t)a.rows * width;
  for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(it / per_row), w = (int)(it % per_row);
    const int pos = a.row_pos[r], slot = a.row_slot[r];
    const int dr = (a.part && a.delta_row) ? a.delta_row[r] : -1;
    // columns c .. c+3 of row r's projection in fp32 (summed from the split-K partials, or as
    // the unsplit projection stored them): q, k and v are rounded to act once, after RoPE
    // (with PAIR also columns c + off .. c + off + 3 into w; every load of both is issued
    // before the first add)
    auto load4 = [&](auto pair, int c, int off, float* v, float* w) {
      constexpr bool PAIR = decltype(pair)::value;
      f32x4_t acc, acc2;
      if (a.part) {
        f32x4_t d = {0.f, 0.f, 0.f, 0.f}, d2 = d;
        if (dr >= 0) {
          d = *(const f32x4_t*)(a.delta + (size_t)dr * a.ldd + c);
          if (PAIR) d2 = *(const f32x4_t*)(a.delta + (size_t)dr * a.ldd + c + off);
        }
        sum_split_partials<MAXS, PAIR>(a.part + (size_t)r * width + c, split_stride, a.splits, off, acc, acc2);
        if (dr >= 0) {
          acc += d;
          if (PAIR) acc2 += d2;
        }
      } else {
        acc = *(const f32x4_t*)(a.qkv + (size_t)r * width + c);
        if (PAIR) acc2 = *(const f32x4_t*)(a.qkv + (size_t)r * width + c + off);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        v[jj] = acc[jj];
        if (PAIR) w[jj] = acc2[jj];
      }
    };
    if (w < qi + ki) {
      // RoPE group: head h, elements e0 .. e0+3 and their partners e0+half ..
      const bool isq = w < qi;
      const int j = isq ? w : w - qi;
      const int h = j / h4, e0 = (j % h4) * 4;
      T* qo = (T*)a.q_out + (size_t)r * qd + h * hd + e0;
      if (pos < 0) {                           // dead row: zero q, no cache write
        if (isq)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) qo[jj] = qo[jj + half] = from_f<T>(0.f);
        continue;
      }
      // the page id (used by k only) and the rotation are loaded ahead of the projection
      const int page = a.page_table[(size_t)slot * a.max_pages + pos / P];
      float cs[4], sn[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        cs[jj] = a.cos_t[(size_t)pos * half + e0 + jj];
        sn[jj] = a.sin_t[(size_t)pos * half + e0 + jj];
      }
      float x1[4], x2[4];
      const int c0 = (isq ? 0 : qd) + h * hd + e0;
      load4(std::true_type{}, c0, half, x1, x2);
      T* dst = qo;
      if (!isq) {
        if (page < 0) continue;                // no page (never after a successful reserve)
        dst = (T*)a.k_pool + (((size_t)page * a.Hkv + h) * P + pos % P) * hd + e0;
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        dst[jj] = from_f<T>(x1[jj] * cs[jj] - x2[jj] * sn[jj]);
        dst[jj + half] = from_f<T>(x2[jj] * cs[jj] + x1[jj] * sn[jj]);
      }
    } else {
      // V: dims d0 .. d0+3 of KV head h, written into the page's transposed layout
      if (pos < 0) continue;
      const int j = w - qi - ki;
      const int h = j / (hd / 4), d0 = (j % (hd / 4)) * 4;
      const int page = a.page_table[(size_t)slot * a.max_pages + pos / P];
      float v[4];
      load4(std::false_type{}, qd + kd + h * hd + d0, 0, v, v);
      if (page < 0) continue;
      T* vp = (T*)a.v_pool + (((size_t)page * a.Hkv + h) * hd + d0) * P + pos % P;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vp[(size_t)jj * P] = from_f<T>(v[jj]);
    }
  }
}

// cos/sin of pos * base^(-2i/hd), computed in double and rounded to float.
__global__ void rope_tables_kernel(float* cos_t, float* sin_t, int max_pos, int hd, double base) {
  const int half = hd / 2;
  const size_t n = (size_t)max_pos * half;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double inv = pow(base, -2.0 * (double)i / (double)hd);
    const double ang = (double)pos * inv;
    cos_t[idx] = (float)cos(ang);
    sin_t[idx] = (float)sin(ang);
  }
}

// Debug record: row r of dst = row rows[r] of src (zeros for an index outside [0, n_src)),
// copied in 16-byte units.
__global__ __launch_bounds__(256) void debug_gather_kernel(const char* src, size_t ld_bytes, const int32_t* rows,
                                                           int n_src, int width_bytes, char* dst,
                                                           const int32_t* row_off, const int32_t* row_len, int R,
                                                           int n_slots) {
  const int r = blockIdx.x;
  int row = rows[r];
  if (row_off) {                       // block row i of slot b -> its packed row
    const bool in = row >= 0 && row < n_slots * R;
    const int b = in ? row / R : 0, i = in ? row % R : 0;
    row = (in && i < row_len[b]) ? row_off[b] + i : -1;
  }
  const bool ok = row >= 0 && row < n_src;
  u32x4_t* d = (u32x4_t*)(dst + (size_t)r * width_bytes);
  for (int c = threadIdx.x; c < width_bytes / 16; c += 256)
    d[c] = ok ? *(const u32x4_t*)(src + (size_t)row * ld_bytes + 16 * (size_t)c) : (u32x4_t){0u, 0u, 0u, 0u};
}

// Context set-up: every slot EMPTY, page tables -1, free stack popping 0, 1, 2, ... first.
__global__ void init_state_kernel(StepMeta m, int n_pages) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = t0; i < (size_t)n_pages; i += stride) m.free_stack[i] = n_pages - 1 - (int)i;
  for (size_t i = t0; i < (size_t)m.max_batch * m.max_pages; i += stride) m.page_table[i] = -1;
  int32_t* sw = (int32_t*)m.slots;
  for (size_t i = t0; i < (size_t)m.max_batch * (sizeof(isd_slot) / 4); i += stride) sw[i] = 0;
  for (size_t i = t0; i < (size_t)m.n_zero_words; i += stride) m.zero_words[i] = 0;
  if (t0 == 0) *m.n_free = n_pages;
}

}  // namespace

hipError_t launch_init_state(const StepMeta& m, int n_pages, hipStream_t s) {
  hipLaunchKernelGGL(init_state_kernel, dim3(256), dim3(256), 0, s, m, n_pages);
  return hipGetLastError();
}

hipError_t launch_assemble(const StepMeta& m, hipStream_t s) {
  hipLaunchKernelGGL(assemble_kernel, dim3(1), dim3(256), 0, s, m);
  return hipGetLastError();
}

hipError_t launch_truncate(const StepMeta& m, const int32_t* order, int n, hipStream_t s) {
  hipLaunchKernelGGL(truncate_kernel, dim3(1), dim3(256), 0, s, m, order, n);
  return hipGetLastError();
}

hipError_t launch_prefill_setup(const StepMeta& m, const PrefillCall& c, const int32_t* prompt_ids, int q_tile,
                                int32_t* order_out, hipStream_t s) {
  hipLaunchKernelGGL(prefill_setup_kernel, dim3(1), dim3(256), 0, s, m, c, prompt_ids, q_tile, order_out);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const int32_t* tok, const T* table, float* X, int rows, int d, int mask_id, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<T>, dim3(rows), dim3(256), 0, s, tok, table, X, d, mask_id);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rmsnorm(const float* X, const T* g, T* Y, int rows, int d, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(rows), dim3(1024), 0, s, X, g, Y, d, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.hd % 8 || (a.part && (a.splits < 1 || a.splits > kRopeMaxSplits))) return hipErrorInvalidValue;
  const size_t items = (size_t)a.rows * ((a.Hq + a.Hkv) * (a.hd / 8) + a.Hkv * (a.hd / 4));
  const unsigned blocks = (unsigned)std::min<size_t>((items + 255) / 256, 4096);
  switch (a.part ? split_bucket(a.splits) : 1) {
    case 1: hipLaunchKernelGGL((rope_append_kernel<T, 1>), dim3(blocks), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((rope_append_kernel<T, 2>), dim3(blocks), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((rope_append_kernel<T, 4>), dim3(blocks), dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((rope_append_kernel<T, 8>), dim3(blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((rope_append_kernel<T, 16>), dim3(blocks), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_debug_gather(const void* src, size_t ld, const int32_t* rows, int n, int n_src, int width,
                               int elem_bytes, void* dst, hipStream_t s, const int32_t* row_off,
                               const int32_t* row_len, int R) {
  if (n <= 0) return hipSuccess;
  if ((width * elem_bytes) % 16 || (ld * elem_bytes) % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(n), dim3(256), 0, s, (const char*)src, ld * elem_bytes, rows, n_src,
                     width * elem_bytes, (char*)dst, row_off, row_len, R, n_src / max(1, R));
  return hipGetLastError();
}

hipError_t launch_rope_tables(float* cos_t, float* sin_t, int max_pos, int hd, float base, hipStream_t s) {
  hipLaunchKernelGGL(rope_tables_kernel, dim3(256), dim3(256), 0, s, cos_t, sin_t, max_pos, hd, (double)base);
  return hipGetLastError();
}

template hipError_t launch_embed<float>(const int32_t*, const float*, float*, int, int, int, hipStream_t);
template hipError_t launch_embed<bf16>(const int32_t*, const bf16*, float*, int, int, int, hipStream_t);
template hipError_t launch_rmsnorm<float>(const float*, const float*, float*, int, int, float, hipStream_t);
template hipError_t launch_rmsnorm<bf16>(const float*, const bf16*, bf16*, int, int, float, hipStream_t);
template hipError_t launch_rope_append<float>(const RopeAppendArgs&, hipStream_t);
template hipError_t launch_rope_append<bf16>(const RopeAppendArgs&, hipStream_t);

}  // namespace isd
