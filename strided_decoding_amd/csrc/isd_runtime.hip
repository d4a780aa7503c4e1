// Host runtime of libisd: configuration checks, workspace carve-up, the per-pass launch
// sequence, and the C ABI declared in include/isd.h.
//
// One ISD pass (isd_step):
//   assemble (rows + page reservation) -> embed -> per layer {RMSNorm -> QKV GEMM (+LoRA on
//   MASK rows) -> RoPE + KV append -> paged attention (+ split combine) -> O GEMM + residual
//   -> RMSNorm -> gate/up GEMM + SwiGLU -> down GEMM + residual} -> final RMSNorm -> LM head
//   -> row statistics -> decide -> truncate.
// Everything is enqueued on the caller's stream; no host synchronization happens.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <new>
#include <vector>

#include "isd_common.h"

using namespace isd;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t n) {
    off = align_up(off);
    T* p = base ? (T*)(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace

struct isd_ctx {
  isd_config cfg{};
  bool bf;                // activations are bf16
  size_t act;             // bytes per activation element
  int R, qd, kd, qkvw;
  int max_pages, max_rows, max_dec_rows, n_chunks, max_splits, items_per_slot, q_max, ncb, q_tile;
  int attn_split;         // keys per context split of a decode pass
  int max_items, n_mask, delta_w;
  int mask_active = 0;          // MASK-row entries of the pass being enqueued (slots 0 .. nb-1)
  size_t part_floats = 0;       // split-K partial buffer (bf16 decode GEMMs)
  float* gemm_part = nullptr;
  // weights
  const void *embed = nullptr, *final_norm = nullptr, *lm_head = nullptr;
  std::vector<const void*> attn_norm, wqkv, wo, ffn_norm, wg, wu, wd, lora_a, lora_b;
  // pools
  char* k_pool = nullptr;
  char* v_pool = nullptr;
  size_t kv_layer_bytes = 0;
  // workspace regions
  isd_slot* slots = nullptr;
  int32_t *page_table = nullptr, *free_stack = nullptr, *n_free = nullptr;
  int32_t *row_tok = nullptr, *row_pos = nullptr, *row_slot = nullptr, *delta_row = nullptr;
  int32_t *mask_rows = nullptr, *ctx_len = nullptr, *last_rows = nullptr, *order = nullptr;
  int32_t *row_off = nullptr, *row_len = nullptr, *m_live = nullptr;   // packed rows of a decode pass
  AttnItem* items = nullptr;
  float* X = nullptr;
  float* QKV = nullptr;   // the unsplit QKV projection in fp32 (q, k, v are rounded once, after RoPE)
  void *Xn = nullptr, *Qr = nullptr, *O = nullptr, *H = nullptr;
  float *part_o = nullptr, *part_ml = nullptr;
  float* logits[2] = {nullptr, nullptr};
  ChunkStat* stats[2] = {nullptr, nullptr};
  float *cos_t = nullptr, *sin_t = nullptr;
  void* lora_s = nullptr;
  float* lora_delta = nullptr;
  int32_t* tile_cnt = nullptr;  // arrival counters of the k-split LoRA shrink
  int n_cnt = 0;
  int cur = 0;            // logits buffer the next pass writes
  bool prefilled = false;
  std::vector<long long> reserved;   // admission reservation per slot (pages)
  long long reserved_total = 0;
  isd_status sticky = ISD_OK;
  int32_t* sticky_host = nullptr;   // pinned host word the truncate kernel reports into (device address)
  int32_t* sticky_host_h = nullptr; // the same word's host address
  // kernel timing (isd_profile)
  bool prof_on = false;
  bool prof_overflow = false;
  std::vector<hipEvent_t> ev_pool;
  std::vector<std::pair<const char*, int>> prof_recs;
  int ev_used = 0;
  // graph replay of isd_step (isd_set_graphs): one executable graph per logits-buffer parity,
  // valid for the output pointers it was captured with
  bool graphs = true;
  bool meter = false;           // introspective acceptance meter (isd_set_meter)
  hipStream_t cap_stream = nullptr;
  struct StepGraph {
    hipGraphExec_t exec = nullptr;
    const void *tokens = nullptr, *n_commit = nullptr, *n_accept = nullptr;
  };
  // one graph per (logits-buffer parity, active slot count, passes per launch)
  std::map<std::tuple<int, int, int>, StepGraph> step_graph;
};

namespace {

constexpr int kProfEvents = 1 << 15;

// Records a HIP event pair around the launches in its scope when profiling is on.
struct ProfScope {
  isd_ctx& x;
  hipStream_t s;
  int idx = -1;
  ProfScope(isd_ctx& x_, const char* name, hipStream_t s_) : x(x_), s(s_) {
    if (!x.prof_on) return;
    if (x.ev_used + 2 > (int)x.ev_pool.size()) {
      x.prof_overflow = true;
      return;
    }
    idx = x.ev_used;
    x.ev_used += 2;
    hipEventRecord(x.ev_pool[idx], s);
    x.prof_recs.emplace_back(name, idx);
  }
  ~ProfScope() {
    if (idx >= 0) hipEventRecord(x.ev_pool[idx + 1], s);
  }
};

}  // namespace

namespace {

isd_status check_config(const isd_config* c) {
  if (!c) return ISD_E_ARG;
  if (c->dtype != ISD_F32 && c->dtype != ISD_BF16) return ISD_E_ARG;
  if (c->propose != ISD_PROPOSE_SAMPLE && c->propose != ISD_PROPOSE_ARGMAX) return ISD_E_ARG;
  if (!(c->temperature >= 0.f)) return ISD_E_ARG;
  if (c->stride_n < 1 || c->stride_n > ISD_MAX_STRIDE) return ISD_E_ARG;
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->d_ffn < 1 || c->vocab < 2 || c->max_batch < 1 || c->max_seq_len < 1 || c->n_pages < 1 ||
      c->max_prefill_tokens < 1 || c->lora_rank < 0 || !(c->rms_eps > 0.f) || !(c->rope_base > 0.f))
    return ISD_E_ARG;
  if (c->page_size != 16) return ISD_E_SHAPE;
  if (c->n_q_heads % c->n_kv_heads) return ISD_E_SHAPE;
  if (c->head_dim % 2 || c->d_model % 4) return ISD_E_SHAPE;
  if (c->vocab > kStatChunk * 256) return ISD_E_SHAPE;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->dtype == ISD_BF16) {
    if (c->head_dim != 128) return ISD_E_SHAPE;
    if (G > 8) return ISD_E_SHAPE;
    if (c->d_model % 64 || c->d_ffn % 64 || (c->n_q_heads * c->head_dim) % 64) return ISD_E_SHAPE;
    if (c->lora_rank % 64) return ISD_E_SHAPE;
  } else {
    if (c->head_dim > 256) return ISD_E_SHAPE;
  }
  return ISD_OK;
}

// Carve the workspace (base == nullptr: size only).
size_t carve(isd_ctx& x, char* base) {
  const isd_config& c = x.cfg;
  Carver cv{base};
  const int B = c.max_batch, d = c.d_model, V = c.vocab, F = c.d_ffn;
  x.slots = cv.take<isd_slot>(B);
  x.page_table = cv.take<int32_t>((size_t)B * x.max_pages);
  x.free_stack = cv.take<int32_t>(c.n_pages);
  x.n_free = cv.take<int32_t>(64);
  x.row_tok = cv.take<int32_t>(x.max_rows);
  x.row_pos = cv.take<int32_t>(x.max_rows);
  x.row_slot = cv.take<int32_t>(x.max_rows);
  x.delta_row = cv.take<int32_t>(x.max_rows);
  x.mask_rows = cv.take<int32_t>(std::max(1, x.n_mask));
  x.ctx_len = cv.take<int32_t>(B);
  x.row_off = cv.take<int32_t>(B);
  x.row_len = cv.take<int32_t>(B);
  x.m_live = cv.take<int32_t>(64);
  x.last_rows = cv.take<int32_t>(B);
  x.order = cv.take<int32_t>(B);
  x.items = cv.take<AttnItem>(x.max_items);
  x.X = cv.take<float>((size_t)x.max_rows * d);
  x.Xn = cv.take<char>((size_t)x.max_rows * d * x.act);
  x.QKV = cv.take<float>((size_t)x.max_rows * x.qkvw);
  x.Qr = cv.take<char>((size_t)x.max_rows * x.qd * x.act);
  x.O = cv.take<char>((size_t)x.max_rows * x.qd * x.act);
  x.H = cv.take<char>((size_t)x.max_rows * F * x.act);
  if (x.bf) {
    x.part_o = cv.take<float>((size_t)x.max_splits * x.max_dec_rows * x.qd);
    x.part_ml = cv.take<float>((size_t)x.max_splits * x.max_dec_rows * c.n_q_heads * 2);
    x.gemm_part = cv.take<float>(x.part_floats);
  }
  for (int i = 0; i < 2; ++i) {
    x.logits[i] = cv.take<float>((size_t)x.max_dec_rows * V);
    x.stats[i] = cv.take<ChunkStat>((size_t)x.max_dec_rows * x.n_chunks);
  }
  const int max_pos = c.max_seq_len + 2 * c.stride_n;
  x.cos_t = cv.take<float>((size_t)max_pos * (c.head_dim / 2));
  x.sin_t = cv.take<float>((size_t)max_pos * (c.head_dim / 2));
  if (c.lora_rank > 0) {
    x.lora_s = cv.take<char>((size_t)std::max(1, x.n_mask) * 3 * c.lora_rank * x.act);
    x.lora_delta = cv.take<float>((size_t)std::max(1, x.n_mask) * x.delta_w);
    x.tile_cnt = cv.take<int32_t>(x.n_cnt);
  }
  return align_up(cv.off);
}

void derive(isd_ctx& x) {
  const isd_config& c = x.cfg;
  x.bf = c.dtype == ISD_BF16;
  x.act = x.bf ? 2 : 4;
  x.R = 2 * c.stride_n - 1;
  x.qd = c.n_q_heads * c.head_dim;
  x.kd = c.n_kv_heads * c.head_dim;
  x.qkvw = x.qd + 2 * x.kd;
  x.max_pages = cdiv(c.max_seq_len + 2 * c.stride_n, c.page_size);
  x.max_dec_rows = c.max_batch * x.R;
  x.max_rows = std::max(x.max_dec_rows, c.max_prefill_tokens);
  x.n_chunks = cdiv(c.vocab, kStatChunk);
  // (a function of the configuration's sequence length, not of the stride, so that an AR
  // context and an ISD context of the same model split every row's keys alike)
  x.attn_split = attn_split_len(c.max_batch, c.n_kv_heads, c.max_seq_len);
  x.max_splits = cdiv(c.max_seq_len + 2 * c.stride_n, x.attn_split);
  const int G = c.n_q_heads / c.n_kv_heads;
  x.ncb = (x.R * G <= 32) ? 2 : 4;
  x.q_max = std::max(1, 16 * x.ncb / G);
  x.items_per_slot = cdiv(x.R, x.q_max);
  x.q_tile = x.q_max;
  x.max_items = std::max(c.max_batch * x.items_per_slot, cdiv(c.max_prefill_tokens, x.q_tile) + c.max_batch);
  x.n_mask = c.max_batch * (c.stride_n - 1);
  x.delta_w = std::max(std::max(x.qkvw, 2 * c.d_ffn), c.d_model);
  // split-K partials: the largest S * rows * width over the decode projections
  {
    const int d = c.d_model, F = c.d_ffn, r = std::max(c.lora_rank, 1);
    const size_t M = x.max_dec_rows, Mm = std::max(1, x.n_mask);
    auto need = [](size_t m, int n, int k, bool dual) {
      return (size_t)gemm_splits(n, k, dual) * m * n * (dual ? 2 : 1);
    };
    size_t p = std::max({need(M, x.qkvw, d, false), need(M, d, x.qd, false), need(M, F, d, true),
                         need(M, d, F, false), need(M, c.vocab, d, false)});
    if (c.lora_rank > 0) {
      p = std::max({p, need(Mm, 3 * r, d, false), need(Mm, 2 * r, d, false), need(Mm, r, d, false),
                    need(Mm, r, x.qd, false), need(Mm, r, F, false)});
      // the single-launch shrink: lora_shrink_splits(K) partials of the stacked width
      p = std::max({p, (size_t)lora_shrink_splits(d) * Mm * 3 * r, (size_t)lora_shrink_splits(x.qd) * Mm * r,
                    (size_t)lora_shrink_splits(F) * Mm * r});
    }
    x.part_floats = x.bf ? p : 0;
  }
  x.kv_layer_bytes = (size_t)c.n_pages * x.kd * c.page_size * x.act;
  x.n_cnt = c.lora_rank > 0 ? cdiv(std::max(1, x.n_mask), 32) * cdiv(3 * c.lora_rank, 32) : 0;
}

StepMeta meta(isd_ctx& x) {
  StepMeta m{};
  m.slots = x.slots;
  m.page_table = x.page_table;
  m.max_pages = x.max_pages;
  m.free_stack = x.free_stack;
  m.n_free = x.n_free;
  m.row_tok = x.row_tok;
  m.row_pos = x.row_pos;
  m.row_slot = x.row_slot;
  m.delta_row = x.delta_row;
  m.mask_rows = x.mask_rows;
  m.ctx_len = x.ctx_len;
  m.items = x.items;
  m.items_per_slot = x.items_per_slot;
  m.q_max = x.q_max;
  m.max_batch = x.cfg.max_batch;
  m.n_active = x.cfg.max_batch;
  m.N = x.cfg.stride_n;
  m.P = x.cfg.page_size;
  m.mask_id = x.cfg.vocab;
  m.last_rows = x.last_rows;
  m.zero_words = x.tile_cnt;
  m.n_zero_words = x.n_cnt;
  m.sticky_host = x.sticky_host;
  m.row_off = x.row_off;
  m.row_len = x.row_len;
  m.m_live = x.m_live;
  return m;
}

#define HIP_OK(expr)                       \
  do {                                     \
    if ((expr) != hipSuccess) return ISD_E_HIP; \
  } while (0)
// launch under a profiling scope (context reference `x` / context pointer `x`, stream `s`)
#define TIMED(name, expr)                  \
  do {                                     \
    ProfScope p_(x, name, s);              \
    HIP_OK(expr);                          \
  } while (0)
#define TIMEDP(name, expr)                 \
  do {                                     \
    ProfScope p_(*x, name, s);             \
    HIP_OK(expr);                          \
  } while (0)

// Launch a projection.  bf16 GEMMs with at most a decode pass's rows use the split-K factor
// of their (N, K); larger row counts (prefill) run unsplit.
GemmArgs plan_gemm(const isd_ctx& x, GemmArgs g) {
  g.splits = 1;
  g.part = nullptr;
  if (x.bf && g.M <= x.max_dec_rows && x.gemm_part) {
    const bool dual = g.epi == EPI_SWIGLU;
    const int S = gemm_splits(g.N, g.K, dual);
    if ((size_t)S * g.M * g.N * (dual ? 2 : 1) <= x.part_floats) {
      g.splits = S;
      g.part = x.gemm_part;
    }
  }
  return g;
}

hipError_t gemm(const isd_ctx& x, GemmArgs g, hipStream_t s) {
  if (!x.bf) return launch_gemm_f32(g, s);
  return launch_gemm_bf16(plan_gemm(x, g), s);
}

GemmArgs gargs(const void* A, int lda, const void* B0, int ldb, int M, int N, int K, int epi) {
  GemmArgs g{};
  g.A = A;
  g.lda = lda;
  g.B0 = B0;
  g.ldb = ldb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi = epi;
  return g;
}

// LoRA of nt targets sharing one input on the MASK rows (targets t0 .. t0+nt-1, output widths
// n[j]): S[:, j r .. (j+1) r] = X[mask_rows] A_j^T, then delta[:, o_j .. o_j + n_j] = S_j B_j^T with
// o_j = n_0 + .. + n_{j-1}, added to the MASK rows of `base`, the group's projection.  When the
// targets' A (and B) matrices are stacked in memory the shrinks run as one product (on the bf16
// path one lora_shrink_kernel launch, k-split partials summed by the last workgroup to
// arrive); on the bf16 path with stacked B the expand is fused into `base` itself (its MASK
// rows run r more k values over S and B, the other rows add zeros), else it runs as separate
// products into an fp32 delta that base's epilogue adds.
isd_status lora_group(isd_ctx& x, int layer, int t0, int nt, const void* Xsrc, int ldx, int k_in, const int* n,
                      hipStream_t s, GemmArgs& base) {
  const int r = x.cfg.lora_rank, M = x.mask_active;
  const char* const* A = (const char* const*)&x.lora_a[(size_t)layer * 7 + t0];
  const char* const* Bm = (const char* const*)&x.lora_b[(size_t)layer * 7 + t0];
  bool stackA = true, stackB = x.bf;     // segmented products: bf16 kernels only
  for (int j = 1; j < nt; ++j) {
    stackA = stackA && A[j] == A[j - 1] + (size_t)r * k_in * x.act;
    stackB = stackB && Bm[j] == Bm[j - 1] + (size_t)n[j - 1] * r * x.act && n[j - 1] % 256 == 0;
  }
  for (int j = 0; j < nt; ++j) {
    if (j > 0 && stackA) break;
    const int ncols = stackA ? nt * r : r;
    if (x.bf && k_in % 128 == 0 && lora_shrink_splits(k_in) <= 32 && ncols % 32 == 0 && x.tile_cnt) {
      ShrinkArgs sa{};
      sa.X = Xsrc;
      sa.ldx = ldx;
      sa.rows = x.mask_rows;
      sa.M = M;
      sa.A = A[j];
      sa.N = ncols;
      sa.K = k_in;
      sa.out = (char*)x.lora_s + (size_t)j * r * x.act;
      sa.ldo = 3 * r;
      sa.part = x.gemm_part;
      sa.part_floats = x.part_floats;
      sa.cnt = x.tile_cnt;
      sa.n_cnt = x.n_cnt;
      TIMED("lora_shrink", launch_lora_shrink(sa, s));
      continue;
    }
    GemmArgs g = gargs(Xsrc, ldx, A[j], k_in, M, ncols, k_in, EPI_STORE);
    g.a_rows = x.mask_rows;
    g.C = (char*)x.lora_s + (size_t)j * r * x.act;
    g.ldc = 3 * r;
    TIMED("lora_shrink", gemm(x, g, s));
  }
  if (stackB && r % 32 == 0) {
    base.lora_rows = x.delta_row;
    base.lora_a = x.lora_s;
    base.ld_la = 3 * r;
    base.lora_r = r;
    base.lora_b0 = Bm[0];
    if (base.epi == EPI_SWIGLU) {
      base.lora_b1 = Bm[1];
      base.lora_nseg = 1;
    } else {
      base.lora_nseg = nt;
      int o = 0;
      for (int j = 0; j < nt; ++j) base.lora_seg_end[j] = (o += n[j]);
    }
    return ISD_OK;
  }
  int o = 0;
  for (int j = 0; j < nt; ++j) {
    if (j > 0 && stackB) break;
    int n_out = n[j];
    GemmArgs e = gargs((const char*)x.lora_s + (size_t)j * r * x.act, 3 * r, Bm[j], r, M, n_out, r, EPI_STORE_F32);
    if (stackB && nt > 1) {
      n_out = 0;
      e.nseg = nt;
      for (int i = 0; i < nt; ++i) {
        n_out += n[i];
        e.seg_end[i] = n_out;
        e.seg_aoff[i] = i * r;
      }
      e.N = n_out;
    }
    e.C = x.lora_delta + o;
    e.ldc = x.delta_w;
    TIMED("lora_expand", gemm(x, e, s));
    o += n_out;
  }
  base.delta = x.lora_delta;
  base.delta_row = x.delta_row;
  base.ldd = x.delta_w;
  if (base.epi == EPI_SWIGLU) base.delta_off2 = n[0];
  return ISD_OK;
}


// The transformer body over M rows.  decode: split-context attention over the decode items;
// prefill: one pass per item.  lm_rows: rows fed to the LM head (gather list or null = all),
// whose fp32 logits go to logits_out.
isd_status forward(isd_ctx& x, int M, int n_items, bool decode, const int32_t* lm_rows, int lm_M, bool lora,
                   float* logits_out, const isd_debug* dbg, hipStream_t s) {
  const isd_config& c = x.cfg;
  const int d = c.d_model, F = c.d_ffn, Hq = c.n_q_heads, Hkv = c.n_kv_heads, hd = c.head_dim;
  const int nd = dbg ? dbg->n_rows : 0;
  // decode passes pack their live rows first; the projections skip the rest
  const int32_t* live = decode ? x.m_live : nullptr;
  // debug record of the followed rows (block row i of slot b, mapped to its packed row): dst
  // slice `idx` of `width` elements per row
  auto record = [&](const void* src, int width, int esize, void* dst, int idx) -> hipError_t {
    if (!nd || !dst) return hipSuccess;
    return launch_debug_gather(src, width, dbg->rows, nd, M, width, esize,
                               (char*)dst + (size_t)idx * nd * width * esize, s, x.row_off, x.row_len, x.R);
  };
  if (x.bf) TIMED("embed", launch_embed<bf16>(x.row_tok, (const bf16*)x.embed, x.X, M, d, c.vocab, s));
  else TIMED("embed", launch_embed<float>(x.row_tok, (const float*)x.embed, x.X, M, d, c.vocab, s));
  for (int l = 0; l < c.n_layers; ++l) {
    char* kl = x.k_pool + (size_t)l * x.kv_layer_bytes;
    char* vl = x.v_pool + (size_t)l * x.kv_layer_bytes;
    HIP_OK(record(x.X, d, 4, dbg ? dbg->layer_in : nullptr, l));
    // attention block (layers after the first get their input norm from the previous
    // layer's down projection)
    if (l == 0) {
      if (x.bf) TIMED("rmsnorm", launch_rmsnorm<bf16>(x.X, (const bf16*)x.attn_norm[0], (bf16*)x.Xn, M, d, c.rms_eps, s));
      else TIMED("rmsnorm", launch_rmsnorm<float>(x.X, (const float*)x.attn_norm[0], (float*)x.Xn, M, d, c.rms_eps, s));
    }
    // QKV projection; with split-K its partials are reduced by rope_append itself
    GemmArgs gq = plan_gemm(x, gargs(x.Xn, d, x.wqkv[l], d, M, x.qkvw, d, EPI_STORE_F32));
    gq.m_live = live;
    gq.C = x.QKV;
    gq.ldc = x.qkvw;
    if (lora) {
      const int n[3] = {x.qd, x.kd, x.kd};
      isd_status st = lora_group(x, l, 0, 3, x.Xn, d, d, n, s, gq);
      if (st != ISD_OK) return st;
    }
    gq.keep_part = 1;
    if (x.bf) TIMED("gemm_qkv", launch_gemm_bf16(gq, s));
    else TIMED("gemm_qkv", launch_gemm_f32(gq, s));
    {
      RopeAppendArgs ra{};
      if (x.bf && gq.splits > 1) {
        ra.part = gq.part;
        ra.splits = gq.splits;
        ra.delta_row = gq.delta_row;
        ra.delta = gq.delta;
        ra.ldd = gq.ldd;
      }
      ra.qkv = x.QKV;
      ra.q_out = x.Qr;
      ra.k_pool = kl;
      ra.v_pool = vl;
      ra.page_table = x.page_table;
      ra.max_pages = x.max_pages;
      ra.row_pos = x.row_pos;
      ra.row_slot = x.row_slot;
      ra.cos_t = x.cos_t;
      ra.sin_t = x.sin_t;
      ra.rows = M;
      ra.Hq = Hq;
      ra.Hkv = Hkv;
      ra.hd = hd;
      ra.P = c.page_size;
      if (x.bf) TIMED("rope_append", launch_rope_append<bf16>(ra, s));
      else TIMED("rope_append", launch_rope_append<float>(ra, s));
    }
    {
      AttnArgs aa{};
      aa.q = x.Qr;
      aa.k_pool = kl;
      aa.v_pool = vl;
      aa.page_table = x.page_table;
      aa.max_pages = x.max_pages;
      aa.items = x.items;
      aa.n_items = n_items;
      aa.ctx_len = x.ctx_len;
      aa.Hq = Hq;
      aa.Hkv = Hkv;
      aa.hd = hd;
      aa.P = c.page_size;
      aa.ncb = x.ncb;
      aa.out = x.O;
      aa.row_pos = x.row_pos;
      aa.row_slot = x.row_slot;
      aa.n_rows = M;
      if (!x.bf) {
        TIMED("attention", launch_attn_f32(aa, s));
      } else if (decode) {
        aa.split = x.attn_split;
        aa.max_splits = x.max_splits;
        aa.part_o = x.part_o;
        aa.part_ml = x.part_ml;
        aa.part_rows = x.max_dec_rows;
        TIMED("attention", launch_attn_bf16(aa, s));
        // with one split every live row is final in the attention kernel (rows past the live
        // ones are never read): no merge
        if (x.max_splits > 1) TIMED("attn_combine", launch_attn_combine_bf16(aa, s));
      } else {
        aa.split = 0;
        TIMED("attention", launch_attn_bf16(aa, s));
      }
    }
    HIP_OK(record(x.O, x.qd, (int)x.act, dbg ? dbg->layer_attn : nullptr, l));
    {
      // O projection + residual, then the FFN input norm of the updated rows
      GemmArgs g = gargs(x.O, x.qd, x.wo[l], x.qd, M, d, x.qd, EPI_RESID);
      g.m_live = live;
      g.R = x.X;
      g.ldr = d;
      g.norm_g = x.ffn_norm[l];
      g.norm_out = x.Xn;
      g.norm_eps = c.rms_eps;
      if (lora) {
        const int n[1] = {d};
        isd_status st = lora_group(x, l, 3, 1, x.O, x.qd, x.qd, n, s, g);
        if (st != ISD_OK) return st;
      }
      TIMED("gemm_o", gemm(x, g, s));
    }
    // FFN block
    {
      GemmArgs g = gargs(x.Xn, d, x.wg[l], d, M, F, d, EPI_SWIGLU);
      g.m_live = live;
      g.B1 = x.wu[l];
      g.C = x.H;
      g.ldc = F;
      if (lora) {
        const int n[2] = {F, F};
        isd_status st = lora_group(x, l, 4, 2, x.Xn, d, d, n, s, g);
        if (st != ISD_OK) return st;
      }
      TIMED("gemm_gate_up", gemm(x, g, s));
    }
    {
      // down projection + residual, then the next layer's input norm (the final norm last)
      GemmArgs g = gargs(x.H, F, x.wd[l], F, M, d, F, EPI_RESID);
      g.m_live = live;
      g.R = x.X;
      g.ldr = d;
      g.norm_g = l + 1 < c.n_layers ? x.attn_norm[l + 1] : x.final_norm;
      g.norm_out = x.Xn;
      g.norm_eps = c.rms_eps;
      if (lora) {
        const int n[1] = {d};
        isd_status st = lora_group(x, l, 6, 1, x.H, F, F, n, s, g);
        if (st != ISD_OK) return st;
      }
      TIMED("gemm_down", gemm(x, g, s));
    }
  }
  HIP_OK(record(x.X, d, 4, dbg ? dbg->layer_in : nullptr, c.n_layers));
  HIP_OK(record(x.Xn, d, (int)x.act, dbg ? dbg->final_normed : nullptr, 0));
  GemmArgs g = gargs(x.Xn, d, x.lm_head, d, lm_M, c.vocab, d, EPI_STORE_F32);
  g.m_live = live;
  g.a_rows = lm_rows;
  g.C = logits_out;
  g.ldc = c.vocab;
  TIMED("lm_head", gemm(x, g, s));
  return ISD_OK;
}

SampleArgs sargs(isd_ctx& x) {
  SampleArgs a{};
  a.slots = x.slots;
  a.N = x.cfg.stride_n;
  a.V = x.cfg.vocab;
  a.propose = x.cfg.propose;
  a.T = x.cfg.temperature;
  a.seed = x.cfg.seed;
  a.n_chunks = x.n_chunks;
  a.meter = x.meter ? 1 : 0;
  return a;
}

// The sticky device status as far as the host has seen it (no synchronization).
isd_status sticky_now(isd_ctx* x) {
  if (x->sticky == ISD_OK && x->sticky_host_h) {
    const int32_t v = *(volatile int32_t*)x->sticky_host_h;
    if (v != 0) x->sticky = (isd_status)v;
  }
  return x->sticky;
}

}  // namespace

extern "C" {

const char* isd_version(void) { return "isd-mi355x 0.1 (gfx950)"; }

isd_status isd_init(const isd_config* cfg, const isd_weights* w, void* kv_pool, void* workspace, isd_sizes* sizes,
                    isd_ctx** out, void* stream) {
  if (!cfg || !sizes || !out) return ISD_E_ARG;
  *out = nullptr;
  isd_status st = check_config(cfg);
  if (st != ISD_OK) return st;
  isd_ctx probe;
  probe.cfg = *cfg;
  derive(probe);
  sizes->kv_pool_bytes = 2 * (size_t)cfg->n_layers * probe.kv_layer_bytes;
  sizes->workspace_bytes = carve(probe, nullptr);
  if (!kv_pool && !workspace) return ISD_OK;
  if (!kv_pool || !workspace || !w) return ISD_E_ARG;
  if (((uintptr_t)kv_pool % kAlign) || ((uintptr_t)workspace % kAlign)) return ISD_E_ARG;
  const int L = cfg->n_layers;
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm ||
      !w->wg || !w->wu || !w->wd)
    return ISD_E_ARG;
  if (cfg->lora_rank > 0 && (!w->lora_a || !w->lora_b)) return ISD_E_ARG;
  isd_ctx* x = new (std::nothrow) isd_ctx();
  if (!x) return ISD_E_ARG;
  x->cfg = *cfg;
  derive(*x);
  carve(*x, (char*)workspace);
  x->embed = w->embed;
  x->final_norm = w->final_norm;
  x->lm_head = w->lm_head;
  x->attn_norm.assign(w->attn_norm, w->attn_norm + L);
  x->wqkv.assign(w->wqkv, w->wqkv + L);
  x->wo.assign(w->wo, w->wo + L);
  x->ffn_norm.assign(w->ffn_norm, w->ffn_norm + L);
  x->wg.assign(w->wg, w->wg + L);
  x->wu.assign(w->wu, w->wu + L);
  x->wd.assign(w->wd, w->wd + L);
  for (int l = 0; l < L; ++l)
    if (!x->attn_norm[l] || !x->wqkv[l] || !x->wo[l] || !x->ffn_norm[l] || !x->wg[l] || !x->wu[l] || !x->wd[l]) {
      delete x;
      return ISD_E_ARG;
    }
  if (cfg->lora_rank > 0) {
    x->lora_a.assign(w->lora_a, w->lora_a + (size_t)L * 7);
    x->lora_b.assign(w->lora_b, w->lora_b + (size_t)L * 7);
    for (size_t i = 0; i < x->lora_a.size(); ++i)
      if (!x->lora_a[i] || !x->lora_b[i]) {
        delete x;
        return ISD_E_ARG;
      }
  }
  x->k_pool = (char*)kv_pool;
  x->v_pool = (char*)kv_pool + (size_t)L * x->kv_layer_bytes;
  x->reserved.assign(cfg->max_batch, 0);
  // the sticky device status: one pinned host word the truncate kernel writes (host memory:
  // the library still allocates no device memory)
  void* hw = nullptr;
  if (hipHostMalloc(&hw, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    delete x;
    return ISD_E_HIP;
  }
  *(volatile int32_t*)hw = 0;
  void* dw = nullptr;
  if (hipHostGetDevicePointer(&dw, hw, 0) != hipSuccess) {
    hipHostFree(hw);
    delete x;
    return ISD_E_HIP;
  }
  x->sticky_host_h = (int32_t*)hw;
  x->sticky_host = (int32_t*)dw;
  hipStream_t s = (hipStream_t)stream;
  StepMeta m = meta(*x);
  if (launch_init_state(m, cfg->n_pages, s) != hipSuccess ||
      launch_rope_tables(x->cos_t, x->sin_t, cfg->max_seq_len + 2 * cfg->stride_n, cfg->head_dim, cfg->rope_base, s) !=
          hipSuccess) {
    hipHostFree(hw);
    delete x;
    return ISD_E_HIP;
  }
  *out = x;
  return ISD_OK;
}

isd_status isd_prefill(isd_ctx* x, int32_t n, const int32_t* slots, const int32_t* prompt_ids, const int32_t* offsets,
                       const int32_t* max_new, int32_t* first_tok, void* stream) {
  if (!x || !slots || !prompt_ids || !offsets || !max_new || !first_tok) return ISD_E_ARG;
  const isd_config& c = x->cfg;
  if (n < 1 || n > c.max_batch || n > kMaxPrefillSlots) return ISD_E_ARG;
  if (offsets[0] != 0) return ISD_E_ARG;
  std::vector<char> seen(c.max_batch, 0);
  long long new_total = x->reserved_total;
  PrefillCall call{};
  call.n = n;
  call.off[0] = 0;
  call.item_off[0] = 0;
  for (int i = 0; i < n; ++i) {
    const int b = slots[i];
    if (b < 0 || b >= c.max_batch || seen[b]) return ISD_E_ARG;
    seen[b] = 1;
    const int len = offsets[i + 1] - offsets[i];
    if (len < 1 || max_new[i] < 1) return ISD_E_ARG;
    if ((long long)len + max_new[i] + 2 * c.stride_n > c.max_seq_len) return ISD_E_CAPACITY;
    const long long res = cdiv(len + max_new[i] + 2 * c.stride_n, c.page_size);
    new_total += res - x->reserved[b];
    call.slot[i] = b;
    call.off[i + 1] = offsets[i + 1];
    call.max_new[i] = max_new[i];
    call.item_off[i + 1] = call.item_off[i] + cdiv(len, x->q_tile);
  }
  const int M = offsets[n];
  if (M > c.max_prefill_tokens) return ISD_E_CAPACITY;
  if (new_total > c.n_pages) return ISD_E_CAPACITY;
  if (call.item_off[n] > x->max_items) return ISD_E_CAPACITY;
  for (int i = 0; i < n; ++i) {
    const int b = slots[i];
    const int len = offsets[i + 1] - offsets[i];
    const long long res = cdiv(len + max_new[i] + 2 * c.stride_n, c.page_size);
    x->reserved_total += res - x->reserved[b];
    x->reserved[b] = res;
  }
  hipStream_t s = (hipStream_t)stream;
  StepMeta m = meta(*x);
  TIMEDP("prefill_setup", launch_prefill_setup(m, call, prompt_ids, x->q_tile, x->order, s));
  isd_status st = forward(*x, M, call.item_off[n], /*decode=*/false, x->last_rows, n, /*lora=*/false,
                          x->logits[x->cur], nullptr, s);
  if (st != ISD_OK) return st;
  TIMEDP("row_stats", launch_row_stats(x->logits[x->cur], n, c.vocab, c.temperature, x->stats[x->cur], s));
  SampleArgs a = sargs(*x);
  a.n_slots = n;
  a.slot_ids = x->order;
  a.logits = x->logits[x->cur];
  a.rows_per_slot = 1;
  a.stats = x->stats[x->cur];
  a.prefill = 1;
  a.first_tok = first_tok;
  TIMEDP("decide", launch_decide(a, s));
  TIMEDP("truncate", launch_truncate(m, x->order, n, s));
  x->prefilled = true;
  return sticky_now(x);
}

namespace {

// The launches of one decode pass over slots 0 .. nb-1 on stream s, reading logits buffer
// parity cur.  The rows of slot b are b R .. b R + R-1 whatever nb is, and every kernel
// computes a row from that row alone, so a slot's results do not depend on nb.
isd_status step_launches(isd_ctx* x, int nb, int32_t* tokens, int32_t* n_commit, int32_t* n_accept, int cur,
                         const isd_debug* dbg, hipStream_t s) {
  const isd_config& c = x->cfg;
  StepMeta m = meta(*x);
  m.n_active = nb;
  TIMEDP("assemble", launch_assemble(m, s));
  const int M = nb * x->R;
  x->mask_active = nb * (c.stride_n - 1);
  isd_status st = forward(*x, M, nb * x->items_per_slot, /*decode=*/true, nullptr, M,
                          /*lora=*/c.lora_rank > 0 && c.stride_n > 1, x->logits[cur], dbg, s);
  if (st != ISD_OK) return st;
  const int prev = cur ^ 1;
  TIMEDP("row_stats", launch_row_stats(x->logits[cur], M, c.vocab, c.temperature, x->stats[cur], s, x->m_live));
  SampleArgs a = sargs(*x);
  a.n_slots = nb;
  a.row_off = x->row_off;
  a.logits = x->logits[cur];
  a.rows_per_slot = x->R;
  a.stats = x->stats[cur];
  a.q_logits = x->logits[prev];
  a.q_stats = x->stats[prev];
  a.q_rows = M;
  a.tokens = tokens;
  a.n_commit = n_commit;
  a.n_accept = n_accept;
  if (dbg) {
    a.margins = dbg->margins;
    a.kinds = dbg->kinds;
  }
  TIMEDP("decide", launch_decide(a, s));
  TIMEDP("truncate", launch_truncate(m, nullptr, c.max_batch, s));
  return ISD_OK;
}

void drop_graphs(isd_ctx* x) {
  for (auto& kv : x->step_graph)
    if (kv.second.exec) hipGraphExecDestroy(kv.second.exec);
  x->step_graph.clear();
}

// n_passes passes over slots 0 .. nb-1: pass i writes tokens + i B N, n_commit + i B,
// n_accept + i B.  From a captured graph (one per parity, nb and n_passes) when graphs are on
// and the passes are neither profiled nor debugged; kernel by kernel otherwise.
isd_status run_passes(isd_ctx* x, int nb, int n_passes, int32_t* tokens, int32_t* n_commit, int32_t* n_accept,
                      const isd_debug* dbg, hipStream_t s) {
  const int B = x->cfg.max_batch, N = x->cfg.stride_n;
  const int cur = x->cur;
  auto launches = [&](hipStream_t st) -> isd_status {
    for (int i = 0; i < n_passes; ++i) {
      const isd_status r = step_launches(x, nb, tokens + (size_t)i * B * N, n_commit + (size_t)i * B,
                                         n_accept + (size_t)i * B, cur ^ (i & 1), dbg, st);
      if (r != ISD_OK) return r;
    }
    return ISD_OK;
  };
  if (x->graphs && !x->prof_on && !dbg) {
    if (!x->cap_stream) HIP_OK(hipStreamCreateWithFlags(&x->cap_stream, hipStreamNonBlocking));
    isd_ctx::StepGraph& g = x->step_graph[std::make_tuple(cur, nb, n_passes)];
    if (g.exec && (g.tokens != tokens || g.n_commit != n_commit || g.n_accept != n_accept)) {
      hipGraphExecDestroy(g.exec);
      g = isd_ctx::StepGraph{};
    }
    if (!g.exec) {
      hipGraph_t graph = nullptr;
      HIP_OK(hipStreamBeginCapture(x->cap_stream, hipStreamCaptureModeRelaxed));
      const isd_status st = launches(x->cap_stream);
      const hipError_t e = hipStreamEndCapture(x->cap_stream, &graph);
      if (st != ISD_OK) {
        if (graph) hipGraphDestroy(graph);
        return st;
      }
      if (e != hipSuccess || !graph) return ISD_E_HIP;
      const hipError_t ei = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
      hipGraphDestroy(graph);
      if (ei != hipSuccess) {
        g.exec = nullptr;
        return ISD_E_HIP;
      }
      g.tokens = tokens;
      g.n_commit = n_commit;
      g.n_accept = n_accept;
    }
    HIP_OK(hipGraphLaunch(g.exec, s));
  } else {
    const isd_status st = launches(s);
    if (st != ISD_OK) return st;
  }
  x->cur = cur ^ (n_passes & 1);
  return sticky_now(x);
}

// A debug record the context can fill: row count in range, and every recorded row width a
// whole number of 16-byte units.
bool debug_ok(const isd_ctx* x, const isd_debug* d) {
  if (!d) return true;
  if (d->n_rows < 0 || d->n_rows > ISD_DEBUG_MAX_ROWS) return false;
  if (d->n_rows > 0 && !d->rows) return false;
  const isd_config& c = x->cfg;
  if ((d->layer_in || d->layer_attn || d->final_normed) && d->n_rows > 0) {
    if (((size_t)c.d_model * 4) % 16 || ((size_t)c.d_model * x->act) % 16 || ((size_t)x->qd * x->act) % 16)
      return false;
  }
  return true;
}

}  // namespace

isd_status isd_step_active(isd_ctx* x, int32_t n_active, int32_t* tokens, int32_t* n_commit, int32_t* n_accept,
                           void* stream) {
  if (!x || !tokens || !n_commit || !n_accept) return ISD_E_ARG;
  if (n_active < 1 || n_active > x->cfg.max_batch) return ISD_E_ARG;
  if (!x->prefilled) return ISD_E_STATE;
  return run_passes(x, n_active, 1, tokens, n_commit, n_accept, nullptr, (hipStream_t)stream);
}

isd_status isd_step(isd_ctx* x, int32_t* tokens, int32_t* n_commit, int32_t* n_accept, const isd_debug* debug,
                    void* stream) {
  if (!x || !tokens || !n_commit || !n_accept) return ISD_E_ARG;
  if (!debug_ok(x, debug)) return ISD_E_ARG;
  if (!x->prefilled) return ISD_E_STATE;
  return run_passes(x, x->cfg.max_batch, 1, tokens, n_commit, n_accept, debug, (hipStream_t)stream);
}

isd_status isd_step_n(isd_ctx* x, int32_t n_passes, int32_t* tokens, int32_t* n_commit, int32_t* n_accept,
                      void* stream) {
  if (!x || !tokens || !n_commit || !n_accept) return ISD_E_ARG;
  if (n_passes < 1 || n_passes > 64) return ISD_E_ARG;
  if (!x->prefilled) return ISD_E_STATE;
  return run_passes(x, x->cfg.max_batch, n_passes, tokens, n_commit, n_accept, nullptr, (hipStream_t)stream);
}

isd_status isd_set_graphs(isd_ctx* x, int32_t enable) {
  if (!x) return ISD_E_ARG;
  if (!enable) drop_graphs(x);
  x->graphs = enable != 0;
  return ISD_OK;
}

isd_status isd_set_meter(isd_ctx* x, int32_t enable) {
  if (!x) return ISD_E_ARG;
  if ((enable != 0) != x->meter) drop_graphs(x);   // the decide launch is captured by value
  x->meter = enable != 0;
  return ISD_OK;
}

isd_status isd_get_buffers(const isd_ctx* x, isd_buffers* out) {
  if (!x || !out) return ISD_E_ARG;
  out->slots = x->slots;
  out->page_table = x->page_table;
  out->max_pages_per_slot = x->max_pages;
  out->free_stack = x->free_stack;
  out->n_free = x->n_free;
  out->logits = x->logits[x->cur ^ 1];
  out->rows_per_slot = x->R;
  out->row_token = x->row_tok;
  out->row_pos = x->row_pos;
  out->k_pool = x->k_pool;
  out->v_pool = x->v_pool;
  out->attn_out = x->O;
  out->prefill_logits = x->logits[x->cur];
  out->row_off = x->row_off;
  out->row_len = x->row_len;
  return ISD_OK;
}

isd_status isd_get_status(isd_ctx* x, void* stream) {
  if (!x) return ISD_E_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return ISD_E_HIP;
  std::vector<isd_slot> h(x->cfg.max_batch);
  if (hipMemcpy(h.data(), x->slots, h.size() * sizeof(isd_slot), hipMemcpyDeviceToHost) != hipSuccess)
    return ISD_E_HIP;
  sticky_now(x);
  for (const auto& sl : h)
    if (sl.status != ISD_OK && x->sticky == ISD_OK) x->sticky = (isd_status)sl.status;
  return x->sticky;
}

isd_status isd_release(isd_ctx* x) {
  if (!x) return ISD_E_ARG;
  for (hipEvent_t e : x->ev_pool) hipEventDestroy(e);
  drop_graphs(x);
  if (x->cap_stream) hipStreamDestroy(x->cap_stream);
  if (x->sticky_host_h) hipHostFree(x->sticky_host_h);
  delete x;
  return ISD_OK;
}

isd_status isd_profile(isd_ctx* x, int32_t enable) {
  if (!x) return ISD_E_ARG;
  if (enable && x->ev_pool.empty()) {
    x->ev_pool.resize(kProfEvents);
    for (auto& e : x->ev_pool)
      if (hipEventCreate(&e) != hipSuccess) return ISD_E_HIP;
  }
  x->prof_on = enable != 0;
  return ISD_OK;
}

isd_status isd_profile_report(isd_ctx* x, isd_prof_entry* out, int32_t cap, int32_t* n) {
  if (!x || !n || (cap > 0 && !out)) return ISD_E_ARG;
  std::vector<isd_prof_entry> agg;
  if (!x->prof_recs.empty()) {
    if (hipEventSynchronize(x->ev_pool[x->prof_recs.back().second + 1]) != hipSuccess) return ISD_E_HIP;
  }
  for (const auto& r : x->prof_recs) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, x->ev_pool[r.second], x->ev_pool[r.second + 1]) != hipSuccess) return ISD_E_HIP;
    isd_prof_entry* e = nullptr;
    for (auto& a : agg)
      if (!strncmp(a.name, r.first, sizeof(a.name))) e = &a;
    if (!e) {
      agg.emplace_back();
      e = &agg.back();
      memset(e, 0, sizeof(*e));
      strncpy(e->name, r.first, sizeof(e->name) - 1);
    }
    e->launches += 1;
    e->total_ms += ms;
  }
  *n = (int32_t)agg.size();
  for (int i = 0; i < cap && i < (int)agg.size(); ++i) out[i] = agg[i];
  const bool overflow = x->prof_overflow;
  x->prof_recs.clear();
  x->ev_used = 0;
  x->prof_overflow = false;
  return overflow ? ISD_E_CAPACITY : ISD_OK;
}

size_t attn_paged_decode_workspace_bytes(const isd_attn_args* a) {
  if (!a) return 0;
  const int splits = cdiv(std::max(1, a->max_ctx), attn_split_len(a->batch, a->n_kv_heads, a->max_ctx));
  const size_t rows = (size_t)a->batch * a->rows;
  size_t off = 0;
  off = align_up(off + a->batch * sizeof(AttnItem));
  off = align_up(off + rows * 4);
  off = align_up(off + rows * 4);
  off = align_up(off + (size_t)splits * rows * a->n_q_heads * a->head_dim * 4);
  off = align_up(off + (size_t)splits * rows * a->n_q_heads * 2 * 4);
  return off;
}

isd_status attn_paged_decode(const isd_attn_args* a, void* stream) {
  if (!a || !a->q || !a->k_pool || !a->v_pool || !a->page_table || !a->ctx_len || !a->q_len || !a->out ||
      !a->workspace)
    return ISD_E_ARG;
  if (a->batch < 1 || a->rows < 1 || a->n_kv_heads < 1 || a->n_q_heads % a->n_kv_heads || a->max_ctx < 1)
    return ISD_E_ARG;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (a->head_dim != 128 || a->page_size != 16 || G * a->rows > 64) return ISD_E_SHAPE;
  const int split = attn_split_len(a->batch, a->n_kv_heads, a->max_ctx);
  const int splits = cdiv(a->max_ctx, split);
  const size_t rows = (size_t)a->batch * a->rows;
  char* w = (char*)a->workspace;
  size_t off = 0;
  AttnItem* items = (AttnItem*)(w + off);
  off = align_up(off + a->batch * sizeof(AttnItem));
  int32_t* row_pos = (int32_t*)(w + off);
  off = align_up(off + rows * 4);
  int32_t* row_slot = (int32_t*)(w + off);
  off = align_up(off + rows * 4);
  float* part_o = (float*)(w + off);
  off = align_up(off + (size_t)splits * rows * a->n_q_heads * a->head_dim * 4);
  float* part_ml = (float*)(w + off);
  hipStream_t s = (hipStream_t)stream;
  HIP_OK(launch_attn_setup(items, row_pos, row_slot, a->ctx_len, a->q_len, a->batch, a->rows, s));
  AttnArgs aa{};
  aa.q = a->q;
  aa.k_pool = a->k_pool;
  aa.v_pool = a->v_pool;
  aa.page_table = a->page_table;
  aa.max_pages = a->max_pages;
  aa.items = items;
  aa.n_items = a->batch;
  aa.ctx_len = a->ctx_len;
  aa.Hq = a->n_q_heads;
  aa.Hkv = a->n_kv_heads;
  aa.hd = a->head_dim;
  aa.P = a->page_size;
  aa.ncb = G * a->rows <= 32 ? 2 : 4;
  aa.split = split;
  aa.max_splits = splits;
  aa.part_o = part_o;
  aa.part_ml = part_ml;
  aa.part_rows = (int)rows;
  aa.out = a->out;
  aa.row_pos = row_pos;
  aa.row_slot = row_slot;
  aa.n_rows = (int)rows;
  HIP_OK(launch_attn_bf16(aa, s));
  HIP_OK(launch_attn_combine_bf16(aa, s));
  return ISD_OK;
}

int32_t isd_gemm_splits(int32_t N, int32_t K, int32_t swiglu) { return gemm_splits(N, K, swiglu != 0); }

isd_status isd_gemm(const isd_gemm_args* a, void* stream) {
  if (!a || !a->X || !a->W) return ISD_E_ARG;
  if (a->dtype != ISD_BF16 && a->dtype != ISD_F32) return ISD_E_ARG;
  if (a->mode < ISD_GEMM_STORE || a->mode > ISD_GEMM_SWIGLU) return ISD_E_ARG;
  if (a->M < 0 || a->N < 1 || a->K < 1 || a->splits < 0) return ISD_E_ARG;
  if (a->mode == ISD_GEMM_RESID ? !a->R : !a->Y) return ISD_E_ARG;
  if (a->mode == ISD_GEMM_SWIGLU && !a->W2) return ISD_E_ARG;
  if (a->path < GEMM_PATH_AUTO || a->path > GEMM_PATH_TILED2) return ISD_E_ARG;
  if (a->path == GEMM_PATH_SKINNY && a->M > kSkinnyMaxRows) return ISD_E_SHAPE;
  GemmArgs g = gargs(a->X, a->K, a->W, a->K, a->M, a->N, a->K, a->mode);
  g.B1 = a->W2;
  g.C = a->Y;
  g.ldc = a->N;
  g.R = a->R;
  g.ldr = a->N;
  g.path = a->path;
  if (a->norm_out) {
    if (a->mode != ISD_GEMM_RESID || !a->norm_g || !(a->norm_eps > 0.f) || a->N % 4) return ISD_E_ARG;
    g.norm_g = a->norm_g;
    g.norm_out = a->norm_out;
    g.norm_eps = a->norm_eps;
  }
  hipStream_t s = (hipStream_t)stream;
  if (a->dtype == ISD_F32) {
    HIP_OK(launch_gemm_f32(g, s));
    return ISD_OK;
  }
  if (a->K % 32 || a->N % 4) return ISD_E_SHAPE;
  const int S = a->splits ? a->splits : gemm_splits(a->N, a->K, a->mode == ISD_GEMM_SWIGLU);
  if ((a->K / 32) % S) return ISD_E_SHAPE;
  if (S > 1) {
    if (!a->workspace) return ISD_E_ARG;
    g.splits = S;
    g.part = (float*)a->workspace;
  }
  HIP_OK(launch_gemm_bf16(g, s));
  return ISD_OK;
}

size_t isd_packed_weight_bytes(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 16 || cols % 16) return 0;
  return packed_weight_elems(rows, cols) * sizeof(uint16_t);
}

isd_status isd_pack_weights(const void* src, void* dst, int32_t rows, int32_t cols, void* stream) {
  if (!src || !dst || src == dst) return ISD_E_ARG;
  if ((((uintptr_t)src) | ((uintptr_t)dst)) % 16) return ISD_E_ARG;
  if (rows < 1 || cols < 16 || cols % 16) return ISD_E_SHAPE;
  HIP_OK(launch_pack_weights(src, dst, rows, cols, (hipStream_t)stream));
  return ISD_OK;
}

size_t isd_sample_step_workspace_bytes(int32_t batch, int32_t rows, int32_t vocab, int32_t q_rows) {
  const int nc = cdiv(vocab, kStatChunk);
  return align_up((size_t)batch * rows * nc * sizeof(ChunkStat)) +
         align_up((size_t)std::max(1, q_rows) * nc * sizeof(ChunkStat));
}

}  // extern "C"

namespace {

// The acceptance step of isd_sample_step with its chunk statistics in `ws` (at least
// isd_sample_step_workspace_bytes of the arguments).
isd_status sample_step(const isd_sample_args* a, void* ws, hipStream_t s) {
  if (!a->slots || !a->logits || !a->tokens || !a->n_commit || !a->n_accept) return ISD_E_ARG;
  if (a->batch < 1 || a->stride_n < 1 || a->stride_n > ISD_MAX_STRIDE || a->vocab < 2 ||
      a->vocab > kStatChunk * 256 || !(a->temperature >= 0.f))
    return ISD_E_ARG;
  if (a->propose != ISD_PROPOSE_SAMPLE && a->propose != ISD_PROPOSE_ARGMAX) return ISD_E_ARG;
  if (a->propose == ISD_PROPOSE_SAMPLE && a->temperature > 0.f && (!a->q_logits || a->q_rows < 1)) return ISD_E_ARG;
  const int R = 2 * a->stride_n - 1, nc = cdiv(a->vocab, kStatChunk);
  char* w = (char*)ws;
  ChunkStat* st = (ChunkStat*)w;
  ChunkStat* qst = (ChunkStat*)(w + align_up((size_t)a->batch * R * nc * sizeof(ChunkStat)));
  HIP_OK(launch_row_stats(a->logits, a->batch * R, a->vocab, a->temperature, st, s));
  if (a->q_logits && a->q_rows > 0)
    HIP_OK(launch_row_stats(a->q_logits, a->q_rows, a->vocab, a->temperature, qst, s));
  SampleArgs sa{};
  sa.slots = a->slots;
  sa.n_slots = a->batch;
  sa.N = a->stride_n;
  sa.V = a->vocab;
  sa.propose = a->propose;
  sa.T = a->temperature;
  sa.seed = a->seed;
  sa.logits = a->logits;
  sa.rows_per_slot = R;
  sa.stats = st;
  sa.q_logits = a->q_logits;
  sa.q_stats = qst;
  sa.q_rows = a->q_rows;
  sa.n_chunks = nc;
  sa.tokens = a->tokens;
  sa.n_commit = a->n_commit;
  sa.n_accept = a->n_accept;
  sa.meter = a->meter != 0;
  sa.margins = a->margins;
  sa.kinds = a->kinds;
  HIP_OK(launch_decide(sa, s));
  return ISD_OK;
}

}  // namespace

extern "C" {

isd_status isd_sample_step(const isd_sample_args* a, void* stream) {
  if (!a || !a->workspace) return ISD_E_ARG;
  return sample_step(a, a->workspace, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// isd_sample_step_noalloc: the acceptance step with its chunk statistics in a file-scope
// device array instead of a caller workspace, for callers that cannot allocate.  Every GPU the
// library runs on holds one copy until the process ends; its address on a device is looked up
// once (hipGetSymbolAddress, with that device current) and kept.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> its copy of `scratch`

isd_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ISD_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ISD_E_HIP;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return ISD_OK;
}

}  // namespace

extern "C" {

isd_status isd_sample_step_noalloc(const isd_sample_args* a, void* stream) {
  if (!a || a->workspace) return ISD_E_ARG;
  if (a->batch < 1 || a->stride_n < 1 || a->stride_n > ISD_MAX_STRIDE || a->vocab < 2) return ISD_E_ARG;
  const size_t need = isd_sample_step_workspace_bytes(a->batch, 2 * a->stride_n - 1, a->vocab, a->q_rows);
  if (need > kNoAllocScratchBytes) return ISD_E_CAPACITY;
  void* ws = nullptr;
  const isd_status st = scratch_on_current_device(&ws);
  if (st != ISD_OK) return st;
  // the kernels write every statistic they read (row_stats before decide), so nothing in the
  // scratch has to start at zero
  return sample_step(a, ws, (hipStream_t)stream);
}

}  // extern "C"
