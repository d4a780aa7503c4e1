/*
 * isd.h - C ABI of the MI355X (gfx950) Introspective Strided Decoding library (libisd.so).
 *
 * Introspective Strided Decoding (ISD) is the decode step of a diffusion language model
 * whose attention stays strictly causal: one forward pass proposes new tokens at MASK
 * positions (distribution q) and re-scores the previously proposed, still pending tokens
 * under the anchor distribution p of the same pass; a pending token x is kept when
 * u < p(x)/q(x), and the first rejected pending token ends the accepted prefix of the pass:
 * the next block resumes from its position (Bud's Wiki note "Introspective Diffusion
 * Language Models", sections Key claims and Method; Agentic Commons post of the same title,
 * section "How Introspective Strided Decoding Works").  R-ISD adds a rank-r LoRA that is
 * active only at MASK positions, so verify positions keep the base weights and the output
 * equals the base AR model's (wiki note, Key claims; GeekNews summaries, section Lossless
 * R-ISD).
 *
 * Conventions for every call:
 *  - Pointers named "device" are device (HBM) addresses on the current HIP device,
 *    "host" are host addresses.  The library allocates NO device memory: weights, the KV
 *    pool, the workspace and all outputs belong to the caller and must stay valid for the
 *    lifetime of the context.  isd_release frees host metadata only (including the one
 *    pinned host word that carries the sticky device status).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls enqueue
 *    work on it and return; outputs are valid once the stream has completed that work.
 *    A context is not thread-safe; use one stream per context.
 *  - Host-side validation failures return a negative isd_status synchronously and enqueue
 *    nothing.  Device-side conditions (non-finite logits, a KV pool found empty on the
 *    device) are recorded per slot in isd_slot.status, and the first one of the context is
 *    kept as its sticky status: isd_prefill / isd_step / isd_step_active / isd_step_n enqueue
 *    their work and then return the sticky status the device has reported so far (ISD_OK
 *    while there is none; passes still in flight may report later), and isd_get_status()
 *    synchronizes the stream and returns it definitively.  ISD_E_NONFINITE is only ever a
 *    device status; ISD_E_CAPACITY and ISD_E_STATE are also host refusals of a call, and
 *    isd_get_status tells the two apart (it reports device statuses only).
 *  - Matrices are row-major.  "act" is the activation/storage type of the context:
 *    bfloat16 (ISD_BF16) or float (ISD_F32).  Weight matrices are stored out x in
 *    (y = x W^T).
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISD_MAX_STRIDE 8          /* largest supported stride N */
#define ISD_DEBUG_MAX_ROWS 64     /* rows one isd_debug record can follow */

typedef enum {
  ISD_OK = 0,
  ISD_E_ARG = -1,        /* NULL pointer, bad enum value, out-of-range scalar */
  ISD_E_SHAPE = -2,      /* model/config shape the kernels do not support */
  ISD_E_CAPACITY = -3,   /* KV page pool, prefill row budget or batch too small */
  ISD_E_STATE = -4,      /* call not valid in the context's current state */
  ISD_E_HIP = -5,        /* a HIP runtime call failed */
  ISD_E_NONFINITE = -6   /* non-finite logits were seen by the sampler (sticky) */
} isd_status;

enum { ISD_F32 = 0, ISD_BF16 = 1 };
enum { ISD_PROPOSE_SAMPLE = 0, ISD_PROPOSE_ARGMAX = 1 };
enum { ISD_SLOT_EMPTY = 0, ISD_SLOT_A = 1, ISD_SLOT_B = 2, ISD_SLOT_DONE = 3 };
/* kinds of the decisions of one pass, in the order a slot takes them (isd_debug.kinds) */
enum { ISD_DEC_ACCEPT = 0, ISD_DEC_RESID = 1, ISD_DEC_Z1 = 2, ISD_DEC_PROPOSE = 3 };

/* Model + decoding configuration.
 * Model: pre-norm causal decoder (RMSNorm, RoPE rotate-half with base rope_base, grouped
 * query attention, SwiGLU FFN, untied LM head, no biases).  The MASK token id is `vocab`
 * and indexes row `vocab` of the (vocab+1)-row embedding table.
 * Decoding: stride_n = N (1 = plain AR); temperature 0 = greedy; `propose` selects how the
 * MASK rows propose (sample from q, or argmax with q := delta); seed keys the Philox4x32-10
 * stream u(slot, t, position, purpose). */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rope_base, rms_eps;
  int32_t dtype;               /* ISD_F32 | ISD_BF16 */
  int32_t stride_n;            /* 1 .. ISD_MAX_STRIDE */
  int32_t page_size;           /* tokens per KV page: 16 */
  int32_t max_batch;           /* number of slots */
  int32_t max_seq_len;         /* prompt + generated tokens of any slot */
  int32_t n_pages;             /* pages in the KV pool */
  int32_t max_prefill_tokens;  /* largest sum of prompt lengths of one isd_prefill call */
  int32_t lora_rank;           /* 0 = ISD, >0 = R-ISD gated LoRA of that rank (multiple of 64) */
  int32_t propose;             /* ISD_PROPOSE_SAMPLE | ISD_PROPOSE_ARGMAX */
  float temperature;           /* >= 0 */
  uint64_t seed;
} isd_config;

/* Device pointers of the weights (act type).  The per-layer fields are HOST arrays of
 * n_layers device pointers; they are copied by isd_init.
 *   embed [vocab+1, d]      final_norm [d]        lm_head [vocab, d]
 *   attn_norm[l] [d]        wqkv[l] [(Hq+2Hkv)*hd, d] (q rows, then k, then v)
 *   wo[l] [d, Hq*hd]        ffn_norm[l] [d]
 *   wg[l], wu[l] [F, d]     wd[l] [d, F]
 *   lora_a[l*7+m] [r, d_in_m], lora_b[l*7+m] [d_out_m, r] for m = q,k,v,o,g,u,d
 *   (HOST arrays of n_layers*7 device pointers; NULL when lora_rank == 0).
 * The matrices are out x in.  With ISD_BF16 the projection matrices (lm_head, wqkv, wo, wg,
 * wu, wd, lora_a, lora_b) are in the packed operand layout made by isd_pack_weights; embed and
 * the norm gains, and every matrix of ISD_F32, are row-major.  The LoRA matrices of q, k, v
 * (and of gate, up) may be stored back to back (packed): the library then runs each group's
 * products as one. */
typedef struct {
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* wg;
  const void* const* wu;
  const void* const* wd;
  const void* const* lora_a;
  const void* const* lora_b;
} isd_weights;

typedef struct {
  size_t kv_pool_bytes;    /* K pool then V pool, every layer */
  size_t workspace_bytes;  /* activations, logits, sampler state, page tables, slots */
} isd_sizes;

/* Per-slot device state (array of max_batch in the workspace; layout fixed, 128 bytes). */
typedef struct {
  int32_t state;                         /* ISD_SLOT_* */
  int32_t L;                             /* cached tokens (positions 0 .. L-1 in the pages) */
  int32_t c;                             /* newest committed token, not yet cached */
  int32_t t;                             /* pass counter of the Philox stream (prefill = 0) */
  int32_t n_gen, max_new;                /* generated tokens so far / stop after max_new */
  int32_t n_pages;                       /* pages in this slot's page table */
  int32_t status;                        /* 0, ISD_E_NONFINITE, ISD_E_CAPACITY (KV pool empty)
                                            or ISD_E_STATE (live past isd_step_active's n_active) */
  int32_t pending[ISD_MAX_STRIDE - 1];   /* v_1 .. v_{N-1} awaiting verification (state A) */
  int32_t q_row[ISD_MAX_STRIDE - 1];     /* logits row (previous pass) that proposed pending[i];
                                            -1: delta q (argmax proposal) */
  int32_t passes, accepted, verified, committed;   /* cumulative counters */
  double meter_sum;                      /* introspective acceptance meter (isd_set_meter): sum of */
  int32_t meter_n;                       /* the acceptance probabilities of meter_n re-scored tokens */
  int32_t pad[3];
} isd_slot;

typedef struct isd_ctx isd_ctx;

/* Device addresses of the context's internal buffers (for tests and benchmarks). */
typedef struct {
  isd_slot* slots;          /* [max_batch] */
  int32_t* page_table;      /* [max_batch, max_pages_per_slot] */
  int32_t max_pages_per_slot;
  int32_t* free_stack;      /* [n_pages], entries 0 .. n_free-1 */
  int32_t* n_free;          /* [1] */
  float* logits;            /* logits of the last pass: [max_batch * (2N-1), vocab] fp32 in the
                               pass's packed row order: row row_off[b] + i is row i of slot b's
                               block, i < row_len[b] (the live rows of all slots come first, slot
                               by slot; the rows after them are dead) */
  int32_t rows_per_slot;    /* 2N-1 */
  int32_t* row_token;       /* [max_batch*(2N-1)] input token of each packed row of the last pass */
  int32_t* row_pos;         /* [max_batch*(2N-1)] position (-1 for a dead row) */
  void* k_pool;             /* [n_layers][n_pages][Hkv][P][hd] act */
  void* v_pool;             /* [n_layers][n_pages][Hkv][hd][P] act (transposed within a page) */
  void* attn_out;           /* last layer's attention output of the last pass [rows, Hq*hd] act */
  float* prefill_logits;    /* logits of the last isd_prefill call, row i = the last prompt row
                               of its i-th slot [n, vocab] fp32; valid until the next pass */
  int32_t* row_off;         /* [max_batch] first packed row of each slot's block in the last pass */
  int32_t* row_len;         /* [max_batch] its live rows: 2N-1 (state A), N (state B) or 0 */
} isd_buffers;

/* Debug surface of one pass (isd_step's `debug`; NULL = off), for the parity harness: the
 * per-layer quantities the pages' pass computes (wiki note, Method: one causal forward over
 * the block's rows, the anchor and proposal distributions read from its logits), recorded for
 * a chosen list of the pass's rows, and every slot's decisions with their margins.
 *   n_rows       rows followed, 0 .. ISD_DEBUG_MAX_ROWS
 *   rows         device [n_rows] int32: pass rows (slot b's block row i is b*(2N-1)+i)
 *   layer_in     device [n_layers+1, n_rows, d_model] fp32: the residual stream entering
 *                layer l; entry n_layers is the residual after the last layer
 *   layer_attn   device [n_layers, n_rows, Hq*head_dim] act: attention output of layer l
 *                (the input of its O projection)
 *   final_normed device [n_rows, d_model] act: RMSNorm of the final residual times
 *                final_norm, the LM head's input
 *   margins      device [max_batch, 2N] double, nullable: margin of the slot's j-th decision
 *                of the pass: |u - min(1, p/q)| for an acceptance test; for a categorical
 *                draw the distance of u*S to the nearest edge of the drawn token's interval
 *                of the cumulative weights, divided by S; for an argmax decision (T = 0 or an
 *                argmax proposal) the gap between the two largest logits of the row;
 *                +inf for the meter's untested commits; -1 past the last decision
 *   kinds        device [max_batch, 2N] int32, nullable: ISD_DEC_* of decision j, -1 past
 *                the last (order: the acceptance tests, then the residual draw, or z1 and the
 *                proposals)
 * Any of layer_in / layer_attn / final_normed may be NULL (not recorded).  A pass with a
 * debug record is launched kernel by kernel (never from a captured graph); its results are
 * identical to a pass without one. */
typedef struct {
  int32_t n_rows;
  const int32_t* rows;
  float* layer_in;
  void* layer_attn;
  void* final_normed;
  double* margins;
  int32_t* kinds;
} isd_debug;

/* Create a context.  With kv_pool == workspace == NULL only `sizes` is filled (size query)
 * and *out is set to NULL.  Otherwise kv_pool/workspace must hold at least the queried
 * sizes (256-byte aligned) and set-up kernels (free stack, slot reset, RoPE tables) are
 * enqueued on `stream` (an argument the set-up needs: the context has no stream of its own).
 * The pages give no API; the calls follow their statement of the problem: an AR-compatible
 * prefill, then ISD passes that commit tokens and roll the paged KV cache back on a
 * rejection (wiki note, TL;DR and Method; GeekNews, Serving).  HIP graph replay of the
 * passes is on by default (see isd_set_graphs).
 * Errors: ISD_E_ARG (NULL cfg/w/sizes/out, bad enum), ISD_E_SHAPE (unsupported dims:
 * head_dim must be 128 for bf16 and <= 256 for f32, Hq a multiple of Hkv, d/F/qkv widths
 * multiples of 64 for bf16), ISD_E_HIP. */
isd_status isd_init(const isd_config* cfg, const isd_weights* w, void* kv_pool, void* workspace,
                    isd_sizes* sizes, isd_ctx** out, void* stream);

/* Prefill n slots with their prompts (an ordinary causal AR prefill, the pages' "AR-compatible
 * serving": wiki note, TL;DR; GeekNews, Serving), sample each slot's first token from the last
 * prompt row with u(slot, 0, prompt_len, 1), and put the slot in state B (DONE if
 * max_new <= 1).
 *   slots      host [n]   distinct slot ids in [0, max_batch)
 *   prompt_ids device [offsets[n]] int32 tokens in [0, vocab), prompts packed back to back
 *   offsets    host [n+1] prompt i is prompt_ids[offsets[i] .. offsets[i+1]), length >= 1
 *   max_new    host [n]   tokens to generate (>= 1), including the first token
 *   first_tok  device [n] int32 out: the first generated token of each slot
 * Pages: in call order each slot frees its old pages then takes ceil(len/P) pages.
 * Admission: ceil((len + max_new + 2N)/P) pages are reserved per slot so that isd_step can
 * never run out; ISD_E_CAPACITY when the reservations exceed the pool, when offsets[n] >
 * max_prefill_tokens or len + max_new + 2N > max_seq_len.  ISD_E_ARG on bad slots/lengths.
 * Returns the sticky device status after enqueuing (see the conventions above). */
isd_status isd_prefill(isd_ctx* ctx, int32_t n, const int32_t* slots, const int32_t* prompt_ids,
                       const int32_t* offsets, const int32_t* max_new, int32_t* first_tok,
                       void* stream);

/* One ISD pass over every live slot (state A or B), the pages' decode step (wiki note, Key
 * claims and Method: one forward pass proposes N tokens at MASK positions and re-scores the
 * N-1 pending ones, accepted with probability min(1, p/q), the residual max(0, p - q) drawn at
 * the first rejection; Agentic Commons, "How Introspective Strided Decoding Works"): assemble
 * the block rows from device state, reserve KV pages, run the causal forward (LoRA on MASK
 * rows when lora_rank > 0), verify / accept / resample / propose, and roll the KV cache back
 * to the committed length.  The rows are packed on the device: A-state slots 2N-1 rows,
 * B-state slots N, finished or empty slots none, slot after slot; the projections and the
 * sampler's statistics skip the rows past the live ones (the pages' continuous batching:
 * wiki note, TL;DR and Key claims).  A slot's results do not depend on the packing.
 *   tokens   device [max_batch, N] int32 out: tokens committed this pass (-1 padded)
 *   n_commit device [max_batch]    int32 out: number of tokens committed this pass
 *   n_accept device [max_batch]    int32 out: pending tokens accepted this pass
 *   debug    host, nullable: an isd_debug record filled by this pass (see isd_debug)
 * Slots that are EMPTY or DONE commit nothing.  No host synchronization happens inside.
 * Errors: ISD_E_STATE if no slot was ever prefilled, ISD_E_ARG on NULL outputs or a bad
 * debug record (nothing enqueued).  Otherwise the sticky device status after enqueuing. */
isd_status isd_step(isd_ctx* ctx, int32_t* tokens, int32_t* n_commit, int32_t* n_accept,
                    const isd_debug* debug, void* stream);

/* isd_step over the slots 0 .. n_active-1 only (1 <= n_active <= max_batch): the block rows,
 * attention items, LoRA MASK rows and decisions of the later slots are not computed, so a
 * partly filled context (a serving loop that admits requests into the lowest free slots and
 * passes the highest live slot + 1) pays for its live slots only - the pages' stationary
 * batch with admission and retirement between passes (wiki note, Key claims; GeekNews,
 * Serving).  Every kernel computes a slot's rows from those rows alone, so a slot's tokens
 * are bit-identical to the ones isd_step gives it.  Slots at or past n_active must be EMPTY
 * or DONE: a live one there is not advanced and gets isd_slot.status = ISD_E_STATE.  The
 * outputs of those slots are not written.  With graphs enabled, one graph is captured per
 * (buffer parity, n_active).
 * Errors: ISD_E_ARG (NULL outputs, n_active out of range), ISD_E_STATE (nothing prefilled);
 * otherwise the sticky device status after enqueuing. */
isd_status isd_step_active(isd_ctx* ctx, int32_t n_active, int32_t* tokens, int32_t* n_commit,
                           int32_t* n_accept, void* stream);

/* n_passes consecutive isd_step passes, the pages' stationary-batch decode loop (wiki note,
 * Key claims: CUDA-graph capture and a stationary batch as the serving-stack gains): with
 * graphs enabled the whole run of passes is one graph launch (captured once per (buffer
 * parity, n_passes)), so the host does no per-pass work.
 *   tokens   device [n_passes, max_batch, N], n_commit / n_accept device [n_passes, max_batch]:
 *            pass i writes the i-th slice, as isd_step writes its outputs
 * Results are identical to n_passes calls of isd_step.  1 <= n_passes <= 64.
 * Errors: as isd_step (ISD_E_ARG also for n_passes out of range). */
isd_status isd_step_n(isd_ctx* ctx, int32_t n_passes, int32_t* tokens, int32_t* n_commit,
                      int32_t* n_accept, void* stream);

/* Replay the passes from HIP graphs (enable != 0, the default) instead of launching their
 * kernels one by one, the serving-loop measure the pages credit with the largest throughput
 * gain (wiki note, Key claims; GeekNews, Serving).  A pass's launch sequence depends only on
 * the configuration and on which of the two logits buffers it writes (and, for
 * isd_step_active, on n_active; for isd_step_n, on n_passes), so the library captures it
 * once per such key (on an internal stream, at the first such call) and then launches the
 * graph on the caller's stream.  Results are identical to eager launches.  A graph is
 * re-captured when the call receives different output pointers; profiling (isd_profile) and
 * debug passes launch eagerly.  enable = 0 frees the graphs.  Errors: ISD_E_ARG, ISD_E_HIP. */
isd_status isd_set_graphs(isd_ctx* ctx, int32_t enable);

/* Device addresses of internal buffers (see isd_buffers).  Errors: ISD_E_ARG. */
isd_status isd_get_buffers(const isd_ctx* ctx, isd_buffers* out);

/* Synchronize `stream` and return the sticky device status: ISD_OK, or the first non-zero
 * isd_slot.status reported (ISD_E_NONFINITE, ISD_E_CAPACITY, ISD_E_STATE). */
isd_status isd_get_status(isd_ctx* ctx, void* stream);

/* Free the host-side context. */
isd_status isd_release(isd_ctx* ctx);

/* Kernel timing for benchmarks.  isd_profile(ctx, 1) starts recording a HIP event pair
 * around every kernel the context launches (on the launch stream); isd_profile(ctx, 0) stops.
 * isd_profile_report synchronizes the recorded events and returns, per kernel name, the
 * number of launches and their summed duration, then clears the record.  At most `cap`
 * entries are written; *n receives the number of distinct names.  Recording is bounded
 * (ISD_E_CAPACITY from isd_step/isd_prefill when the event pool is exhausted). */
typedef struct {
  char name[32];
  int32_t launches;
  double total_ms;
} isd_prof_entry;

isd_status isd_profile(isd_ctx* ctx, int32_t enable);
isd_status isd_profile_report(isd_ctx* ctx, isd_prof_entry* out, int32_t cap, int32_t* n);

/* ---------------------------------------------------------------------------------------
 * Kernel-level entry points (used by the attention + acceptance microbench).
 * ------------------------------------------------------------------------------------- */

/* Paged causal attention of blocks of query rows (wiki note, TL;DR: attention stays strictly
 * causal; the block's own keys are read from the pages, as a paged-only kernel does; wiki
 * note, Key claims: paged-only attention as a serving gain).
 *   q          device [B, R, Hq, hd] bf16, query rows after RoPE; row i of sequence b sits
 *              at position ctx_len[b] - q_len[b] + i
 *   k_pool     device [n_pages, Hkv, P, hd] bf16;  v_pool device [n_pages, Hkv, hd, P] bf16
 *   page_table device [B, max_pages] int32;  ctx_len, q_len device [B] int32
 *              (keys 0 .. ctx_len-1 are in the pages; q_len <= R)
 *   out        device [B, R, Hq, hd] bf16 (rows >= q_len are written as zeros)
 *   workspace  device, at least attn_paged_decode_workspace_bytes(...) bytes
 * head_dim must be 128, page_size 16, Hq/Hkv * R <= 64.  Errors: ISD_E_ARG, ISD_E_SHAPE. */
typedef struct {
  int32_t batch, rows, n_q_heads, n_kv_heads, head_dim, page_size, max_pages, max_ctx;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;
  const int32_t* ctx_len;
  const int32_t* q_len;
  void* out;
  void* workspace;
} isd_attn_args;

size_t attn_paged_decode_workspace_bytes(const isd_attn_args* a);
isd_status attn_paged_decode(const isd_attn_args* a, void* stream);

/* The fused vocabulary-wide acceptance step for a batch of slots, as inside isd_step
 * (wiki note, Method: accept when u < p(x)/q(x); Agentic Commons, "How Introspective
 * Strided Decoding Works": speculative-sampling rule; residual draw from
 * normalize(max(0, p - q)) on the first rejection).
 *   slots      device [B] isd_slot, in/out (state machine as in isd_step; L, c, t advance)
 *   logits     device [B, R, V] fp32, the current pass (R = 2N-1 rows per slot)
 *   q_logits   device [B*R', V] fp32 rows named by slots[b].q_row (the previous pass),
 *              may be NULL in argmax mode
 *   q_rows     number of rows of q_logits (bounds check of q_row)
 *   tokens/n_commit/n_accept  device outputs as in isd_step
 *   workspace  device, at least isd_sample_step_workspace_bytes(B, R, V, q_rows) bytes
 *   margins, kinds  device [B, 2N], nullable: the decisions and their margins as in isd_debug
 * The slot ids used in the Philox counters are the array indices b.  Page tables are not
 * touched.  Non-finite logits in a row a slot needs end that slot: state DONE, status
 * ISD_E_NONFINITE, nothing committed; the other slots are unaffected.  Errors: ISD_E_ARG. */
typedef struct {
  int32_t batch, stride_n, vocab, propose, q_rows;
  float temperature;
  uint64_t seed;
  isd_slot* slots;
  const float* logits;
  const float* q_logits;
  int32_t* tokens;
  int32_t* n_commit;
  int32_t* n_accept;
  void* workspace;
  int32_t meter;           /* 1: introspective acceptance meter mode (see isd_set_meter) */
  double* margins;
  int32_t* kinds;
} isd_sample_args;

size_t isd_sample_step_workspace_bytes(int32_t batch, int32_t rows, int32_t vocab, int32_t q_rows);
isd_status isd_sample_step(const isd_sample_args* a, void* stream);

/* isd_sample_step for callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with the chunk statistics in a fixed scratch array of 8 MiB that the
 * library holds on every GPU it runs on until the process ends.  a->workspace must be NULL.
 * The call allocates nothing: no hipMalloc or hipFree, no allocating library routine.  Every
 * call on one GPU shares that GPU's scratch, so calls that overlap on one GPU (different
 * streams, or threads) race; calls in one stream are ordered.  Limit: isd_sample_step_workspace_
 * bytes(batch, 2N-1, vocab, q_rows) <= 8 MiB (e.g. 64 slots x 7 rows and 448 previous rows at
 * vocab 151936 need 0.8 MiB).  Errors: ISD_E_ARG (as isd_sample_step, or a non-NULL workspace),
 * ISD_E_CAPACITY (beyond the scratch size), ISD_E_HIP. */
isd_status isd_sample_step_noalloc(const isd_sample_args* a, void* stream);

/* Introspective acceptance meter (wiki note, TL;DR and Key claims: the introspective
 * acceptance rate - whether a model accepts, under argmax or sampling, its own previously
 * generated tokens when it re-evaluates them; AR models ~0.98).  With the meter on, every
 * pending token of an A-state pass - the model's own proposal from the previous pass - is
 * committed without a test (teacher forcing of the model's own generation, so that no
 * rejection cuts the block short) and re-scored by the pass's anchor distribution: the slot
 * adds its acceptance probability to meter_sum and 1 to meter_n.  The probability is
 * min(1, p(x)/q(x)) for a sampled proposal, p(x) for an argmax proposal (q = delta), and
 * [x == argmax p] at temperature 0.  Off (default): ordinary ISD.  Changing it drops
 * captured graphs.  Errors: ISD_E_ARG. */
isd_status isd_set_meter(isd_ctx* ctx, int32_t enable);

/* Packed operand layout of the bf16 projection weights (the MFMA B operands of the GEMMs,
 * one contiguous kilobyte per 32x32x16 product): W [rows, cols] row-major bf16 becomes
 * ceil(rows/32) x (cols/16) blocks of 64 x 8 elements, block (nb, kb) at element
 * (nb * cols/16 + kb) * 512, whose lane-l part (8 elements) is row 32 nb + l%32, columns
 * 16 kb + 8 (l/32) .. + 7; rows past `rows` are zero.  (A storage layout of this library;
 * the pages fix none.)
 * isd_packed_weight_bytes: bytes of the packed matrix (0 if cols is not a positive multiple
 * of 16 or rows < 1).  isd_pack_weights: converts src (device, row-major [rows, cols]) into
 * dst (device, caller-owned, isd_packed_weight_bytes); both 16-byte aligned, not overlapping;
 * enqueued on stream.  Errors: ISD_E_ARG (pointers), ISD_E_SHAPE (sizes), ISD_E_HIP. */
size_t isd_packed_weight_bytes(int32_t rows, int32_t cols);
isd_status isd_pack_weights(const void* src, void* dst, int32_t rows, int32_t cols, void* stream);

/* One projection of the decode step (wiki note, Key claims: decode of a causal transformer,
 * weight streaming in the memory-bound regime): Y = X W^T (X [M, K] row-major, W [N, K],
 * i.e. out x in) in the context's arithmetic, as isd_step runs it.
 *   dtype    ISD_BF16 (MFMA path, X bf16 row-major, W and W2 bf16 packed by isd_pack_weights)
 *            or ISD_F32 (W row-major)
 *   mode     ISD_GEMM_STORE: Y act [M, N]; ISD_GEMM_STORE_F32: Y float [M, N];
 *            ISD_GEMM_RESID: R float [M, N] += X W^T;
 *            ISD_GEMM_SWIGLU: Y act [M, N] = silu(X W^T) * (X W2^T), W2 [N, K]
 *   splits   split-K factor (bf16 only): 0 = the rule isd_step uses (a function of N and K)
 *   workspace device fp32 [splits, M, N (x2 for SwiGLU)] when splits > 1, else unused
 *   norm_g, norm_out  ISD_GEMM_RESID only, optional (NULL = off): after the residual update,
 *            norm_out [M, N] act = RMSNorm(R row) * norm_g, eps norm_eps (as isd_step fuses
 *            the next block's input norm into the O and down projections)
 *   path     bf16 kernel: 0 = automatic (the skinny kernel up to 32 rows, up to 64 when
 *            N > 65536, else the tiled one), 1 = tiled, 2 = skinny (M <= 128 only),
 *            3 / 4 / 5 = tiled with 4 / 3 / 2 waves per workgroup (0 and 1 choose the count
 *            that fills the CUs best).  Every kernel accumulates each output element in the
 *            same order, so the choice never changes the result.
 * K must be a multiple of 32 and N of 4 for bf16.  Errors: ISD_E_ARG, ISD_E_SHAPE. */
enum { ISD_GEMM_STORE = 0, ISD_GEMM_STORE_F32 = 1, ISD_GEMM_RESID = 2, ISD_GEMM_SWIGLU = 3 };
typedef struct {
  int32_t dtype, mode, M, N, K, splits;
  const void* X;
  const void* W;
  const void* W2;
  void* Y;
  float* R;
  void* workspace;
  const void* norm_g;
  void* norm_out;
  float norm_eps;
  int32_t path;
} isd_gemm_args;

int32_t isd_gemm_splits(int32_t N, int32_t K, int32_t swiglu);
isd_status isd_gemm(const isd_gemm_args* a, void* stream);

/* Library version string. */
const char* isd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ISD_H */
