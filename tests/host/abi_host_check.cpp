// Host-side checks of libisd's C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only): size queries, configuration validation
// and argument checks of every entry point, including the paths that build and free a
// context's host metadata.  None of them reaches a HIP runtime call or a kernel launch, so
// the program runs without a GPU.  Exit status 0 and "abi host checks passed" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "isd.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static isd_config cfg_8b() {
  isd_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 36;
  c.d_model = 4096;
  c.n_q_heads = 32;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.d_ffn = 12288;
  c.vocab = 151936;
  c.rope_base = 1e4f;
  c.rms_eps = 1e-6f;
  c.dtype = ISD_BF16;
  c.stride_n = 4;
  c.page_size = 16;
  c.max_batch = 64;
  c.max_seq_len = 2064;
  c.n_pages = 64 * 130;
  c.max_prefill_tokens = 16384;
  c.lora_rank = 0;
  c.propose = ISD_PROPOSE_ARGMAX;
  c.temperature = 1.f;
  c.seed = 1;
  return c;
}

int main() {
  CHECK(std::strncmp(isd_version(), "isd-mi355x", 10) == 0);

  // size queries
  isd_sizes sz;
  isd_ctx* ctx = reinterpret_cast<isd_ctx*>(0x1);
  isd_config c = cfg_8b();
  CHECK(isd_init(&c, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == ISD_OK);
  CHECK(ctx == nullptr);
  CHECK(sz.kv_pool_bytes == 2ull * 36 * 64 * 130 * 8 * 16 * 128 * 2);
  CHECK(sz.workspace_bytes > 2ull * 64 * 7 * 151936 * 4);
  for (int N = 1; N <= ISD_MAX_STRIDE; ++N) {
    c = cfg_8b();
    c.stride_n = N;
    c.lora_rank = (N % 2) ? 128 : 0;
    CHECK(isd_init(&c, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == ISD_OK);
  }
  c = cfg_8b();
  c.dtype = ISD_F32;
  c.head_dim = 32;
  c.n_layers = 2;
  c.d_model = 128;
  c.n_q_heads = 4;
  c.n_kv_heads = 4;
  c.d_ffn = 512;
  c.vocab = 1024;
  c.max_batch = 2;
  c.max_seq_len = 96;
  c.n_pages = 16;
  c.max_prefill_tokens = 64;
  CHECK(isd_init(&c, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == ISD_OK);
  CHECK(sz.kv_pool_bytes == 2ull * 2 * 16 * 4 * 16 * 32 * 4);

  // configuration validation
  struct Bad {
    int field;
    int value;
    isd_status code;
  };
  const Bad bad[] = {{0, 64, ISD_E_SHAPE}, {1, 32, ISD_E_SHAPE}, {2, 7, ISD_E_SHAPE}, {3, 0, ISD_E_ARG},
                     {3, 9, ISD_E_ARG},    {4, 5, ISD_E_ARG},    {5, 100, ISD_E_SHAPE}, {6, 3, ISD_E_ARG},
                     {7, 0, ISD_E_ARG},    {8, -1, ISD_E_ARG}};
  for (const Bad& b : bad) {
    c = cfg_8b();
    int* f[] = {&c.head_dim, &c.page_size, &c.n_kv_heads, &c.stride_n, &c.dtype, &c.lora_rank, &c.propose,
                &c.max_batch, &c.n_layers};
    *f[b.field] = b.value;
    CHECK(isd_init(&c, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == b.code);
  }
  c = cfg_8b();
  c.temperature = -1.f;
  CHECK(isd_init(&c, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(isd_init(nullptr, nullptr, nullptr, nullptr, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(isd_init(&c, nullptr, nullptr, nullptr, nullptr, &ctx, nullptr) == ISD_E_ARG);

  // binding checks that build (and free) a context's host metadata before any HIP call:
  // misaligned buffers, missing weights, a missing per-layer or LoRA pointer
  c = cfg_8b();
  alignas(256) static char fake[512];
  std::vector<const void*> layer(c.n_layers, fake), lora((size_t)c.n_layers * 7, fake);
  isd_weights w;
  w.embed = w.final_norm = w.lm_head = fake;
  w.attn_norm = w.wqkv = w.wo = w.ffn_norm = w.wg = w.wu = w.wd = layer.data();
  w.lora_a = w.lora_b = nullptr;
  CHECK(isd_init(&c, &w, fake + 1, fake, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(isd_init(&c, nullptr, fake, fake, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(isd_init(&c, &w, fake, nullptr, &sz, &ctx, nullptr) == ISD_E_ARG);
  std::vector<const void*> holey(layer);
  holey[c.n_layers - 1] = nullptr;
  w.wd = holey.data();
  CHECK(isd_init(&c, &w, fake, fake, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(ctx == nullptr);
  w.wd = layer.data();
  c.lora_rank = 128;
  CHECK(isd_init(&c, &w, fake, fake, &sz, &ctx, nullptr) == ISD_E_ARG);   // no LoRA arrays
  std::vector<const void*> holey_lora(lora);
  holey_lora[5] = nullptr;
  w.lora_a = lora.data();
  w.lora_b = holey_lora.data();
  CHECK(isd_init(&c, &w, fake, fake, &sz, &ctx, nullptr) == ISD_E_ARG);
  CHECK(ctx == nullptr);

  // the other entry points' argument checks
  int32_t i32[8] = {0};
  CHECK(isd_prefill(nullptr, 1, i32, i32, i32, i32, i32, nullptr) == ISD_E_ARG);
  CHECK(isd_step(nullptr, i32, i32, i32, nullptr, nullptr) == ISD_E_ARG);
  CHECK(isd_step_active(nullptr, 1, i32, i32, i32, nullptr) == ISD_E_ARG);
  CHECK(isd_step_n(nullptr, 2, i32, i32, i32, nullptr) == ISD_E_ARG);
  CHECK(isd_set_graphs(nullptr, 1) == ISD_E_ARG);
  CHECK(isd_set_meter(nullptr, 1) == ISD_E_ARG);
  CHECK(isd_get_buffers(nullptr, nullptr) == ISD_E_ARG);
  CHECK(isd_get_status(nullptr, nullptr) == ISD_E_ARG);
  CHECK(isd_release(nullptr) == ISD_E_ARG);
  CHECK(isd_profile(nullptr, 1) == ISD_E_ARG);
  int32_t n = 0;
  CHECK(isd_profile_report(nullptr, nullptr, 0, &n) == ISD_E_ARG);

  CHECK(isd_packed_weight_bytes(4096, 4096) == 4096ull * 4096 * 2);
  CHECK(isd_packed_weight_bytes(33, 16) == 64ull * 16 * 2);
  CHECK(isd_packed_weight_bytes(0, 16) == 0 && isd_packed_weight_bytes(32, 24) == 0);
  CHECK(isd_pack_weights(nullptr, fake, 32, 16, nullptr) == ISD_E_ARG);
  CHECK(isd_pack_weights(fake, fake, 32, 16, nullptr) == ISD_E_ARG);
  CHECK(isd_pack_weights(fake, fake + 256, 32, 24, nullptr) == ISD_E_SHAPE);
  CHECK(isd_pack_weights(fake + 1, fake + 256, 32, 16, nullptr) == ISD_E_ARG);

  CHECK(isd_gemm_splits(4096, 4096, 0) == 8);
  CHECK(isd_gemm_splits(6144, 4096, 0) == 4);
  CHECK(isd_gemm_splits(12288, 4096, 1) == 1);
  isd_gemm_args g;
  std::memset(&g, 0, sizeof g);
  CHECK(isd_gemm(nullptr, nullptr) == ISD_E_ARG);
  CHECK(isd_gemm(&g, nullptr) == ISD_E_ARG);
  g.X = g.W = g.Y = fake;
  g.dtype = ISD_BF16;
  g.M = 4;
  g.N = 64;
  g.K = 48;                                   // not a multiple of 32
  CHECK(isd_gemm(&g, nullptr) == ISD_E_SHAPE);
  g.K = 64;
  g.mode = 9;
  CHECK(isd_gemm(&g, nullptr) == ISD_E_ARG);
  g.mode = ISD_GEMM_SWIGLU;                   // no W2
  CHECK(isd_gemm(&g, nullptr) == ISD_E_ARG);
  g.mode = ISD_GEMM_STORE;
  g.path = 2;
  g.M = 300;                                  // the skinny kernel holds at most 128 rows
  CHECK(isd_gemm(&g, nullptr) == ISD_E_SHAPE);

  isd_attn_args a;
  std::memset(&a, 0, sizeof a);
  a.batch = 64;
  a.rows = 7;
  a.n_q_heads = 32;
  a.n_kv_heads = 8;
  a.head_dim = 128;
  a.page_size = 16;
  a.max_pages = 256;
  a.max_ctx = 4096;
  CHECK(attn_paged_decode_workspace_bytes(&a) > 64ull * 7 * 32 * 128 * 4);
  CHECK(attn_paged_decode_workspace_bytes(nullptr) == 0);
  CHECK(attn_paged_decode(&a, nullptr) == ISD_E_ARG);           // NULL buffers
  a.q = a.k_pool = a.v_pool = fake;
  a.page_table = a.ctx_len = a.q_len = i32;
  a.out = a.workspace = fake;
  a.head_dim = 64;
  CHECK(attn_paged_decode(&a, nullptr) == ISD_E_SHAPE);
  a.head_dim = 128;
  a.rows = 17;                                 // 4 x 17 query rows per KV head > 64
  CHECK(attn_paged_decode(&a, nullptr) == ISD_E_SHAPE);

  CHECK(isd_sample_step_workspace_bytes(64, 7, 151936, 448) >= 2ull * 448 * 38 * 24);
  isd_sample_args s;
  std::memset(&s, 0, sizeof s);
  CHECK(isd_sample_step(&s, nullptr) == ISD_E_ARG);
  s.slots = reinterpret_cast<isd_slot*>(fake);
  s.logits = reinterpret_cast<const float*>(fake);
  s.tokens = s.n_commit = s.n_accept = i32;
  s.workspace = fake;
  s.batch = 4;
  s.stride_n = 9;
  s.vocab = 1000;
  CHECK(isd_sample_step(&s, nullptr) == ISD_E_ARG);
  s.stride_n = 4;
  s.propose = ISD_PROPOSE_SAMPLE;
  s.temperature = 1.f;                         // sampled proposals need the previous logits
  CHECK(isd_sample_step(&s, nullptr) == ISD_E_ARG);

  if (failures) {
    std::fprintf(stderr, "%d abi host check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks passed\n");
  return 0;
}
