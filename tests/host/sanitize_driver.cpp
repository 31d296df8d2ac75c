// Host-only driver of the engine's C ABI for an AddressSanitizer / UndefinedBehaviorSanitizer
// build (tests/test_host_sanitize.py compiles it with g++ together with the engine's host
// source).  It runs every path that needs no GPU: model and option validation, the item-trie
// build (distinct, duplicate and dense item sets), workspace sizing, calls before a workspace
// is bound, scheduler argument checks, top-K argument checks, and destruction.  The device
// launchers are stubbed: none of these paths reaches them.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "gr_beam.h"
#include "gr_internal.h"

namespace gr {
#define GR_STUB(name, ...) \
  hipError_t name(__VA_ARGS__) { std::abort(); }
GR_STUB(launch_ctx_attn, const Dev &, const StepReq *, int, int, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_beam_merge, const Dev &, const StepReq *, int, int, int, hipStream_t, LaunchEv, int)
GR_STUB(launch_finish_layer, const Dev &, const StepReq *, int, int, int, hipStream_t, LaunchEv, int)
GR_STUB(launch_ctx_attn_first_level, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_ctx_attn_layered, const Dev &, const StepReq *, int, int, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_sum_hparts, const Dev &, const StepReq *, int, hipStream_t, LaunchEv)
GR_STUB(wave_times_select, int, int)
GR_STUB(wave_times_read, long long *, size_t)
GR_STUB(launch_finish_first_level, const Dev &, const StepReq *, int, hipStream_t, LaunchEv)
GR_STUB(launch_logits, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_lsm, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_label_head, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_topk, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_init_slots, const Dev &, const int32_t *, int, hipStream_t)
GR_STUB(launch_gather_results, const Dev &, const int32_t *, int, int, uint8_t *, size_t, hipStream_t)
GR_STUB(launch_load_ctx, const void *, const void *, void *, void *, bool, int, int, int, int, int, int, float *,
        float *, hipStream_t)
GR_STUB(launch_load_v16, const void *, void *, const float *, int, int, int, int, hipStream_t)
GR_STUB(launch_topk_select, const float *, int, int, int, int32_t *, float *, int32_t *, hipStream_t)
GR_STUB(launch_soft_token, const float *, const float *, int, int, const float *, const float *, const float *, int,
        int, int, float *, float *, hipStream_t)
GR_STUB(launch_prefill_ctx, int, const void *, const void *, const int32_t *, int, int, int, const float *, int, int,
        int, int, int, void *, void *, float *, float *, hipStream_t)
GR_STUB(launch_prefill_q, int, const void *, int, const int32_t *, const float *, int, int, int, int, int, void *,
        void *, float *, float *, hipStream_t)
hipError_t prefill_scratch(float **) { std::abort(); }
GR_STUB(launch_chain_start, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_chain_norm, const Dev &, const float *, int, hipStream_t, LaunchEv)
GR_STUB(launch_chain_gemm, const Dev &, const StepReq *, int, int, int, int, int, hipStream_t, LaunchEv)
GR_STUB(launch_chain_final, const Dev &, const StepReq *, int, int, hipStream_t, LaunchEv)
#undef GR_STUB
}  // namespace gr

static int failures = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "expectation failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

static const void *kFake = reinterpret_cast<const void *>(0x1000);  // never dereferenced here

static gr_model_desc desc(int L, int Hq, int Hkv, int d, int lv, int V, gr_dtype dt) {
  gr_model_desc m{};
  m.n_layers = L;
  m.n_q_heads = Hq;
  m.n_kv_heads = Hkv;
  m.head_dim = d;
  m.n_levels = lv;
  m.codebook_size = V;
  m.dtype = dt;
  m.norm = GR_NORM_VALID;
  m.tok_q = m.tok_k = m.tok_v = kFake;
  m.w_sid = static_cast<const float *>(kFake);
  return m;
}

static gr_engine_opts opts(int R, int W, int64_t ctx) {
  gr_engine_opts o{};
  o.max_requests = R;
  o.max_beam_width = W;
  o.max_ctx_tokens = ctx;
  return o;
}

// items: n distinct random code tuples (plus `dups` repeats of the first ones)
static std::vector<int32_t> items(int lv, int V, int n, int dups, unsigned seed) {
  std::mt19937 g(seed);
  std::vector<int32_t> out;
  for (int i = 0; i < n; ++i)
    for (int t = 0; t < lv; ++t) out.push_back((int32_t)(g() % (unsigned)V));
  for (int i = 0; i < dups && i < n; ++i)
    for (int t = 0; t < lv; ++t) out.push_back(out[(size_t)i * lv + t]);
  return out;
}

int main() {
  // a Qwen3-1.7B-shaped bf16 engine over 50,000 items, and a dense float32 one
  struct Case { gr_model_desc m; int n, dups, R, W; };
  const Case cases[] = {
      {desc(28, 16, 8, 128, 3, 256, GR_DTYPE_BF16), 50000, 100, 8, 256},
      {desc(1, 4, 2, 64, 3, 16, GR_DTYPE_F32), 4096, 0, 1, 4},
      {desc(2, 8, 8, 64, 5, 256, GR_DTYPE_BF16), 20000, 7, 4, 30},
  };
  for (const Case &c : cases) {
    std::vector<int32_t> it = items(c.m.n_levels, c.m.codebook_size, c.n, c.dups, 7u);
    gr_item_set is{(int64_t)(it.size() / c.m.n_levels), it.data()};
    gr_engine_opts o = opts(c.R, c.W, 4096);
    gr_engine *e = nullptr;
    EXPECT(gr_engine_create(&c.m, &is, &o, &e) == GR_OK);
    if (!e) continue;
    int64_t nodes = 0;
    EXPECT(gr_engine_trie_nodes(e, 0, &nodes) == GR_OK && nodes == 1);
    EXPECT(gr_engine_trie_nodes(e, c.m.n_levels, &nodes) == GR_OK && nodes > 0 && nodes <= c.n);
    EXPECT(gr_engine_workspace_bytes(e) > 0);
    // nothing that needs the device before a workspace is bound
    int64_t rid = 1;
    EXPECT(gr_ctx_kv_load(e, rid, 10, 4, kFake, kFake, kFake, 0, nullptr) == GR_E_BAD_STATE);
    EXPECT(gr_beam_step(e, &rid, 1, nullptr) == GR_E_BAD_STATE);
    EXPECT(gr_request_release(e, rid) == GR_E_NOT_FOUND);
    // prefill before a workspace or tables, and a description the engine refuses
    {
      const int32_t toks[3] = {0, 1, 2};
      EXPECT(gr_ctx_prefill(e, rid, toks, 3, -1, nullptr, 1, nullptr, nullptr, nullptr, nullptr) == GR_E_BAD_STATE);
      EXPECT(gr_ctx_prefill_noalloc(e, rid, toks, 3, -1, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
             GR_E_BAD_STATE);
      EXPECT(gr_ctx_prefill_noalloc(nullptr, rid, toks, 3, -1, nullptr, 1, nullptr, nullptr, nullptr, nullptr) ==
             GR_E_INVALID_ARG);
      gr_prefill_desc pd{};
      EXPECT(gr_engine_set_prefill(e, &pd) == GR_E_INVALID_ARG);
      pd.vocab = 4;
      pd.tok_q = pd.tok_k = pd.tok_v = kFake;
      pd.user_dim = 3;
      EXPECT(gr_engine_set_prefill(e, &pd) == GR_E_INVALID_ARG);
      EXPECT(gr_engine_set_prefill(nullptr, &pd) == GR_E_INVALID_ARG);
    }
    gr_sched *s = nullptr;
    EXPECT(gr_sched_create(e, 1, nullptr, &s) == GR_E_BAD_STATE && s == nullptr);
    // a result record unpacked from host memory: full, empty, over capacity, not a record
    {
      const size_t rb = gr_beams_result_bytes(e);
      const int lv = c.m.n_levels;
      std::vector<uint8_t> rec(rb, 0);
      int32_t nl = c.W;
      std::memcpy(rec.data(), &nl, 4);
      std::vector<int32_t> codes((size_t)c.W * lv);
      std::vector<float> scores((size_t)c.W);
      int32_t got = -1;
      EXPECT(gr_beams_unpack(e, rec.data(), 0, c.W, codes.data(), scores.data(), &got) == GR_OK && got == c.W);
      EXPECT(gr_beams_unpack(e, rec.data(), 0, c.W - 1, codes.data(), scores.data(), &got) == GR_E_INVALID_ARG);
      nl = c.W + 1;
      std::memcpy(rec.data(), &nl, 4);
      EXPECT(gr_beams_unpack(e, rec.data(), 0, c.W + 8, codes.data(), scores.data(), &got) == GR_E_INVALID_ARG);
      EXPECT(gr_beams_get_batch_async(e, &rid, 1, rec.data(), nullptr) == GR_E_BAD_STATE);
    }
    EXPECT(gr_engine_bind_workspace(e, const_cast<void *>(kFake), 16, nullptr) == GR_E_OUT_OF_MEMORY);
    EXPECT(gr_engine_destroy(e) == GR_OK);
  }
  // rejected models, options and item sets
  {
    std::vector<int32_t> it = items(3, 16, 200, 0, 3u);
    gr_item_set is{200, it.data()};
    gr_engine_opts o = opts(1, 4, 64);
    gr_engine *e = nullptr;
    gr_model_desc bad = desc(1, 4, 3, 64, 3, 16, GR_DTYPE_F32);  // Hq % Hkv != 0
    EXPECT(gr_engine_create(&bad, &is, &o, &e) == GR_E_INVALID_ARG && e == nullptr);
    gr_model_desc m = desc(1, 4, 2, 64, 3, 16, GR_DTYPE_F32);
    gr_engine_opts bo = opts(0, 4, 64);
    EXPECT(gr_engine_create(&m, &is, &bo, &e) != GR_OK && e == nullptr);
    bo = opts(1, 4, 64);
    bo.max_layers_per_launch = -1;
    EXPECT(gr_engine_create(&m, &is, &bo, &e) != GR_OK && e == nullptr);
    bo = opts(1, 4, 64);
    bo.flags = 8u;  // not an engine flag
    EXPECT(gr_engine_create(&m, &is, &bo, &e) == GR_E_INVALID_ARG && e == nullptr);
    bo.flags = GR_ENGINE_PER_LAYER | GR_ENGINE_DEBUG_ATTN | GR_ENGINE_GRAPH;
    EXPECT(gr_engine_create(&m, &is, &bo, &e) == GR_OK && e != nullptr);
    EXPECT(gr_engine_destroy(e) == GR_OK);
    e = nullptr;
    it[5] = 16;  // code out of range
    EXPECT(gr_engine_create(&m, &is, &o, &e) != GR_OK && e == nullptr);
    gr_item_set none{0, it.data()};
    EXPECT(gr_engine_create(&m, &none, &o, &e) != GR_OK && e == nullptr);
    EXPECT(gr_last_error()[0] != '\0');
  }
  // handles and outputs that are null
  int32_t n = 0;
  EXPECT(gr_sched_advance(nullptr, &n) == GR_E_INVALID_ARG);
  EXPECT(gr_sched_submit(nullptr, 1, 10, 4, kFake, kFake, kFake, 0) == GR_E_INVALID_ARG);
  EXPECT(gr_sched_destroy(nullptr) == GR_OK);
  EXPECT(gr_engine_destroy(nullptr) == GR_OK);
  EXPECT(gr_topk_select(nullptr, 1, 16, 4, nullptr, nullptr, nullptr, nullptr) == GR_E_INVALID_ARG);
  EXPECT(gr_topk_select(static_cast<const float *>(kFake), 4, 16, 0, (int32_t *)kFake, (float *)kFake,
                        (int32_t *)kFake, nullptr) == GR_E_INVALID_ARG);
  EXPECT(gr_ctx_padded_len(65) == 128);
  if (failures) {
    std::fprintf(stderr, "%d expectations failed\n", failures);
    return 1;
  }
  std::printf("host paths clean\n");
  return 0;
}
