// Host side of the semantic-ID beam-decode library: argument validation, the
// item trie, workspace layout, request table, per-step work descriptors and the
// C ABI declared in include/gr_beam.h.
//
// The split of the KV cache into a per-request ContextKV, a short per-beam
// BeamKV and a BeamPath ancestry table, continuous batching of requests at
// different levels, and the item-constrained top-K all follow the zhiding.cn
// article on NVIDIA recsys-examples, section "语义ID生成式推荐专用推理框架".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <deque>
#include <map>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "gr_beam.h"
#include "gr_internal.h"

namespace {

thread_local std::string g_err;

gr_status fail(gr_status st, const std::string &msg) {
  g_err = msg;
  return st;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kRing = 16;  // per-step descriptor buffers in flight

}  // namespace

constexpr int kAuxStreams = 3;
constexpr size_t kChainPartFloats = size_t(8) << 20;  // split-K partials of the chain projections

struct gr_engine {
  gr::Dims dm{};
  gr::SlotLayout sl{};
  gr::Dev dev{};
  gr_model_desc model{};
  gr_engine_opts opts{};
  gr_chain_desc chain{};  // the layer-chain model (dm.chain), copied at create
  gr_label_desc label{};  // the label head (dm.n_labels > 0), copied at create
  int elem = 2;

  // trie, host copy: levels 0..n_levels-1 hold masks and first-child indices
  std::vector<int64_t> nodes;  // nodes[t] = valid prefixes of length t, t = 0..n_levels
  std::vector<uint32_t> h_mask;
  std::vector<int32_t> h_child;
  std::vector<int64_t> trie_off;

  // workspace layout (byte offsets)
  size_t off_mask = 0, off_child = 0, off_slots = 0, off_pool = 0, off_work = 0, off_out = 0, ws_need = 0;
  size_t off_chain = 0, chain_bytes = 0;  // the layer chain's activation rows
  size_t off_label = 0;                   // label-step log-probs [max_requests][W_max][n_labels] f32
  size_t off_chain_dbg = 0, chain_dbg_layer = 0;  // debug copies of them, per layer
  int chain_rows = 0;                     // rows of those buffers (a multiple of 128)
  size_t work_bytes = 0;  // one ring entry
  size_t out_bytes = 0;   // results of one request in the staging area (gr_beams_get_batch)
  uint8_t *out_host = nullptr;  // pinned copy of the staging area
  uint8_t *ws = nullptr;
  bool bound = false;
  bool poisoned = false;

  // context pool: padded tokens, first fit
  int64_t pool_tokens = 0;
  size_t pool_tok_bytes = 0;
  bool v16 = false;  // loaded contexts also keep V^T as float16 for the eight-wave kernel (bf16, head_dim 128)
  std::map<int64_t, int64_t> pool_free;  // offset -> length

  struct Req {
    int slot = -1;
    int N = 0, Np = 0, W = 0, level = 0, n_bound = 1;
    int n_items = 0;  // > 0 while the request scores given items (gr_score_items)
    int last_row0 = 0;  // the layer chain: the request's first packed row in its last step
    bool adopt = false;
    int64_t pool_off = -1;
    const void *k = nullptr, *vt = nullptr;
    const void *vt16 = nullptr;  // float16 copy of V^T (pool contexts of v16 engines), else null
  };
  std::unordered_map<int64_t, Req> reqs;
  std::vector<int> free_slots;

  // profiling: timing events carried by the launches themselves (no marker packets between
  // kernels), folded into [kind][level] buckets.  A record spans two events of the pool.
  bool prof = false;
  uint32_t prof_mask = ~0u;  // the kinds (bit 1 << GR_PROF_*) profiled while prof is on
  int prof_stride = 1;       // one-launch-per-layer sequences: only layers l % prof_stride == 0 are timed
  std::vector<hipEvent_t> prof_ev;
  int prof_next = 0;  // next unused event of the pool
  struct ProfRec { int kind, level, a, b, count, disp; };  // count: layer steps, disp: kernel dispatches
  std::vector<ProfRec> prof_pending;
  static constexpr int kProfKinds = GR_PROF_NORM + 1;
  double prof_ms[kProfKinds][gr::kMaxLevels + 1] = {};
  int64_t prof_n[kProfKinds][gr::kMaxLevels + 1] = {};
  int64_t prof_d[kProfKinds][gr::kMaxLevels + 1] = {};

  // split-K steps with several variant groups: each group's chain of layer launches depends
  // only on itself, so groups 1..3 (mod 4) run on their own streams, forked from and joined
  // into the caller's stream (default priority, created when the workspace is bound)
  hipStream_t aux[kAuxStreams] = {};
  hipEvent_t fork_ev = nullptr, join_ev[kAuxStreams] = {};
  // graph replay (GR_ENGINE_GRAPH): one executable graph per step shape (the launch sequence's
  // every parameter), captured on cap_st; the descriptors of graph steps go to one fixed
  // device area (gdesc), and gdone_ev marks the last graph launch's end for the next upload
  hipStream_t cap_st = nullptr;
  hipEvent_t gdone_ev = nullptr;
  bool gdone_used = false;
  std::map<std::vector<int64_t>, hipGraphExec_t> graphs;
  std::deque<std::vector<int64_t>> graph_fifo;
  int64_t graph_hits = 0, graph_captures = 0;
  std::vector<gr::StepReq *> pinned;
  std::vector<hipEvent_t> events;
  std::vector<bool> event_used;
  int ring = 0;

  // prefill (gr_engine_set_prefill): the tables, a pinned token buffer and its device copy
  // (grown on demand; an event guards the pinned buffer until its upload has run), and the
  // soft token's embedding and partial projections
  gr_prefill_desc pf{};
  bool has_pf = false;
  int32_t *pf_tok_host = nullptr, *pf_tok_dev = nullptr;
  int64_t pf_tok_cap = 0;
  float *pf_soft = nullptr;
  hipEvent_t pf_ev = nullptr;
  bool pf_ev_used = false;
  // the allocation-free prefill's fixed device array on the engine's device (resolved at bind)
  float *noalloc_scratch = nullptr;
};

namespace {

gr_status check_dev(gr_engine *e, hipError_t err, const char *what) {
  if (err == hipSuccess) return GR_OK;
  e->poisoned = true;
  return fail(GR_E_DEVICE, std::string(what) + ": " + hipGetErrorString(err));
}

constexpr int kProfPool = 2048;  // events

gr_status prof_fold(gr_engine *e) {
  for (const auto &p : e->prof_pending) {
    hipEvent_t a = e->prof_ev[(size_t)p.a], b = e->prof_ev[(size_t)p.b];
    gr_status r = check_dev(e, hipEventSynchronize(b), "profiling event");
    if (r != GR_OK) return r;
    float ms = 0.f;
    if ((r = check_dev(e, hipEventElapsedTime(&ms, a, b), "profiling event")) != GR_OK) return r;
    e->prof_ms[p.kind][p.level] += ms;
    e->prof_n[p.kind][p.level] += p.count;
    e->prof_d[p.kind][p.level] += p.disp;
  }
  e->prof_pending.clear();
  e->prof_next = 0;
  return GR_OK;
}

// Makes room for `count` events before a step starts (every pending record is complete
// then, so folding is safe).  Returns false when profiling is off or the step needs more
// events than the pool holds.
bool prof_reserve(gr_engine *e, int count) {
  if (!e->prof || count > kProfPool) return false;
  if (e->prof_next + count > kProfPool && prof_fold(e) != GR_OK) return false;
  return true;
}

// A fresh (start, stop) event pair for a profiled launch; {-1, -1} when off.
std::pair<int, int> prof_pair(gr_engine *e, bool on) {
  if (!on) return {-1, -1};
  const int a = e->prof_next;
  e->prof_next += 2;
  return {a, a + 1};
}

gr::LaunchEv prof_ev(gr_engine *e, int a, int b) {
  gr::LaunchEv ev;
  if (a >= 0) ev.start = e->prof_ev[(size_t)a];
  if (b >= 0) ev.stop = e->prof_ev[(size_t)b];
  return ev;
}

void prof_record(gr_engine *e, int kind, int level, std::pair<int, int> ab, int count = 1, int disp = 1) {
  if (ab.first >= 0) e->prof_pending.push_back({kind, level, ab.first, ab.second, count, disp});
}

gr_status build_trie(gr_engine *e, const gr_item_set *items) {
  const int lv = e->dm.levels, V = e->dm.V;
  std::vector<uint64_t> keys((size_t)items->n_items);
  for (int64_t i = 0; i < items->n_items; ++i) {
    uint64_t k = 0;
    for (int t = 0; t < lv; ++t) {
      const int32_t c = items->codes[i * lv + t];
      if (c < 0 || c >= V) return fail(GR_E_INVALID_ARG, "item code out of range [0, codebook_size)");
      k = k * (uint64_t)V + (uint64_t)c;
    }
    keys[(size_t)i] = k;
  }
  std::sort(keys.begin(), keys.end());
  keys.erase(std::unique(keys.begin(), keys.end()), keys.end());
  std::vector<uint64_t> powv(lv + 1, 1);
  for (int t = 1; t <= lv; ++t) powv[t] = powv[t - 1] * (uint64_t)V;
  // count nodes per level
  e->nodes.assign(lv + 1, 0);
  e->nodes[0] = 1;
  {
    std::vector<uint64_t> last(lv + 1, ~0ull);
    for (uint64_t k : keys)
      for (int t = 1; t <= lv; ++t) {
        const uint64_t p = k / powv[lv - t];
        if (p != last[t]) {
          last[t] = p;
          e->nodes[t]++;
        }
      }
  }
  const int MW = e->dm.MW;
  e->trie_off.assign(lv + 1, 0);
  for (int t = 1; t <= lv; ++t) e->trie_off[t] = e->trie_off[t - 1] + e->nodes[t - 1];
  const int64_t total = e->trie_off[lv];
  e->h_mask.assign((size_t)total * MW, 0u);
  e->h_child.assign((size_t)total, -1);
  std::vector<uint64_t> last(lv + 1, ~0ull);
  std::vector<int64_t> cnt(lv + 1, 0);
  cnt[0] = 1;
  for (uint64_t k : keys) {
    for (int t = 1; t <= lv; ++t) {
      const uint64_t p = k / powv[lv - t];
      if (p == last[t]) continue;
      last[t] = p;
      const int64_t idx = cnt[t]++;
      const int64_t parent = cnt[t - 1] - 1;  // keys are sorted: the parent is the newest node above
      const int c = (int)(p % (uint64_t)V);
      const int64_t prow = e->trie_off[t - 1] + parent;
      e->h_mask[(size_t)prow * MW + (c >> 5)] |= 1u << (c & 31);
      if (e->h_child[(size_t)prow] < 0) e->h_child[(size_t)prow] = (int32_t)idx;
    }
  }
  return GR_OK;
}

void layout(gr_engine *e) {
  const gr::Dims &d = e->dm;
  const size_t A = 256;
  const size_t W = d.W_max, el = e->elem;
  gr::SlotLayout &s = e->sl;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o = align_up(o + bytes, A);
    return r;
  };
  const size_t kv = (size_t)d.L * d.tl * W * d.Hkv * d.d * el;
  s.beamkv_k = take(kv);
  s.beamkv_v = take(kv);
  s.q_last = take(std::max((size_t)d.L * d.Hq * d.d * el, (size_t)d.Hq * d.d * 4));  // chain: x_last [D] f32
  s.knmax = take((size_t)d.L * d.Hkv * 4);
  s.vscale = take((size_t)d.L * d.Hkv * 4);
  s.h = take(W * d.Hq * d.d * 4);
  s.logits = take(W * d.V * 4);
  s.logits_part = take((size_t)gr::kLogitsKS * W * d.V * 4);
  s.cand = take(W * d.V * 4);
  s.lkeys = take((size_t)((W + gr::kLsmRows - 1) / gr::kLsmRows) * W * 8);
  s.lcnt = take((size_t)((W + gr::kLsmRows - 1) / gr::kLsmRows) * 4);
  for (int b = 0; b < 2; ++b) {
    s.part_o[b] = take((size_t)d.Hkv * d.S_max * W * d.g * d.d * 4);
    s.part_ml[b] = take((size_t)d.Hkv * d.S_max * W * d.g * 8);
  }
  for (int b = 0; b < 2; ++b) {
    s.codes[b] = take(W * d.levels * 4);
    s.score[b] = take(W * 4);
    s.node[b] = take(W * 4);
    s.anc[b] = take(W * d.levels * 4);
    s.parent[b] = take(W * 4);
  }
  s.n_live = take(8);
  s.items = take(W * d.levels * 4);
  s.dbg_attn = d.debug_attn ? take((size_t)d.L * W * d.Hq * d.d * 4) : 0;
  const bool full_ctx = d.dtype == 1 && d.d == 128;  // full-context (layered) steps possible
  s.hl = full_ctx ? take((size_t)d.L * W * d.Hq * d.d * 4) : 0;
  s.slot_bytes = align_up(o, A);

  size_t w = 0;
  e->off_mask = w;
  w = align_up(w + e->h_mask.size() * 4, A);
  e->off_child = w;
  w = align_up(w + e->h_child.size() * 4, A);
  e->off_slots = w;
  w = align_up(w + s.slot_bytes * (size_t)e->opts.max_requests, A);
  e->v16 = d.dtype == 1 && d.d == 128;
  e->pool_tok_bytes = (size_t)(e->v16 ? 3 : 2) * d.L * d.Hkv * d.d * el;
  e->pool_tokens = e->opts.max_ctx_tokens;
  e->off_pool = w;
  w = align_up(w + (size_t)e->pool_tokens * e->pool_tok_bytes, A);
  e->work_bytes = align_up(sizeof(gr::StepReq) * (size_t)e->opts.max_requests, A);
  e->off_work = w;
  w = align_up(w + e->work_bytes * (kRing + 1), A);  // the ring, then the graph steps' area
  // result staging: per request n_live (16-byte header), codes [W][levels], scores [W]
  e->out_bytes = align_up(16 + W * d.levels * 4 + W * 4, A);
  e->off_out = w;
  w = align_up(w + e->out_bytes * (size_t)e->opts.max_requests, A);
  if (d.n_labels > 0) {
    e->off_label = w;
    w = align_up(w + (size_t)e->opts.max_requests * W * d.n_labels * 4, A);
  }
  if (d.chain) {
    // every request's beams packed at 32-row boundaries, padded to 128: x f32 [D], xn bf16 [D],
    // q and o bf16 [Hq d], act bf16 [I]
    const size_t rows = align_up((size_t)e->opts.max_requests * align_up(W, 32), 128);
    const size_t D = (size_t)d.Hq * d.d, I = (size_t)e->chain.intermediate;
    e->chain_rows = (int)rows;
    e->off_chain = w;
    // + the split-K partial sums of the few-row projections (32 MiB)
    e->chain_bytes = align_up(rows * (D * 4 + D * 2 + 2 * D * 2 + I * 2), A) + kChainPartFloats * 4;
    w = align_up(w + e->chain_bytes, A);
    if (d.debug_attn) {
      // per layer, copies of the rows entering and leaving each projection (gr_debug_chain_rows)
      e->off_chain_dbg = w;
      e->chain_dbg_layer = align_up(rows * (4 * D * 4 + 2 * D * 2 + 2 * D * 2 + I * 2), A);
      w = align_up(w + e->chain_dbg_layer * (size_t)d.L, A);
    }
  }
  e->ws_need = w;
}

bool pool_alloc(gr_engine *e, int64_t n, int64_t *off) {
  for (auto it = e->pool_free.begin(); it != e->pool_free.end(); ++it) {
    if (it->second >= n) {
      *off = it->first;
      const int64_t rest = it->second - n, roff = it->first + n;
      e->pool_free.erase(it);
      if (rest > 0) e->pool_free[roff] = rest;
      return true;
    }
  }
  return false;
}

void pool_free(gr_engine *e, int64_t off, int64_t n) {
  auto it = e->pool_free.emplace(off, n).first;
  auto nx = std::next(it);
  if (nx != e->pool_free.end() && it->first + it->second == nx->first) {
    it->second += nx->second;
    e->pool_free.erase(nx);
  }
  if (it != e->pool_free.begin()) {
    auto pv = std::prev(it);
    if (pv->first + pv->second == it->first) {
      pv->second += it->second;
      e->pool_free.erase(it);
    }
  }
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// debug copy of chain rows `which` of layer l (layout of one layer: X_IN, X_MID, X_OUT f32 [rows][D];
// XN_ATTN, XN_MLP bf16 [rows][D]; Q, O bf16 [rows][Hq d]; ACT bf16 [rows][I]; one spare f32 [rows][D])
uint8_t *chain_dbg(gr_engine *e, int l, int which) {
  const size_t rows = (size_t)e->chain_rows, D = (size_t)e->dm.Hq * e->dm.d;
  uint8_t *b = e->ws + e->off_chain_dbg + e->chain_dbg_layer * (size_t)l;
  switch (which) {
    case GR_CHAIN_X_IN: return b;
    case GR_CHAIN_X_MID: return b + rows * D * 4;
    case GR_CHAIN_X_OUT: return b + 2 * rows * D * 4;
    case GR_CHAIN_XN_ATTN: return b + 4 * rows * D * 4;
    case GR_CHAIN_XN_MLP: return b + 4 * rows * D * 4 + rows * D * 2;
    case GR_CHAIN_Q: return b + 4 * rows * D * 4 + 2 * rows * D * 2;
    case GR_CHAIN_O: return b + 4 * rows * D * 4 + 3 * rows * D * 2;
    default: return b + 4 * rows * D * 4 + 4 * rows * D * 2;
  }
}

}  // namespace

extern "C" {

const char *gr_last_error(void) { return g_err.c_str(); }

int32_t gr_ctx_padded_len(int32_t ctx_len) {
  if (ctx_len <= 0) return 0;
  return (int32_t)align_up((size_t)ctx_len, gr::kTileTok);
}

gr_status gr_engine_create(const gr_model_desc *m, const gr_item_set *items, const gr_engine_opts *o,
                           gr_engine **out) {
  g_err.clear();
  if (!m || !items || !o || !out) return fail(GR_E_INVALID_ARG, "null argument");
  *out = nullptr;
  if (m->n_layers < 1 || m->n_q_heads < 1 || m->n_kv_heads < 1)
    return fail(GR_E_INVALID_ARG, "n_layers, n_q_heads and n_kv_heads must be >= 1");
  if (m->n_q_heads % m->n_kv_heads != 0) return fail(GR_E_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (m->n_q_heads / m->n_kv_heads > gr::kMaxGroup)
    return fail(GR_E_UNSUPPORTED, "more than 8 query heads per kv head");
  if (m->head_dim != 64 && m->head_dim != 128) return fail(GR_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if ((m->n_q_heads * m->head_dim) % (32 * gr::kLogitsKS) != 0)
    return fail(GR_E_UNSUPPORTED, "n_q_heads * head_dim must be a multiple of 128");
  if (m->n_levels < 1 || m->n_levels > gr::kMaxLevels) return fail(GR_E_INVALID_ARG, "n_levels must be in [1, 8]");
  if (m->codebook_size < 2 || m->codebook_size > 1024) return fail(GR_E_INVALID_ARG, "codebook_size must be in [2, 1024]");
  {
    double bits = m->n_levels * std::log2((double)m->codebook_size);
    if (bits >= 62.0) return fail(GR_E_UNSUPPORTED, "codebook_size**n_levels must be < 2**62");
  }
  if (m->dtype != GR_DTYPE_F32 && m->dtype != GR_DTYPE_BF16) return fail(GR_E_INVALID_ARG, "dtype");
  if (m->norm != GR_NORM_VALID && m->norm != GR_NORM_FULL) return fail(GR_E_INVALID_ARG, "norm");
  if (!m->w_sid) return fail(GR_E_INVALID_ARG, "w_sid is null");
  if (m->chain) {
    const gr_chain_desc *c = m->chain;
    if (m->dtype != GR_DTYPE_BF16) return fail(GR_E_UNSUPPORTED, "the layer chain runs in bf16 only");
    if ((m->n_q_heads * m->head_dim) % 128 != 0 || (m->n_kv_heads * m->head_dim) % 128 != 0)
      return fail(GR_E_UNSUPPORTED, "the layer chain needs n_q_heads*head_dim and n_kv_heads*head_dim multiples of 128");
    if (c->intermediate < 64 || c->intermediate % 64 != 0 || c->intermediate > (1 << 20))
      return fail(GR_E_UNSUPPORTED, "intermediate must be a positive multiple of 64");
    if (!(c->rms_eps > 0.f)) return fail(GR_E_INVALID_ARG, "rms_eps must be > 0");
    if ((m->n_levels > 1 && !c->embed) || !c->w_q || !c->w_k || !c->w_v || !c->w_o || !c->w_gate || !c->w_up ||
        !c->w_down || !c->g_attn || !c->g_mlp || !c->g_final)
      return fail(GR_E_INVALID_ARG, "a layer-chain weight is null");
  } else if ((m->n_levels > 1 || m->label) && (!m->tok_q || !m->tok_k || !m->tok_v)) {
    return fail(GR_E_INVALID_ARG, "token tables are null");
  }
  if (m->label) {
    if (m->chain) return fail(GR_E_UNSUPPORTED, "a label head needs the table model, not a layer chain");
    if (m->label->n_labels < 1 || m->label->n_labels > 16) return fail(GR_E_UNSUPPORTED, "n_labels must be in [1, 16]");
    if (!m->label->w_label) return fail(GR_E_INVALID_ARG, "w_label is null");
  }
  if (items->n_items < 1 || !items->codes) return fail(GR_E_INVALID_ARG, "empty item set");
  if (o->max_requests < 1 || o->max_requests > 65536) return fail(GR_E_INVALID_ARG, "max_requests must be in [1, 65536]");
  if (o->max_beam_width < 1 || o->max_beam_width > gr::kMaxBeam)
    return fail(GR_E_INVALID_ARG, "max_beam_width must be in [1, 1024]");
  if (o->max_ctx_tokens < 0) return fail(GR_E_INVALID_ARG, "max_ctx_tokens < 0");
  if (o->max_splits < 0 || o->max_splits > 64) return fail(GR_E_INVALID_ARG, "max_splits must be in [0, 64]");
  if (o->max_layers_per_launch < 0) return fail(GR_E_INVALID_ARG, "max_layers_per_launch must be >= 0");
  if (o->flags & ~(GR_ENGINE_DEBUG_ATTN | GR_ENGINE_PER_LAYER | GR_ENGINE_GRAPH))
    return fail(GR_E_INVALID_ARG, "unknown engine flag");

  gr_engine *e = new gr_engine();
  e->model = *m;
  e->opts = *o;
  if (m->chain) e->chain = *m->chain;
  if (m->label) e->label = *m->label;
  e->model.chain = nullptr;  // the descriptions are copied: the caller's may go away
  e->model.label = nullptr;
  if (e->opts.max_splits == 0) e->opts.max_splits = 4;
  e->elem = m->dtype == GR_DTYPE_BF16 ? 2 : 4;
  gr::Dims &d = e->dm;
  d.L = m->n_layers;
  d.Hq = m->n_q_heads;
  d.Hkv = m->n_kv_heads;
  d.g = d.Hq / d.Hkv;
  d.d = m->head_dim;
  d.levels = m->n_levels;
  d.V = m->codebook_size;
  d.MW = (d.V + 31) / 32;
  d.W_max = o->max_beam_width;
  d.S_max = e->opts.max_splits;
  d.dtype = m->dtype == GR_DTYPE_BF16 ? 1 : 0;
  d.norm = m->norm == GR_NORM_FULL ? 1 : 0;
  d.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.d));
  d.debug_attn = (o->flags & GR_ENGINE_DEBUG_ATTN) ? 1 : 0;
  d.chain = m->chain ? 1 : 0;
  d.n_labels = m->label ? m->label->n_labels : 0;
  d.tl = d.levels - 1 + (d.n_labels > 0 ? 1 : 0);
  gr_status st = build_trie(e, items);
  if (st != GR_OK) {
    delete e;
    return st;
  }
  layout(e);
  for (int s = e->opts.max_requests - 1; s >= 0; --s) e->free_slots.push_back(s);
  if (e->pool_tokens > 0) e->pool_free[0] = e->pool_tokens;
  *out = e;
  return GR_OK;
}

size_t gr_engine_workspace_bytes(const gr_engine *e) { return e ? e->ws_need : 0; }

gr_status gr_engine_trie_nodes(const gr_engine *e, int32_t level, int64_t *n) {
  if (!e || !n) return fail(GR_E_INVALID_ARG, "null argument");
  if (level < 0 || level > e->dm.levels) return fail(GR_E_INVALID_ARG, "level out of range");
  *n = e->nodes[level];
  return GR_OK;
}

gr_status gr_engine_bind_workspace(gr_engine *e, void *ws, size_t bytes, void *stream) {
  if (!e || !ws) return fail(GR_E_INVALID_ARG, "null argument");
  if (e->bound) return fail(GR_E_BAD_STATE, "workspace already bound");
  if (bytes < e->ws_need) return fail(GR_E_OUT_OF_MEMORY, "workspace smaller than gr_engine_workspace_bytes");
  if (((uintptr_t)ws & 255u) != 0) return fail(GR_E_INVALID_ARG, "workspace must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  e->ws = (uint8_t *)ws;
  gr_status r;
  if ((r = check_dev(e, hipMemcpyAsync(e->ws + e->off_mask, e->h_mask.data(), e->h_mask.size() * 4,
                                       hipMemcpyHostToDevice, st), "trie upload")) != GR_OK)
    return r;
  if ((r = check_dev(e, hipMemcpyAsync(e->ws + e->off_child, e->h_child.data(), e->h_child.size() * 4,
                                       hipMemcpyHostToDevice, st), "trie upload")) != GR_OK)
    return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "trie upload")) != GR_OK) return r;
  if ((r = check_dev(e, hipHostMalloc((void **)&e->out_host, e->out_bytes * (size_t)e->opts.max_requests,
                                      hipHostMallocDefault), "pinned result staging")) != GR_OK)
    return r;
  e->pinned.assign(kRing, nullptr);
  e->events.assign(kRing, nullptr);
  e->event_used.assign(kRing, false);
  for (int i = 0; i < kRing; ++i) {
    if ((r = check_dev(e, hipHostMalloc((void **)&e->pinned[i], e->work_bytes, hipHostMallocDefault),
                       "pinned descriptor ring")) != GR_OK)
      return r;
    if ((r = check_dev(e, hipEventCreateWithFlags(&e->events[i], hipEventDisableTiming), "event")) != GR_OK)
      return r;
  }
  e->prof_ev.assign(kProfPool, nullptr);
  for (auto &ev : e->prof_ev)
    if ((r = check_dev(e, hipEventCreate(&ev), "event")) != GR_OK) return r;
  // streams (default priority) and fork/join events for steps with several variant groups
  for (int i = 0; i < kAuxStreams; ++i) {
    if ((r = check_dev(e, hipStreamCreateWithFlags(&e->aux[i], hipStreamNonBlocking), "stream create")) != GR_OK)
      return r;
    if ((r = check_dev(e, hipEventCreateWithFlags(&e->join_ev[i], hipEventDisableTiming), "event create")) != GR_OK)
      return r;
  }
  if ((r = check_dev(e, hipEventCreateWithFlags(&e->fork_ev, hipEventDisableTiming), "event create")) != GR_OK)
    return r;
  if (e->opts.flags & GR_ENGINE_GRAPH) {
    if ((r = check_dev(e, hipStreamCreateWithFlags(&e->cap_st, hipStreamNonBlocking), "stream create")) != GR_OK)
      return r;
    if ((r = check_dev(e, hipEventCreateWithFlags(&e->gdone_ev, hipEventDisableTiming), "event create")) != GR_OK)
      return r;
  }
  if ((r = check_dev(e, gr::prefill_scratch(&e->noalloc_scratch), "scratch address")) != GR_OK) return r;
  gr::Dev &dv = e->dev;
  dv.dm = e->dm;
  dv.sl = e->sl;
  dv.slots = e->ws + e->off_slots;
  dv.trie_mask = (const uint32_t *)(e->ws + e->off_mask);
  dv.trie_child = (const int32_t *)(e->ws + e->off_child);
  for (int t = 0; t <= e->dm.levels && t <= gr::kMaxLevels; ++t) dv.trie_off[t] = e->trie_off[t];
  dv.tok_q = e->model.tok_q;
  dv.tok_k = e->model.tok_k;
  dv.tok_v = e->model.tok_v;
  dv.w_sid = e->model.w_sid;
  dv.w_label = e->dm.n_labels > 0 ? e->label.w_label : nullptr;
  dv.label_out = e->dm.n_labels > 0 ? (float *)(e->ws + e->off_label) : nullptr;
  if (e->dm.chain) {
    gr::ChainDev &c = dv.ch;
    const gr_chain_desc &cd = e->chain;
    const size_t rows = (size_t)e->chain_rows, D = (size_t)e->dm.Hq * e->dm.d, I = (size_t)cd.intermediate;
    c.D = (int)D;
    c.I = (int)I;
    c.eps = cd.rms_eps;
    c.embed = (const uint16_t *)cd.embed;
    c.wq = (const uint16_t *)cd.w_q;
    c.wk = (const uint16_t *)cd.w_k;
    c.wv = (const uint16_t *)cd.w_v;
    c.wo = (const uint16_t *)cd.w_o;
    c.wg = (const uint16_t *)cd.w_gate;
    c.wu = (const uint16_t *)cd.w_up;
    c.wd = (const uint16_t *)cd.w_down;
    c.g_attn = cd.g_attn;
    c.g_mlp = cd.g_mlp;
    c.g_final = cd.g_final;
    uint8_t *b = e->ws + e->off_chain;
    c.x = (float *)b;
    c.xn = (uint16_t *)(b + rows * D * 4);
    c.q = c.xn + rows * D;
    c.o = c.q + rows * D;
    c.act = c.o + rows * D;
    c.part = (float *)(b + align_up(rows * (D * 4 + D * 2 + 2 * D * 2 + I * 2), 256));
    c.part_floats = kChainPartFloats;
    // padding rows are read by the projections: start every row at zero (finite)
    if ((r = check_dev(e, hipMemsetAsync(b, 0, e->chain_bytes, st), "chain rows")) != GR_OK) return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "chain rows")) != GR_OK) return r;
  }
  e->bound = true;
  return GR_OK;
}

gr_status gr_engine_destroy(gr_engine *e) {
  if (!e) return GR_OK;
  if (e->bound) {
    (void)hipDeviceSynchronize();
    for (auto &ev : e->events)
      if (ev) (void)hipEventDestroy(ev);
    for (auto &ev : e->prof_ev)
      if (ev) (void)hipEventDestroy(ev);
    for (int i = 0; i < kAuxStreams; ++i) {
      if (e->aux[i]) (void)hipStreamDestroy(e->aux[i]);
      if (e->join_ev[i]) (void)hipEventDestroy(e->join_ev[i]);
    }
    if (e->fork_ev) (void)hipEventDestroy(e->fork_ev);
    for (auto &kv : e->graphs) (void)hipGraphExecDestroy(kv.second);
    if (e->cap_st) (void)hipStreamDestroy(e->cap_st);
    if (e->gdone_ev) (void)hipEventDestroy(e->gdone_ev);
    for (auto *p : e->pinned)
      if (p) (void)hipHostFree(p);
    if (e->out_host) (void)hipHostFree(e->out_host);
  }
  if (e->pf_tok_host || e->pf_tok_dev || e->pf_soft || e->pf_ev) {
    (void)hipDeviceSynchronize();
    if (e->pf_tok_host) (void)hipHostFree(e->pf_tok_host);
    if (e->pf_tok_dev) (void)hipFree(e->pf_tok_dev);
    if (e->pf_soft) (void)hipFree(e->pf_soft);
    if (e->pf_ev) (void)hipEventDestroy(e->pf_ev);
  }
  delete e;
  return GR_OK;
}

gr_status gr_engine_set_prefill(gr_engine *e, const gr_prefill_desc *p) {
  if (!e || !p) return fail(GR_E_INVALID_ARG, "null engine or prefill description");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (e->dm.chain) return fail(GR_E_UNSUPPORTED, "the layer chain takes its context from gr_ctx_kv_load");
  if (p->vocab < 1 || !p->tok_q || !p->tok_k || !p->tok_v) return fail(GR_E_INVALID_ARG, "need vocab >= 1 and three tables");
  if (p->user_dim < 0 || p->user_dim > 8192) return fail(GR_E_INVALID_ARG, "user_dim must be in [0, 8192]");
  if (p->user_dim > 0 && (p->embed_dim < 1 || p->embed_dim > 8192 || !p->proj || !p->w_q || !p->w_k || !p->w_v))
    return fail(GR_E_INVALID_ARG, "a soft token needs embed_dim in [1, 8192] and proj, w_q, w_k, w_v");
  if (((uintptr_t)p->tok_k | (uintptr_t)p->tok_v) & 15u) return fail(GR_E_INVALID_ARG, "tables must be 16-byte aligned");
  gr_status r;
  if (!e->pf_ev && (r = check_dev(e, hipEventCreateWithFlags(&e->pf_ev, hipEventDisableTiming), "event")) != GR_OK)
    return r;
  // the new soft-token staging first: on failure the engine keeps its previous tables and
  // staging, which stay consistent with each other
  float *soft = nullptr;
  if (p->user_dim > 0) {
    const size_t ct = (size_t)(e->dm.Hq + 2 * e->dm.Hkv) * e->dm.d;
    const size_t n = (size_t)gr::kSoftSplit * (p->embed_dim + e->dm.L * ct);
    if (hipMalloc((void **)&soft, n * sizeof(float)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GR_E_OUT_OF_MEMORY, "soft-token staging");
    }
  }
  if (e->pf_soft) {
    if ((r = check_dev(e, hipDeviceSynchronize(), "sync")) != GR_OK) {
      if (soft) (void)hipFree(soft);
      return r;
    }
    (void)hipFree(e->pf_soft);
  }
  e->pf_soft = soft;
  e->pf = *p;
  e->has_pf = true;
  return GR_OK;
}

gr_status gr_ctx_prefill(gr_engine *e, int64_t rid, const int32_t *tokens, int32_t N, int32_t soft_pos,
                         const float *u, int32_t W, void *kn, void *vtn, void *q_out, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!e->has_pf) return fail(GR_E_BAD_STATE, "no prefill tables (gr_engine_set_prefill)");
  if (!tokens) return fail(GR_E_INVALID_ARG, "null tokens");
  if (N < 1) return fail(GR_E_INVALID_ARG, "ctx_len must be >= 1");
  if (W < 1 || W > e->dm.W_max) return fail(GR_E_INVALID_ARG, "beam_width must be in [1, max_beam_width]");
  if (soft_pos < -1 || soft_pos >= N) return fail(GR_E_INVALID_ARG, "soft_pos must be -1 or in [0, ctx_len)");
  if (soft_pos >= 0 && e->pf.user_dim < 1) return fail(GR_E_BAD_STATE, "no soft-token projection set");
  if (soft_pos >= 0 && !u) return fail(GR_E_INVALID_ARG, "null user vector");
  if ((kn == nullptr) != (vtn == nullptr)) return fail(GR_E_INVALID_ARG, "k_native and vt_native go together");
  if (((uintptr_t)kn | (uintptr_t)vtn) & 15u) return fail(GR_E_INVALID_ARG, "k_native and vt_native must be 16-byte aligned");
  if (e->reqs.count(rid)) return fail(GR_E_INVALID_ARG, "request id already loaded");
  if (e->free_slots.empty()) return fail(GR_E_OUT_OF_MEMORY, "no free request slot (max_requests)");
  for (int32_t n = 0; n < N; ++n)
    if (n != soft_pos && (tokens[n] < 0 || tokens[n] >= e->pf.vocab))
      return fail(GR_E_INVALID_ARG, "token id outside [0, vocab)");
  const int Np = gr_ctx_padded_len(N);
  hipStream_t st = (hipStream_t)stream;
  gr_status r;
  // token staging: the pinned buffer is reused once its last upload has run
  if (e->pf_ev_used && (r = check_dev(e, hipEventSynchronize(e->pf_ev), "prefill staging")) != GR_OK) return r;
  if (N > e->pf_tok_cap) {
    const int64_t cap = std::max<int64_t>(N, 2 * e->pf_tok_cap);
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
    if (e->pf_tok_host) (void)hipHostFree(e->pf_tok_host);
    if (e->pf_tok_dev) (void)hipFree(e->pf_tok_dev);
    e->pf_tok_host = nullptr;
    e->pf_tok_dev = nullptr;
    e->pf_tok_cap = 0;
    if (hipHostMalloc((void **)&e->pf_tok_host, (size_t)cap * 4, hipHostMallocDefault) != hipSuccess ||
        hipMalloc((void **)&e->pf_tok_dev, (size_t)cap * 4) != hipSuccess) {
      (void)hipGetLastError();
      return fail(GR_E_OUT_OF_MEMORY, "prefill token staging");
    }
    e->pf_tok_cap = cap;
  }
  std::memcpy(e->pf_tok_host, tokens, (size_t)N * 4);
  if (soft_pos >= 0) e->pf_tok_host[soft_pos] = 0;
  gr_engine::Req R;
  R.N = N;
  R.Np = Np;
  R.W = W;
  if (kn) {
    R.adopt = true;
    R.k = kn;
    R.vt = vtn;
  } else {
    int64_t off;
    if (!pool_alloc(e, Np, &off)) return fail(GR_E_OUT_OF_MEMORY, "context pool exhausted (max_ctx_tokens)");
    R.pool_off = off;
    uint8_t *dk = e->ws + e->off_pool + (size_t)off * e->pool_tok_bytes;
    R.k = dk;
    R.vt = dk + (size_t)e->dm.L * e->dm.Hkv * Np * e->dm.d * e->elem;
    if (e->v16) R.vt16 = dk + (size_t)2 * e->dm.L * e->dm.Hkv * Np * e->dm.d * e->elem;
  }
  R.slot = e->free_slots.back();
  uint8_t *sb = e->ws + e->off_slots + (size_t)R.slot * e->sl.slot_bytes;
  const int L = e->dm.L, Hq = e->dm.Hq, Hkv = e->dm.Hkv, d = e->dm.d;
  float *part = e->pf_soft ? e->pf_soft + (size_t)gr::kSoftSplit * e->pf.embed_dim : nullptr;
  auto run = [&]() -> gr_status {
    gr_status q;
    if ((q = check_dev(e, hipMemcpyAsync(e->pf_tok_dev, e->pf_tok_host, (size_t)N * 4, hipMemcpyHostToDevice, st),
                       "token upload")) != GR_OK)
      return q;
    if ((q = check_dev(e, hipEventRecord(e->pf_ev, st), "prefill staging")) != GR_OK) return q;
    e->pf_ev_used = true;
    if (soft_pos >= 0 &&
        (q = check_dev(e, gr::launch_soft_token(u, e->pf.proj, e->pf.user_dim, e->pf.embed_dim, e->pf.w_q, e->pf.w_k,
                                                e->pf.w_v, L, Hq * d, Hkv * d, e->pf_soft, part, st),
                       "soft token")) != GR_OK)
      return q;
    // the last query first: its launch also clears the maxima the context launch folds into
    const int last = (soft_pos == N - 1) ? -1 : tokens[N - 1];
    if ((q = check_dev(e, gr::launch_prefill_q(e->elem, e->pf.tok_q, last, nullptr, part, L, Hq, Hkv, d, e->pf.vocab,
                                               sb + e->sl.q_last, q_out, (float *)(sb + e->sl.knmax),
                                               (float *)(sb + e->sl.vscale), st),
                       "prefill query")) != GR_OK)
      return q;
    // the context in the native layout, with its key-norm bounds and value scales
    if ((q = check_dev(e, gr::launch_prefill_ctx(e->elem, e->pf.tok_k, e->pf.tok_v, e->pf_tok_dev, N, Np, soft_pos,
                                                 part, L, Hq, Hkv, d, e->pf.vocab, const_cast<void *>(R.k),
                                                 const_cast<void *>(R.vt), (float *)(sb + e->sl.knmax),
                                                 (float *)(sb + e->sl.vscale), st),
                       "prefill")) != GR_OK)
      return q;
    return R.vt16 ? check_dev(e, gr::launch_load_v16(R.vt, const_cast<void *>(R.vt16), (float *)(sb + e->sl.vscale), L,
                                                     Hkv, d, Np, st),
                              "float16 V")
                  : GR_OK;
  };
  if ((r = run()) != GR_OK) {
    if (!R.adopt) pool_free(e, R.pool_off, Np);
    return r;
  }
  if ((r = check_dev(e, gr::launch_init_slots(e->dev, &R.slot, 1, st), "slot init")) != GR_OK) return r;
  e->free_slots.pop_back();
  e->reqs[rid] = R;
  return GR_OK;
}

gr_status gr_ctx_prefill_noalloc(gr_engine *e, int64_t rid, const int32_t *tokens_dev, int32_t N, int32_t soft_pos,
                                 const float *u, int32_t W, void *kn, void *vtn, void *q_out, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!e->has_pf) return fail(GR_E_BAD_STATE, "no prefill tables (gr_engine_set_prefill)");
  if (!tokens_dev) return fail(GR_E_INVALID_ARG, "null tokens");
  if (N < 1) return fail(GR_E_INVALID_ARG, "ctx_len must be >= 1");
  if (W < 1 || W > e->dm.W_max) return fail(GR_E_INVALID_ARG, "beam_width must be in [1, max_beam_width]");
  if (soft_pos < -1 || soft_pos >= N) return fail(GR_E_INVALID_ARG, "soft_pos must be -1 or in [0, ctx_len)");
  if (soft_pos >= 0 && e->pf.user_dim < 1) return fail(GR_E_BAD_STATE, "no soft-token projection set");
  if (soft_pos >= 0 && !u) return fail(GR_E_INVALID_ARG, "null user vector");
  if ((kn == nullptr) != (vtn == nullptr)) return fail(GR_E_INVALID_ARG, "k_native and vt_native go together");
  if (((uintptr_t)kn | (uintptr_t)vtn) & 15u) return fail(GR_E_INVALID_ARG, "k_native and vt_native must be 16-byte aligned");
  if (e->reqs.count(rid)) return fail(GR_E_INVALID_ARG, "request id already loaded");
  if (e->free_slots.empty()) return fail(GR_E_OUT_OF_MEMORY, "no free request slot (max_requests)");
  const int L = e->dm.L, Hq = e->dm.Hq, Hkv = e->dm.Hkv, d = e->dm.d;
  float *part = nullptr;
  if (soft_pos >= 0) {
    const size_t need = (size_t)gr::kSoftSplit * ((size_t)e->pf.embed_dim + (size_t)L * (Hq + 2 * Hkv) * d);
    if (need > gr::kPrefillScratchFloats)
      return fail(GR_E_UNSUPPORTED, "the soft token's partial sums (" + std::to_string(need * 4) +
                                        " bytes) exceed the fixed 4 MiB device array of the allocation-free prefill");
    part = e->noalloc_scratch + (size_t)gr::kSoftSplit * e->pf.embed_dim;
  }
  const int Np = gr_ctx_padded_len(N);
  hipStream_t st = (hipStream_t)stream;
  gr_engine::Req R;
  R.N = N;
  R.Np = Np;
  R.W = W;
  if (kn) {
    R.adopt = true;
    R.k = kn;
    R.vt = vtn;
  } else {
    int64_t off;
    if (!pool_alloc(e, Np, &off)) return fail(GR_E_OUT_OF_MEMORY, "context pool exhausted (max_ctx_tokens)");
    R.pool_off = off;
    uint8_t *dk = e->ws + e->off_pool + (size_t)off * e->pool_tok_bytes;
    R.k = dk;
    R.vt = dk + (size_t)L * Hkv * Np * d * e->elem;
    if (e->v16) R.vt16 = dk + (size_t)2 * L * Hkv * Np * d * e->elem;
  }
  R.slot = e->free_slots.back();
  uint8_t *sb = e->ws + e->off_slots + (size_t)R.slot * e->sl.slot_bytes;
  auto run = [&]() -> gr_status {
    gr_status q;
    if (soft_pos >= 0 &&
        (q = check_dev(e, gr::launch_soft_token(u, e->pf.proj, e->pf.user_dim, e->pf.embed_dim, e->pf.w_q, e->pf.w_k,
                                                e->pf.w_v, L, Hq * d, Hkv * d, e->noalloc_scratch, part, st),
                       "soft token")) != GR_OK)
      return q;
    // the last query first (its id read on the device): it also clears the bound maxima
    const bool soft_last = soft_pos == N - 1;
    if ((q = check_dev(e, gr::launch_prefill_q(e->elem, e->pf.tok_q, -1, soft_last ? nullptr : tokens_dev + (N - 1),
                                               part, L, Hq, Hkv, d, e->pf.vocab, sb + e->sl.q_last, q_out,
                                               (float *)(sb + e->sl.knmax), (float *)(sb + e->sl.vscale), st),
                       "prefill query")) != GR_OK)
      return q;
    if ((q = check_dev(e, gr::launch_prefill_ctx(e->elem, e->pf.tok_k, e->pf.tok_v, tokens_dev, N, Np, soft_pos, part,
                                                 L, Hq, Hkv, d, e->pf.vocab, const_cast<void *>(R.k),
                                                 const_cast<void *>(R.vt), (float *)(sb + e->sl.knmax),
                                                 (float *)(sb + e->sl.vscale), st),
                       "prefill")) != GR_OK)
      return q;
    return R.vt16 ? check_dev(e, gr::launch_load_v16(R.vt, const_cast<void *>(R.vt16), (float *)(sb + e->sl.vscale), L,
                                                     Hkv, d, Np, st),
                              "float16 V")
                  : GR_OK;
  };
  gr_status r;
  if ((r = run()) != GR_OK) {
    if (!R.adopt) pool_free(e, R.pool_off, Np);
    return r;
  }
  if ((r = check_dev(e, gr::launch_init_slots(e->dev, &R.slot, 1, st), "slot init")) != GR_OK) return r;
  e->free_slots.pop_back();
  e->reqs[rid] = R;
  return GR_OK;
}

gr_status gr_ctx_kv_load(gr_engine *e, int64_t rid, int32_t N, int32_t W, const void *k, const void *v,
                         const void *q_last, uint32_t flags, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!k || !v || !q_last) return fail(GR_E_INVALID_ARG, "null k, v or q_last");
  if (((uintptr_t)k | (uintptr_t)v) & 15u) return fail(GR_E_INVALID_ARG, "k and v must be 16-byte aligned");
  if (N < 1) return fail(GR_E_INVALID_ARG, "ctx_len must be >= 1");
  if (W < 1 || W > e->dm.W_max) return fail(GR_E_INVALID_ARG, "beam_width must be in [1, max_beam_width]");
  if (flags & ~GR_LOAD_ADOPT) return fail(GR_E_INVALID_ARG, "unknown load flag");
  if (e->reqs.count(rid)) return fail(GR_E_INVALID_ARG, "request id already loaded");
  if (e->free_slots.empty()) return fail(GR_E_OUT_OF_MEMORY, "no free request slot (max_requests)");
  const int Np = gr_ctx_padded_len(N);
  gr_engine::Req R;
  R.N = N;
  R.Np = Np;
  R.W = W;
  hipStream_t st = (hipStream_t)stream;
  gr_status r;
  const bool adopt = (flags & GR_LOAD_ADOPT) != 0;
  if (adopt) {
    R.adopt = true;
    R.k = k;
    R.vt = v;
  } else {
    int64_t off;
    if (!pool_alloc(e, Np, &off)) return fail(GR_E_OUT_OF_MEMORY, "context pool exhausted (max_ctx_tokens)");
    R.pool_off = off;
    uint8_t *dk = e->ws + e->off_pool + (size_t)off * e->pool_tok_bytes;
    R.k = dk;
    R.vt = dk + (size_t)e->dm.L * e->dm.Hkv * Np * e->dm.d * e->elem;
    if (e->v16) R.vt16 = dk + (size_t)2 * e->dm.L * e->dm.Hkv * Np * e->dm.d * e->elem;
  }
  R.slot = e->free_slots.back();
  uint8_t *sb = e->ws + e->off_slots + (size_t)R.slot * e->sl.slot_bytes;
  // native layout (unless adopted), key-norm bounds and value scales in one pass over the context
  if ((r = check_dev(e, gr::launch_load_ctx(k, v, const_cast<void *>(R.k), const_cast<void *>(R.vt), !adopt,
                                            e->dm.L, e->dm.Hkv, N, Np, e->dm.d, e->elem, (float *)(sb + e->sl.knmax),
                                            (float *)(sb + e->sl.vscale), st),
                     "context load")) != GR_OK ||
      (R.vt16 && (r = check_dev(e, gr::launch_load_v16(R.vt, const_cast<void *>(R.vt16), (float *)(sb + e->sl.vscale),
                                                       e->dm.L, e->dm.Hkv, e->dm.d, Np, st),
                                "float16 V")) != GR_OK)) {
    if (!adopt) pool_free(e, R.pool_off, Np);
    return r;
  }
  const size_t qbytes = e->dm.chain ? (size_t)e->dm.Hq * e->dm.d * 4 : (size_t)e->dm.L * e->dm.Hq * e->dm.d * e->elem;
  if ((r = check_dev(e, hipMemcpyAsync(sb + e->sl.q_last, q_last, qbytes, hipMemcpyDeviceToDevice, st), "q_last copy")) !=
      GR_OK)
    return r;
  if ((r = check_dev(e, gr::launch_init_slots(e->dev, &R.slot, 1, st), "slot init")) != GR_OK) return r;
  e->free_slots.pop_back();
  e->reqs[rid] = R;
  return GR_OK;
}

gr_status gr_request_release(gr_engine *e, int64_t rid) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  auto it = e->reqs.find(rid);
  if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
  if (!it->second.adopt && it->second.pool_off >= 0) pool_free(e, it->second.pool_off, it->second.Np);
  e->free_slots.push_back(it->second.slot);
  e->reqs.erase(it);
  return GR_OK;
}

gr_status gr_request_reset_batch(gr_engine *e, const int64_t *ids, int32_t n, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!ids || n < 1) return fail(GR_E_INVALID_ARG, "need at least one request id");
  std::vector<gr_engine::Req *> rs((size_t)n);
  std::vector<int32_t> slots((size_t)n);
  for (int i = 0; i < n; ++i) {
    auto it = e->reqs.find(ids[i]);
    if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
    rs[(size_t)i] = &it->second;
    slots[(size_t)i] = it->second.slot;
  }
  gr_status r;
  for (int i0 = 0; i0 < n; i0 += gr::kGatherMax) {
    const int m = std::min(gr::kGatherMax, n - i0);
    if ((r = check_dev(e, gr::launch_init_slots(e->dev, slots.data() + i0, m, (hipStream_t)stream), "slot init")) !=
        GR_OK)
      return r;
  }
  for (auto *R : rs) {
    R->level = 0;
    R->n_bound = 1;
    R->n_items = 0;
  }
  return GR_OK;
}

gr_status gr_request_reset(gr_engine *e, int64_t rid, void *stream) {
  return gr_request_reset_batch(e, &rid, 1, stream);
}

namespace {
// One decode step (label_order == nullptr), or the label step of gr_score_items_labels: every
// listed request at level n_levels, its beams' last codes run as tokens and the label head
// instead of logits and selection; *label_order receives the request index of each descriptor
// (the row order of the label output).
gr_status step_impl(gr_engine *e, const int64_t *ids, int32_t n, void *stream, std::vector<int> *label_order) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!ids || n < 1) return fail(GR_E_INVALID_ARG, "need at least one request id");
  if (n > e->opts.max_requests) return fail(GR_E_INVALID_ARG, "more ids than max_requests");
  const gr::Dims &d = e->dm;
  std::vector<gr_engine::Req *> rs((size_t)n);
  {
    std::unordered_set<int64_t> seen;
    for (int i = 0; i < n; ++i) {
      if (!seen.insert(ids[i]).second) return fail(GR_E_INVALID_ARG, "duplicate request id in one step");
      auto it = e->reqs.find(ids[i]);
      if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
      if (label_order ? it->second.level != d.levels : it->second.level >= d.levels)
        return fail(GR_E_BAD_STATE, label_order ? "the label step follows the last level" : "request already decoded every level");
      rs[(size_t)i] = &it->second;
    }
  }
  hipStream_t st = (hipStream_t)stream;
  gr_status r;
  // ---- work decomposition: requests grouped by context-attention variant (one launch per
  // group); within a group, enough split-K token ranges to fill the chip
  // A first-level step (every request at level 0) runs all layers' context attention in one
  // launch: each layer's query is an input there.  Needs room for every layer's partials in
  // one partial buffer and for the per-layer outputs in the other.
  // no launch covers two layers (the layer chain: every layer reads the previous one's output)
  const bool per_layer = (e->opts.flags & GR_ENGINE_PER_LAYER) != 0 || d.chain;
  bool first_fused = !per_layer && d.dtype == 1 && d.d == 128 && d.L > 1 && (int64_t)d.L <= (int64_t)d.S_max * d.W_max;
  for (int i = 0; i < n && first_fused; ++i) first_fused = rs[(size_t)i]->level == 0;
  std::vector<int> kind((size_t)n);
  for (int i = 0; i < n; ++i)
    kind[(size_t)i] = d.dtype == 1 ? gr::ctx_kind_for(rs[(size_t)i]->n_bound * d.g, rs[(size_t)i]->N, d.d) : 0;
  // A step whose row blocks fill the chip (three quarters of the resident workgroups) over
  // min(L, S_max) layers runs without split partials: each workgroup covers the whole context
  // of one layer and finishes it, every layer's output goes to its own fp16 hidden partial,
  // and the partials are summed into h at the end.  Wide requests run on the 8-wave kernel;
  // every narrower one (level-0 beams included) on the two-wave stream kernel in 64-row
  // blocks, so a step that mixes levels (continuous batching) stays on this path.
  const int lg_max = per_layer ? 1 : std::min(d.L, d.S_max);
  auto full_ctx_kind = [](int k) { return (k & 0xFF) == 8 ? k : (2 | gr::kCtxHiLo); };
  bool layered = d.dtype == 1 && d.d == 128 && !first_fused && !d.chain;
  double fill = 0.0;  // resident-workgroup rounds the step's row blocks fill over lg_max layers
  for (int i = 0; i < n && layered; ++i) {
    const int k = full_ctx_kind(kind[(size_t)i]);
    const int64_t units = (int64_t)d.Hkv * ceil_div((int64_t)rs[(size_t)i]->n_bound * d.g, gr::ctx_rows_per_wg(k));
    fill += (double)units * lg_max / ((k & 0xFF) == 8 ? 256.0 : 512.0);
  }
  layered = layered && fill >= 0.75;
  if (layered)
    for (int i = 0; i < n; ++i) kind[(size_t)i] = full_ctx_kind(kind[(size_t)i]);
  // a split-K step of first-level requests only (one beam each, head_dim 128) runs on the
  // 8-wave kernel too: its 64-token tiles fetch whole 128-byte lines of V^T, and a quarter of
  // the ranges halves the merge (headline level 0, same box: 37.5 against 38.2 us per layer,
  // layer finish 13.2 against 13.7 us); steps that mix levels keep the one-wave kernel in a
  // group of its own
  if (!layered && !first_fused && d.dtype == 1 && d.d == 128) {
    bool all_first = true;
    for (int i = 0; i < n; ++i) all_first = all_first && rs[(size_t)i]->level == 0 && (kind[(size_t)i] & 0xFF) == 1;
    if (all_first)
      for (int i = 0; i < n; ++i) kind[(size_t)i] = 8;
  }
  bool any_hparts = false;
  // split-K steps of bf16 models finish layer l inside the launch of layer l+1 (the model
  // stand-in's layers do not read each other's output); with one layer per launch every layer
  // is finished by its own merge launch before the next layer starts
  const bool defer = d.dtype == 1 && !per_layer;
  std::vector<int> order((size_t)n);
  for (int i = 0; i < n; ++i) order[(size_t)i] = i;
  // within a variant, longest context first: workgroups are dealt out in order as compute
  // units free up, so the long ones start first and the short ones fill the end
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    if (kind[(size_t)a] != kind[(size_t)b]) return kind[(size_t)a] < kind[(size_t)b];
    return rs[(size_t)a]->N > rs[(size_t)b]->N;
  });
  struct Group { int kind, start, count, wgs, lgroups, merge0, merge_wgs, fin0, fin_wgs; };
  std::vector<Group> groups;
  for (int i = 0; i < n; ++i) {
    const int k = kind[(size_t)order[(size_t)i]];
    if (groups.empty() || groups.back().kind != k) groups.push_back({k, i, 0, 0, 0, 0, 0, 0, 0});
    groups.back().count++;
  }
  const int slot_i = e->ring;
  e->ring = (e->ring + 1) % kRing;
  if (e->event_used[slot_i]) {
    if ((r = check_dev(e, hipEventSynchronize(e->events[slot_i]), "descriptor ring")) != GR_OK) return r;
  }
  gr::StepReq *hw = e->pinned[slot_i];
  int wg_merge = 0, wg_fin = 0, wg_logits = 0, wg_lsm = 0, max_cand = 0, row_acc = 0;
  for (Group &G : groups) {
    const int nw = G.kind & 0xFF;
    const int rows_wg = d.dtype == 1 ? gr::ctx_rows_per_wg(G.kind) : 32;
    // workgroups per launch: one per compute unit for the 8-wave kernel, two per unit for the
    // one- and two-wave streaming kernels (head_dim 128; their LDS ring allows two), else
    // about two per compute unit of 4 waves
    const int want = d.dtype == 1 ? (nw == 8 ? 256 : nw == 4 ? 512 : nw == 2 ? (d.d == 128 ? 512 : 1024)
                                                                           : d.d == 128 ? 512 : 2048)
                                  : 256;
    int64_t units = 0;
    for (int i = G.start; i < G.start + G.count; ++i)
      units += (int64_t)d.Hkv * ceil_div((int64_t)rs[(size_t)order[(size_t)i]]->n_bound * d.g, rows_wg);
    int lgroups = 0;
    if (layered) {
      // about seven rounds of workgroups per launch (later rounds start on the units the
      // earlier ones free), the layers split as evenly as possible over the launches: few
      // launch ends, and no short last launch.  Same-box, headline workload: 83.9 us per layer
      // with two rounds, 82.5-83.2 with seven or fourteen; 8+8+8+4 layers measured 95.2.
      int64_t target =
          std::min<int64_t>(d.L, std::max<int64_t>(1, (7 * want + units - 1) / std::max<int64_t>(units, 1)));
      if (e->opts.max_layers_per_launch > 0) target = std::min<int64_t>(target, e->opts.max_layers_per_launch);
      if (per_layer) target = 1;
      const int64_t launches = (d.L + target - 1) / target;
      lgroups = (int)((d.L + launches - 1) / launches);
      G.lgroups = lgroups;
      any_hparts = true;  // every layer's output goes to its own partial
    }
    int wg_ctx = 0;
    for (int i = G.start; i < G.start + G.count; ++i) {
      gr_engine::Req *R = rs[(size_t)order[(size_t)i]];
      gr::StepReq &w = hw[i];
      std::memset(&w, 0, sizeof(w));
      w.ctx_k = R->k;
      w.ctx_vt = R->vt;
      w.ctx_vt16 = R->vt16;
      w.ctx_lstride = (int64_t)d.Hkv * R->Np * d.d;
      w.N = R->N;
      w.Np = R->Np;
      w.slot = R->slot;
      w.level = R->level;
      w.n_items = R->n_items;
      w.W = R->W;
      w.n_bound = R->n_bound;
      const int rows = R->n_bound * d.g;
      w.rows_b = rows;
      w.row_blocks = ceil_div(rows, rows_wg);
      // split-K: enough workgroups, at least two tiles per range, and no more partial rows
      // than the slot holds (Hkv * S_max * W_max * g)
      int S = layered ? 1 : (int)std::max<int64_t>(1, (want + units - 1) / std::max<int64_t>(units, 1));
      S = std::min(S, std::max(1, ceil_div(R->N, 2 * gr::kTileTok)));
      S = (int)std::min<int64_t>(S, std::max<int64_t>(1, (int64_t)d.S_max * d.W_max * d.g / rows));
      S = std::min(S, 256);
      if (first_fused) S = std::max(1, std::min<int>(S, (int)((int64_t)d.S_max * d.W_max * d.g / ((int64_t)d.L * rows))));
      int tps = (int)align_up((size_t)ceil_div(R->N, S), gr::kTileTok);
      S = ceil_div(R->N, tps);
      if (S > 1) {
        // the last range takes the rest: of the two tile multiples around N/S, the one whose
        // longest range has fewer 32-token sub-tiles (5000 tokens in two: 2496 + 2504, not
        // 2560 + 2440), each range keeping at least two tiles
        const int lo = R->N / S / gr::kTileTok * gr::kTileTok;
        auto longest = [&](int t) { return std::max(ceil_div(t, 32), ceil_div(R->N - (int64_t)(S - 1) * t, 32)); };
        if (lo >= 2 * gr::kTileTok && longest(lo) < longest(tps)) tps = lo;
      }
      w.splits = S;
      w.tps = tps;
      w.lgroups = lgroups;
      w.defer_finish = defer ? 1 : 0;
      w.row0 = row_acc;  // the layer chain's packed rows: each request at a multiple of 32
      row_acc += (int)align_up((size_t)R->n_bound, 32);
      w.wg_ctx = wg_ctx;
      if (layered)
        wg_ctx += (int)align_up((size_t)d.Hkv * lgroups, 8) * w.row_blocks;
      else if (d.dtype == 1)
        wg_ctx += (int)align_up((size_t)d.Hkv * S, 8) * w.row_blocks;  // multiple of 8: XCD-aware order
      else
        wg_ctx += ceil_div((int64_t)d.Hkv * rows * S, 4);
      w.wg_merge = wg_merge;
      if (i == G.start) G.merge0 = wg_merge;
      G.merge_wgs += R->n_bound;
      wg_merge += R->n_bound;
      // the bf16 layer finish: workgroups over (row block, kv head)
      const int fin = d.Hkv * ceil_div(rows, gr::fin_rows_per_wg(d.d));
      w.wg_fin = wg_fin;
      if (i == G.start) G.fin0 = wg_fin;
      G.fin_wgs += fin;
      wg_fin += fin;
      w.wg_logits = wg_logits;
      wg_logits += ceil_div(R->n_bound, 64) * ceil_div(d.V, 64) * gr::kLogitsKS;
      w.wg_lsm = wg_lsm;
      wg_lsm += ceil_div(R->n_bound, gr::kLsmRows);
      // two-stage top-K when the chunks' kept keys fit the second stage's registers
      w.sel2 = R->n_items == 0 &&
               (int64_t)ceil_div(R->n_bound, gr::kLsmRows) * R->W <= (int64_t)gr::kTopkThreads * gr::kSel2CPT;
      max_cand = std::max(max_cand, R->n_bound * d.V);
    }
    G.wgs = wg_ctx;
  }
  const bool graph = (e->opts.flags & GR_ENGINE_GRAPH) && !e->prof && !d.debug_attn && !label_order;
  gr::StepReq *dw = (gr::StepReq *)(e->ws + e->off_work + e->work_bytes * (size_t)(graph ? kRing : slot_i));
  if (graph && e->gdone_used &&
      (r = check_dev(e, hipStreamWaitEvent(st, e->gdone_ev, 0), "graph order")) != GR_OK)
    return r;
  if ((r = check_dev(e, hipMemcpyAsync(dw, hw, sizeof(gr::StepReq) * (size_t)n, hipMemcpyHostToDevice, st),
                     "descriptor upload")) != GR_OK)
    return r;
  if ((r = check_dev(e, hipEventRecord(e->events[slot_i], st), "descriptor ring")) != GR_OK) return r;
  e->event_used[slot_i] = true;
  // graph replay: the step's shape (every value the launch sequence below depends on)
  std::vector<int64_t> key;
  hipGraphExec_t exec = nullptr;
  if (graph) {
    key = {n, first_fused, layered, per_layer, defer, any_hparts, d.chain, wg_merge, wg_fin, wg_logits, wg_lsm,
           max_cand, row_acc, (int64_t)groups.size()};
    for (const Group &G : groups)
      key.insert(key.end(), {G.kind, G.start, G.count, G.wgs, G.lgroups, G.merge0, G.merge_wgs, G.fin0, G.fin_wgs});
    auto it = e->graphs.find(key);
    if (it != e->graphs.end()) exec = it->second;
  }
  // the launch sequence, enqueued on `st` (the caller's stream, or the capture stream)
  auto enqueue = [&](hipStream_t st) -> gr_status {
  gr_status r;
  int plevel = rs[0]->level;
  for (auto *R : rs)
    if (R->level != plevel) plevel = d.levels;
  const bool pon = prof_reserve(e, 2 * ((d.chain ? 8 : 2) * d.L + 4));
  auto pk = [&](int kind) { return pon && ((e->prof_mask >> kind) & 1u) != 0; };  // this kind is timed
  int step_start = -1;
  if (first_fused) {
    const auto pc = prof_pair(e, pk(GR_PROF_CTX_ATTN));
    step_start = pc.first;
    if ((r = check_dev(e, gr::launch_ctx_attn_first_level(e->dev, dw, n, groups[0].wgs, st,
                                                          prof_ev(e, pc.first, pc.second)),
                       "context attention")) != GR_OK)
      return r;
    prof_record(e, GR_PROF_CTX_ATTN, plevel, pc, d.L);
    const auto pm = prof_pair(e, pk(GR_PROF_BEAM_MERGE));
    if ((r = check_dev(e, gr::launch_finish_first_level(e->dev, dw, n, st, prof_ev(e, pm.first, pm.second)),
                       "first-level finish")) != GR_OK)
      return r;
    prof_record(e, GR_PROF_BEAM_MERGE, plevel, pm);
  }
  // several variant groups: each group's launches depend only on that group's earlier ones,
  // so group gi runs on stream gi mod 4 (the caller's stream or an engine-owned one), forked
  // from and joined into the caller's stream; a span record then uses marker events on it
  const int nstreams =
      d.dtype == 1 && !first_fused && !d.chain ? (int)std::min<size_t>(kAuxStreams + 1, groups.size()) : 1;
  auto group_stream = [&](size_t gi) { return gi % (kAuxStreams + 1) == 0 ? st : e->aux[gi % (kAuxStreams + 1) - 1]; };
  auto fork = [&]() -> gr_status {
    gr_status q;
    if ((q = check_dev(e, hipEventRecord(e->fork_ev, st), "stream fork")) != GR_OK) return q;
    for (int i = 0; i + 1 < nstreams; ++i)
      if ((q = check_dev(e, hipStreamWaitEvent(e->aux[i], e->fork_ev, 0), "stream fork")) != GR_OK) return q;
    return GR_OK;
  };
  auto join = [&]() -> gr_status {
    gr_status q;
    for (int i = 0; i + 1 < nstreams; ++i) {
      if ((q = check_dev(e, hipEventRecord(e->join_ev[i], e->aux[i]), "stream join")) != GR_OK) return q;
      if ((q = check_dev(e, hipStreamWaitEvent(st, e->join_ev[i], 0), "stream join")) != GR_OK) return q;
    }
    return GR_OK;
  };
  // the finish of one layer for requests [i0, i0 + m) of the step (bf16: the phased finish
  // kernel over row blocks; float32: one workgroup per beam)
  auto finish = [&](int i0, int m, int layer, int fin_wgs, int fin0, int merge_wgs, int merge0, hipStream_t s,
                    gr::LaunchEv ev) -> hipError_t {
    if (d.dtype == 1) return gr::launch_finish_layer(e->dev, dw + i0, m, layer, fin_wgs, s, ev, fin0);
    return gr::launch_beam_merge(e->dev, dw + i0, m, layer, merge_wgs, s, ev, merge0);
  };
  auto marker = [&](int ev) -> gr_status {
    return ev >= 0 ? check_dev(e, hipEventRecord(e->prof_ev[(size_t)ev], st), "profiling event") : GR_OK;
  };
  if (layered) {
    const auto pc = prof_pair(e, pk(GR_PROF_CTX_ATTN));
    step_start = pc.first;
    if (nstreams > 1 && ((r = marker(pc.first)) != GR_OK || (r = fork()) != GR_OK)) return r;
    int disp = 0;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group &G = groups[gi];
      for (int l0 = 0; l0 < d.L; l0 += G.lgroups, ++disp) {
        const bool first = gi == 0 && l0 == 0, last = gi + 1 == groups.size() && l0 + G.lgroups >= d.L;
        const gr::LaunchEv ev = nstreams > 1 ? gr::LaunchEv{} : prof_ev(e, first ? pc.first : -1, last ? pc.second : -1);
        if ((r = check_dev(e, gr::launch_ctx_attn_layered(e->dev, dw + G.start, G.count, l0, G.wgs, G.kind,
                                                          group_stream(gi), ev),
                           "context attention")) != GR_OK)
          return r;
      }
    }
    if (nstreams > 1 && ((r = join()) != GR_OK || (r = marker(pc.second)) != GR_OK)) return r;
    prof_record(e, GR_PROF_CTX_ATTN, plevel, pc, d.L, disp);
    if (any_hparts) {
      const auto pm = prof_pair(e, pk(GR_PROF_BEAM_MERGE));
      if ((r = check_dev(e, gr::launch_sum_hparts(e->dev, dw, n, st, prof_ev(e, pm.first, pm.second)),
                         "layer-group sum")) != GR_OK)
        return r;
      prof_record(e, GR_PROF_BEAM_MERGE, plevel, pm);
    }
  }
  // split-K steps with several groups: the same streams; layer l of a group is finished inside
  // the group's launch of layer l+1 and the last layer of every request after the join, or (one
  // layer per launch) by the group's own merge launch after each layer; the span record then
  // holds the merges too
  const bool multi = !first_fused && !layered && nstreams > 1;
  if (multi) {
    const auto pc = prof_pair(e, pk(GR_PROF_CTX_ATTN));
    step_start = pc.first;
    if ((r = marker(pc.first)) != GR_OK || (r = fork()) != GR_OK) return r;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group &G = groups[gi];
      for (int l = 0; l < d.L; ++l) {
        if ((r = check_dev(e, gr::launch_ctx_attn(e->dev, dw + G.start, G.count, l, G.wgs, G.kind, group_stream(gi)),
                           "context attention")) != GR_OK)
          return r;
        if (!defer && (r = check_dev(e, finish(G.start, G.count, l, G.fin_wgs, G.fin0, G.merge_wgs, G.merge0,
                                               group_stream(gi), gr::LaunchEv{}),
                                     "beam attention/merge")) != GR_OK)
          return r;
      }
    }
    if ((r = join()) != GR_OK || (r = marker(pc.second)) != GR_OK) return r;
    prof_record(e, GR_PROF_CTX_ATTN, plevel, pc, d.L, d.L * (int)groups.size());
    if (defer) {
      const auto pm = prof_pair(e, pk(GR_PROF_BEAM_MERGE));
      if ((r = check_dev(e, finish(0, n, d.L - 1, wg_fin, 0, wg_merge, 0, st, prof_ev(e, pm.first, pm.second)),
                         "beam attention/merge")) != GR_OK)
        return r;
      prof_record(e, GR_PROF_BEAM_MERGE, plevel, pm);
    }
  }
  if (d.chain) {
    // the layer chain, one layer after another: q/k/v projection (k, v into BeamKV), context
    // attention (split-K, every variant group), the layer's finish (o rows), output projection
    // into the residual, the MLP's norm, gate/up with SwiGLU, down into the residual, the next
    // layer's norm; then the final norm into each request's hidden rows
    const int rows = (int)align_up((size_t)row_acc, 128);
    if (rows > e->chain_rows) return fail(GR_E_BAD_STATE, "step rows exceed the chain buffers");  // cannot happen
    auto rec = [&](int kind, std::pair<int, int> ab) { prof_record(e, kind, plevel, ab); };
    auto pn = prof_pair(e, pk(GR_PROF_NORM));
    step_start = pn.first;
    if ((r = check_dev(e, gr::launch_chain_start(e->dev, dw, n, rows, st, prof_ev(e, pn.first, pn.second)),
                       "chain start")) != GR_OK)
      return r;
    rec(GR_PROF_NORM, pn);
    const size_t D = (size_t)d.Hq * d.d;
    // every request at the first level (one live row each): the projections' few-row kernel
    int few = 2;
    for (int i = 0; i < n && few > 0; ++i)
      if (rs[(size_t)i]->n_bound != 1 || rs[(size_t)i]->level != 0) few = 0;
    for (int l = 0; l < d.L; ++l) {
      const bool lp = l % e->prof_stride == 0;  // this layer's launches are timed
      auto gemm = [&](int kind) -> gr_status {
        const auto pg = prof_pair(e, pk(GR_PROF_GEMM) && lp);
        gr_status q = check_dev(
            e, gr::launch_chain_gemm(e->dev, dw, n, rows, kind, l, few, st, prof_ev(e, pg.first, pg.second)),
            "chain projection");
        if (q == GR_OK) rec(GR_PROF_GEMM, pg);
        return q;
      };
      auto norm = [&](const float *g) -> gr_status {
        const auto pq = prof_pair(e, pk(GR_PROF_NORM) && lp);
        gr_status q = check_dev(e, gr::launch_chain_norm(e->dev, g, rows, st, prof_ev(e, pq.first, pq.second)),
                                "chain norm");
        if (q == GR_OK) rec(GR_PROF_NORM, pq);
        return q;
      };
      // debug engines keep a copy of the rows entering and leaving each projection
      const size_t crow = (size_t)rows;
      auto snap = [&](int which) -> gr_status {
        if (!d.debug_attn) return GR_OK;
        const gr::ChainDev &c = e->dev.ch;
        const size_t Dq = D, I = (size_t)c.I;
        const void *src = nullptr;
        size_t bytes = 0;
        switch (which) {
          case GR_CHAIN_X_IN: case GR_CHAIN_X_MID: case GR_CHAIN_X_OUT: src = c.x; bytes = crow * D * 4; break;
          case GR_CHAIN_XN_ATTN: case GR_CHAIN_XN_MLP: src = c.xn; bytes = crow * D * 2; break;
          case GR_CHAIN_Q: src = c.q; bytes = crow * Dq * 2; break;
          case GR_CHAIN_O: src = c.o; bytes = crow * Dq * 2; break;
          default: src = c.act; bytes = crow * I * 2; break;
        }
        return check_dev(e, hipMemcpyAsync(chain_dbg(e, l, which), src, bytes, hipMemcpyDeviceToDevice, st), "debug copy");
      };
      if ((r = snap(GR_CHAIN_X_IN)) != GR_OK || (r = snap(GR_CHAIN_XN_ATTN)) != GR_OK) return r;
      if ((r = gemm(gr::kChainQKV)) != GR_OK) return r;
      if ((r = snap(GR_CHAIN_Q)) != GR_OK) return r;
      const auto pc = prof_pair(e, pk(GR_PROF_CTX_ATTN) && lp);
      for (size_t gi = 0; gi < groups.size(); ++gi) {
        const Group &G = groups[gi];
        const gr::LaunchEv ev = prof_ev(e, gi == 0 ? pc.first : -1, gi + 1 == groups.size() ? pc.second : -1);
        if ((r = check_dev(e, gr::launch_ctx_attn(e->dev, dw + G.start, G.count, l, G.wgs, G.kind, st, ev),
                           "context attention")) != GR_OK)
          return r;
      }
      prof_record(e, GR_PROF_CTX_ATTN, plevel, pc, 1, (int)groups.size());
      const auto pm = prof_pair(e, pk(GR_PROF_BEAM_MERGE) && lp);
      if ((r = check_dev(e, finish(0, n, l, wg_fin, 0, wg_merge, 0, st, prof_ev(e, pm.first, pm.second)),
                         "layer finish")) != GR_OK)
        return r;
      rec(GR_PROF_BEAM_MERGE, pm);
      if ((r = snap(GR_CHAIN_O)) != GR_OK) return r;
      if ((r = gemm(gr::kChainO)) != GR_OK) return r;
      if ((r = snap(GR_CHAIN_X_MID)) != GR_OK) return r;
      if ((r = norm(e->chain.g_mlp + (size_t)l * D)) != GR_OK) return r;
      if ((r = snap(GR_CHAIN_XN_MLP)) != GR_OK) return r;
      if ((r = gemm(gr::kChainGateUp)) != GR_OK) return r;
      if ((r = snap(GR_CHAIN_ACT)) != GR_OK) return r;
      if ((r = gemm(gr::kChainDown)) != GR_OK) return r;
      if ((r = snap(GR_CHAIN_X_OUT)) != GR_OK) return r;
      if (l + 1 < d.L && (r = norm(e->chain.g_attn + (size_t)(l + 1) * D)) != GR_OK) return r;
    }
    pn = prof_pair(e, pk(GR_PROF_NORM));
    if ((r = check_dev(e, gr::launch_chain_final(e->dev, dw, n, rows, st, prof_ev(e, pn.first, pn.second)),
                       "chain final norm")) != GR_OK)
      return r;
    rec(GR_PROF_NORM, pn);
  }
  for (int l = 0; l < (first_fused || layered || multi || d.chain ? 0 : d.L); ++l) {
    const bool lp = l % e->prof_stride == 0;  // this layer's launches are timed
    const auto pc = prof_pair(e, pk(GR_PROF_CTX_ATTN) && lp);
    if (l == 0) step_start = pc.first;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group &G = groups[gi];
      const gr::LaunchEv ev = prof_ev(e, gi == 0 ? pc.first : -1, gi + 1 == groups.size() ? pc.second : -1);
      if ((r = check_dev(e, gr::launch_ctx_attn(e->dev, dw + G.start, G.count, l, G.wgs, G.kind, st, ev),
                         "context attention")) != GR_OK)
        return r;
    }
    prof_record(e, GR_PROF_CTX_ATTN, plevel, pc, 1, (int)groups.size());
    // float32 (and one layer per launch): finish every layer separately; otherwise layer l is
    // finished inside layer l+1's context kernel, and the last layer here
    if (!defer || l == d.L - 1) {
      const auto pm = prof_pair(e, pk(GR_PROF_BEAM_MERGE) && lp);
      if ((r = check_dev(e, finish(0, n, l, wg_fin, 0, wg_merge, 0, st, prof_ev(e, pm.first, pm.second)),
                         "beam attention/merge")) != GR_OK)
        return r;
      prof_record(e, GR_PROF_BEAM_MERGE, plevel, pm);
    }
  }
  if (label_order) {
    if ((r = check_dev(e, gr::launch_label_head(e->dev, dw, n, wg_merge, st), "label head")) != GR_OK) return r;
    label_order->assign(order.begin(), order.end());
    return GR_OK;
  }
  const auto pl = prof_pair(e, pk(GR_PROF_LOGITS));
  if ((r = check_dev(e, gr::launch_logits(e->dev, dw, n, wg_logits, st, prof_ev(e, pl.first, pl.second)),
                     "logits")) != GR_OK)
    return r;
  prof_record(e, GR_PROF_LOGITS, plevel, pl);
  const auto pt = prof_pair(e, pk(GR_PROF_TOPK));
  if ((r = check_dev(e, gr::launch_lsm(e->dev, dw, n, wg_lsm, st, prof_ev(e, pt.first, -1)), "log-softmax")) != GR_OK)
    return r;
  if ((r = check_dev(e, gr::launch_topk(e->dev, dw, n, max_cand, st, prof_ev(e, -1, pt.second)), "top-k")) != GR_OK)
    return r;
  prof_record(e, GR_PROF_TOPK, plevel, pt);
  if (step_start >= 0 && pt.second >= 0 && pk(GR_PROF_STEP)) prof_record(e, GR_PROF_STEP, plevel, {step_start, pt.second});
  return GR_OK;
  };
  if (!graph) {
    if ((r = enqueue(st)) != GR_OK || label_order) return r;
  } else {
    if (!exec) {
      // capture this shape once on the engine's own stream, then keep its executable graph
      if ((r = check_dev(e, hipStreamBeginCapture(e->cap_st, hipStreamCaptureModeThreadLocal), "graph capture")) !=
          GR_OK)
        return r;
      const gr_status q = enqueue(e->cap_st);
      hipGraph_t g = nullptr;
      const hipError_t ce = hipStreamEndCapture(e->cap_st, &g);
      if (q != GR_OK) {
        if (g) (void)hipGraphDestroy(g);
        return q;
      }
      if ((r = check_dev(e, ce, "graph capture")) != GR_OK) return r;
      const hipError_t ie = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if ((r = check_dev(e, ie, "graph instantiate")) != GR_OK) return r;
      if (e->graph_fifo.size() >= 64) {
        auto old = e->graphs.find(e->graph_fifo.front());
        if (old != e->graphs.end()) {
          (void)hipGraphExecDestroy(old->second);
          e->graphs.erase(old);
        }
        e->graph_fifo.pop_front();
      }
      e->graphs[key] = exec;
      e->graph_fifo.push_back(key);
      ++e->graph_captures;
    } else {
      ++e->graph_hits;
    }
    if ((r = check_dev(e, hipGraphLaunch(exec, st), "graph launch")) != GR_OK) return r;
    if ((r = check_dev(e, hipEventRecord(e->gdone_ev, st), "graph order")) != GR_OK) return r;
    e->gdone_used = true;
  }
  for (int i = 0; i < n; ++i)  // descriptor i belongs to request order[i]
    rs[(size_t)order[(size_t)i]]->last_row0 = hw[i].row0;
  for (auto *R : rs) {
    const int s = R->level;
    int64_t nb = std::min<int64_t>((int64_t)R->W, (int64_t)R->n_bound * d.V);
    nb = std::min<int64_t>(nb, e->nodes[s + 1]);
    if (R->n_items > 0) nb = R->n_items;  // scoring: one beam per candidate
    R->n_bound = (int)nb;
    R->level = s + 1;
  }
  return GR_OK;
}
}  // namespace

gr_status gr_beam_step(gr_engine *e, const int64_t *ids, int32_t n, void *stream) {
  return step_impl(e, ids, n, stream, nullptr);
}

namespace {
gr_status find_req(gr_engine *e, int64_t rid, gr_engine::Req **out) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  auto it = e->reqs.find(rid);
  if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
  *out = &it->second;
  return GR_OK;
}
uint8_t *slot_ptr(gr_engine *e, const gr_engine::Req *R) {
  return e->ws + e->off_slots + (size_t)R->slot * e->sl.slot_bytes;
}
gr_status d2h(gr_engine *e, void *dst, const void *src, size_t bytes, hipStream_t st) {
  return check_dev(e, hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, st), "device to host copy");
}
}  // namespace

gr_status gr_beams_get_batch_async(gr_engine *e, const int64_t *ids, int32_t n, void *out_host, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!ids || n < 1 || n > e->opts.max_requests) return fail(GR_E_INVALID_ARG, "need 1..max_requests ids");
  if (!out_host) return fail(GR_E_INVALID_ARG, "null output");
  const int lv = e->dm.levels;
  std::vector<int32_t> slots((size_t)n);
  for (int i = 0; i < n; ++i) {
    auto it = e->reqs.find(ids[i]);
    if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
    if (it->second.level != lv) return fail(GR_E_BAD_STATE, "request has not decoded every level yet");
    slots[(size_t)i] = it->second.slot;
  }
  hipStream_t st = (hipStream_t)stream;
  uint8_t *dst = e->ws + e->off_out;
  gr_status r;
  for (int i0 = 0; i0 < n; i0 += gr::kGatherMax) {
    const int m = std::min(gr::kGatherMax, n - i0);
    if ((r = check_dev(e, gr::launch_gather_results(e->dev, slots.data() + i0, m, lv & 1, dst + e->out_bytes * i0,
                                                    e->out_bytes, st),
                       "result gather")) != GR_OK)
      return r;
  }
  return check_dev(e, hipMemcpyAsync(out_host, dst, e->out_bytes * (size_t)n, hipMemcpyDeviceToHost, st),
                   "result copy");
}

size_t gr_beams_result_bytes(const gr_engine *e) { return e ? e->out_bytes : 0; }

gr_status gr_beams_unpack(const gr_engine *e, const void *out_host, int32_t i, int32_t cap, int32_t *codes,
                          float *scores, int32_t *n_beams) {
  if (!e || !out_host || !n_beams || i < 0 || cap < 0 || (cap > 0 && (!codes || !scores)))
    return fail(GR_E_INVALID_ARG, "null argument");
  const int lv = e->dm.levels;
  const size_t W = (size_t)e->dm.W_max;
  const uint8_t *src = (const uint8_t *)out_host + e->out_bytes * (size_t)i;
  int32_t nl;
  std::memcpy(&nl, src, 4);
  *n_beams = nl;
  if (nl < 0 || (size_t)nl > W) return fail(GR_E_INVALID_ARG, "not a completed result record");
  if (nl > cap) return fail(GR_E_INVALID_ARG, "capacity smaller than the number of beams");
  if (nl > 0) {
    std::memcpy(codes, src + 16, (size_t)nl * lv * 4);
    std::memcpy(scores, src + 16 + W * lv * 4, (size_t)nl * 4);
  }
  return GR_OK;
}

gr_status gr_beams_get_batch(gr_engine *e, const int64_t *ids, int32_t n, int32_t cap, int32_t *codes,
                             float *scores, int32_t *n_beams, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (!n_beams || cap < 0 || (cap > 0 && (!codes || !scores))) return fail(GR_E_INVALID_ARG, "null output");
  gr_status r;
  if ((r = gr_beams_get_batch_async(e, ids, n, e->out_host, stream)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize((hipStream_t)stream), "sync")) != GR_OK) return r;
  const int lv = e->dm.levels;
  bool over = false;
  for (int i = 0; i < n; ++i) {
    if (gr_beams_unpack(e, e->out_host, i, cap, codes + (size_t)i * cap * lv, scores + (size_t)i * cap,
                        n_beams + i) != GR_OK)
      over = true;
  }
  if (over) return fail(GR_E_INVALID_ARG, "capacity smaller than the number of beams");
  return GR_OK;
}

gr_status gr_beams_get(gr_engine *e, int64_t rid, int32_t cap, int32_t *codes, float *scores, int32_t *n_beams,
                       void *stream) {
  return gr_beams_get_batch(e, &rid, 1, cap, codes, scores, n_beams, stream);
}

gr_status gr_score_items_batch(gr_engine *e, const int64_t *ids, int32_t n_req, const int32_t *items, int32_t n,
                               float *scores, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (!ids || !items || !scores) return fail(GR_E_INVALID_ARG, "null ids, items or scores");
  if (n_req < 1 || n_req > e->opts.max_requests) return fail(GR_E_INVALID_ARG, "need 1..max_requests ids");
  if (n < 1 || n > e->dm.W_max) return fail(GR_E_INVALID_ARG, "n_items must be in [1, max_beam_width]");
  const int lv = e->dm.levels;
  for (int64_t i = 0; i < (int64_t)n_req * n * lv; ++i)
    if (items[i] < 0 || items[i] >= e->dm.V) return fail(GR_E_INVALID_ARG, "item code outside the codebook");
  std::vector<gr_engine::Req *> rs((size_t)n_req);
  std::vector<int32_t> slots((size_t)n_req);
  {
    std::unordered_set<int64_t> seen;
    for (int i = 0; i < n_req; ++i) {
      if (!seen.insert(ids[i]).second) return fail(GR_E_INVALID_ARG, "duplicate request id");
      auto it = e->reqs.find(ids[i]);
      if (it == e->reqs.end()) return fail(GR_E_NOT_FOUND, "unknown request id");
      rs[(size_t)i] = &it->second;
      slots[(size_t)i] = it->second.slot;
    }
  }
  hipStream_t st = (hipStream_t)stream;
  gr_status r;
  const size_t bytes = (size_t)n * lv * sizeof(int32_t);
  for (int i = 0; i < n_req; ++i)
    if ((r = check_dev(e, hipMemcpyAsync(slot_ptr(e, rs[(size_t)i]) + e->sl.items, items + (size_t)i * n * lv, bytes,
                                         hipMemcpyHostToDevice, st), "items upload")) != GR_OK)
      return r;
  for (int i0 = 0; i0 < n_req; i0 += gr::kGatherMax)
    if ((r = check_dev(e, gr::launch_init_slots(e->dev, slots.data() + i0, std::min(gr::kGatherMax, n_req - i0), st),
                       "slot init")) != GR_OK)
      return r;
  for (auto *R : rs) {
    R->level = 0;
    R->n_bound = 1;
    R->n_items = n;
  }
  for (int s = 0; s < lv; ++s)
    if ((r = gr_beam_step(e, ids, n_req, stream)) != GR_OK) return r;
  std::vector<int32_t> codes((size_t)n_req * n * lv), nb((size_t)n_req);
  return gr_beams_get_batch(e, ids, n_req, n, codes.data(), scores, nb.data(), stream);
}

gr_status gr_score_items(gr_engine *e, int64_t rid, const int32_t *items, int32_t n, float *scores, void *stream) {
  return gr_score_items_batch(e, &rid, 1, items, n, scores, stream);
}

gr_status gr_score_items_labels(gr_engine *e, const int64_t *ids, int32_t n_req, const int32_t *items, int32_t n,
                                float *scores, float *label_logp, void *stream) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (e->dm.n_labels < 1) return fail(GR_E_BAD_STATE, "the engine has no label head");
  if (!label_logp) return fail(GR_E_INVALID_ARG, "null label_logp");
  gr_status r = gr_score_items_batch(e, ids, n_req, items, n, scores, stream);  // validates, synchronises
  if (r != GR_OK) return r;
  std::vector<int> order;
  if ((r = step_impl(e, ids, n_req, stream, &order)) != GR_OK) return r;
  const int nl = e->dm.n_labels, W = e->dm.W_max;
  std::vector<float> out((size_t)n_req * W * nl);
  hipStream_t st = (hipStream_t)stream;
  if ((r = check_dev(e, hipMemcpyAsync(out.data(), e->ws + e->off_label, out.size() * 4, hipMemcpyDeviceToHost, st),
                     "label copy")) != GR_OK)
    return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  for (int i = 0; i < n_req; ++i)  // descriptor i holds request order[i]
    std::memcpy(label_logp + (size_t)order[(size_t)i] * n * nl, out.data() + (size_t)i * W * nl,
                (size_t)n * nl * sizeof(float));
  return GR_OK;
}

gr_status gr_debug_beam_state(gr_engine *e, int64_t rid, int32_t cap, int32_t *parent, int32_t *codes,
                              float *scores, int32_t *n, int32_t *level, void *stream) {
  gr_engine::Req *R;
  gr_status r = find_req(e, rid, &R);
  if (r != GR_OK) return r;
  if (!parent || !codes || !scores || !n || !level) return fail(GR_E_INVALID_ARG, "null output");
  hipStream_t st = (hipStream_t)stream;
  uint8_t *sb = slot_ptr(e, R);
  const int cur = R->level & 1, lv = e->dm.levels;
  int32_t nl = 0;
  if ((r = d2h(e, &nl, sb + e->sl.n_live + 4 * cur, 4, st)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  *n = nl;
  *level = R->level;
  const int m = std::min(nl, cap);
  if (m > 0) {
    if ((r = d2h(e, parent, sb + e->sl.parent[cur], (size_t)m * 4, st)) != GR_OK) return r;
    if ((r = d2h(e, codes, sb + e->sl.codes[cur], (size_t)m * lv * 4, st)) != GR_OK) return r;
    if ((r = d2h(e, scores, sb + e->sl.score[cur], (size_t)m * 4, st)) != GR_OK) return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  }
  return GR_OK;
}

gr_status gr_debug_beam_path(gr_engine *e, int64_t rid, int32_t cap, int32_t *anc, int32_t *n, void *stream) {
  gr_engine::Req *R;
  gr_status r = find_req(e, rid, &R);
  if (r != GR_OK) return r;
  if (!anc || !n) return fail(GR_E_INVALID_ARG, "null output");
  hipStream_t st = (hipStream_t)stream;
  uint8_t *sb = slot_ptr(e, R);
  const int cur = R->level & 1;
  int32_t nl = 0;
  if ((r = d2h(e, &nl, sb + e->sl.n_live + 4 * cur, 4, st)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  *n = nl;
  const int m = std::min(nl, cap);
  if (m > 0) {
    if ((r = d2h(e, anc, sb + e->sl.anc[cur], (size_t)m * e->dm.levels * 4, st)) != GR_OK) return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  }
  return GR_OK;
}

gr_status gr_debug_hidden(gr_engine *e, int64_t rid, int32_t cap, float *hidden, float *logits, int32_t *n,
                          void *stream) {
  gr_engine::Req *R;
  gr_status r = find_req(e, rid, &R);
  if (r != GR_OK) return r;
  if (!n) return fail(GR_E_INVALID_ARG, "null output");
  if (R->level < 1) return fail(GR_E_BAD_STATE, "no step completed yet");
  hipStream_t st = (hipStream_t)stream;
  uint8_t *sb = slot_ptr(e, R);
  const int prev = (R->level - 1) & 1;
  int32_t nl = 0;
  if ((r = d2h(e, &nl, sb + e->sl.n_live + 4 * prev, 4, st)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  *n = nl;
  const int m = std::min(nl, cap);
  const size_t H = (size_t)e->dm.Hq * e->dm.d;
  if (m > 0) {
    if (hidden && (r = d2h(e, hidden, sb + e->sl.h, (size_t)m * H * 4, st)) != GR_OK) return r;
    if (logits && (r = d2h(e, logits, sb + e->sl.logits, (size_t)m * e->dm.V * 4, st)) != GR_OK) return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  }
  return GR_OK;
}

gr_status gr_debug_attn_out(gr_engine *e, int64_t rid, int32_t layer, int32_t cap, float *out, int32_t *n,
                            void *stream) {
  gr_engine::Req *R;
  gr_status r = find_req(e, rid, &R);
  if (r != GR_OK) return r;
  if (!e->dm.debug_attn) return fail(GR_E_BAD_STATE, "engine created without GR_ENGINE_DEBUG_ATTN");
  if (!out || !n) return fail(GR_E_INVALID_ARG, "null output");
  if (layer < 0 || layer >= e->dm.L) return fail(GR_E_INVALID_ARG, "layer out of range");
  if (R->level < 1) return fail(GR_E_BAD_STATE, "no step completed yet");
  hipStream_t st = (hipStream_t)stream;
  uint8_t *sb = slot_ptr(e, R);
  const int prev = (R->level - 1) & 1;
  int32_t nl = 0;
  if ((r = d2h(e, &nl, sb + e->sl.n_live + 4 * prev, 4, st)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  *n = nl;
  const int m = std::min(nl, cap);
  const size_t row = (size_t)e->dm.Hq * e->dm.d;
  if (m > 0) {
    if ((r = d2h(e, out, sb + e->sl.dbg_attn + (size_t)layer * e->dm.W_max * row * 4, (size_t)m * row * 4, st)) !=
        GR_OK)
      return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  }
  return GR_OK;
}

gr_status gr_debug_chain_rows(gr_engine *e, int64_t rid, int32_t layer, int32_t which, int32_t cap, float *out,
                              int32_t *n, void *stream) {
  gr_engine::Req *R;
  gr_status r = find_req(e, rid, &R);
  if (r != GR_OK) return r;
  if (!e->dm.chain || !e->dm.debug_attn) return fail(GR_E_BAD_STATE, "needs a layer-chain engine with GR_ENGINE_DEBUG_ATTN");
  if (!out || !n || cap < 0) return fail(GR_E_INVALID_ARG, "null output");
  if (layer < 0 || layer >= e->dm.L) return fail(GR_E_INVALID_ARG, "layer out of range");
  if (which < GR_CHAIN_X_IN || which > GR_CHAIN_X_OUT) return fail(GR_E_INVALID_ARG, "unknown row kind");
  if (R->level < 1) return fail(GR_E_BAD_STATE, "no step completed yet");
  hipStream_t st = (hipStream_t)stream;
  uint8_t *sb = slot_ptr(e, R);
  const int prev = (R->level - 1) & 1;
  int32_t nl = 0;
  if ((r = d2h(e, &nl, sb + e->sl.n_live + 4 * prev, 4, st)) != GR_OK) return r;
  if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
  *n = nl;
  const int m = std::min(nl, cap);
  const size_t D = (size_t)e->dm.Hq * e->dm.d;
  const size_t width = which == GR_CHAIN_ACT ? (size_t)e->chain.intermediate : D;
  const bool f32 = which == GR_CHAIN_X_IN || which == GR_CHAIN_X_MID || which == GR_CHAIN_X_OUT;
  if (m > 0) {
    const uint8_t *src = chain_dbg(e, layer, which) + (size_t)R->last_row0 * width * (f32 ? 4 : 2);
    std::vector<uint8_t> raw((size_t)m * width * (f32 ? 4 : 2));
    if ((r = d2h(e, raw.data(), src, raw.size(), st)) != GR_OK) return r;
    if ((r = check_dev(e, hipStreamSynchronize(st), "sync")) != GR_OK) return r;
    if (f32) {
      std::memcpy(out, raw.data(), raw.size());
    } else {
      for (size_t i = 0; i < (size_t)m * width; ++i) {
        const uint32_t b = (uint32_t)raw[2 * i] | ((uint32_t)raw[2 * i + 1] << 8);
        const uint32_t u = b << 16;
        std::memcpy(out + i, &u, 4);
      }
    }
  }
  return GR_OK;
}

gr_status gr_engine_set_profiling(gr_engine *e, int32_t enable) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  e->prof = enable != 0;
  e->prof_mask = ~0u;
  return GR_OK;
}

gr_status gr_engine_set_profiling_kinds(gr_engine *e, uint32_t kinds) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  e->prof = kinds != 0;
  e->prof_mask = kinds;
  return GR_OK;
}

gr_status gr_wave_times_select(int32_t level, int32_t layer) {
  if (level < -1 || layer < -1) return fail(GR_E_INVALID_ARG, "level and layer must be >= -1");
  const hipError_t err = gr::wave_times_select(level, layer);
  return err == hipSuccess ? GR_OK : fail(GR_E_DEVICE, hipGetErrorString(err));
}

gr_status gr_wave_times_read(int64_t *host, size_t count) {
  const size_t full = (size_t)gr::kWaveTimesWgs * 8 * gr::kWaveTimesFields;
  if (!host || count != full) return fail(GR_E_INVALID_ARG, "host buffer of kWaveTimesWgs x 8 x 8 values");
  const hipError_t err = gr::wave_times_read(reinterpret_cast<long long *>(host), count);
  if (err == hipErrorNotSupported) return fail(GR_E_UNSUPPORTED, "not a wave-timeline build");
  return err == hipSuccess ? GR_OK : fail(GR_E_DEVICE, hipGetErrorString(err));
}

gr_status gr_engine_set_profiling_stride(gr_engine *e, int32_t stride) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  if (stride < 1) return fail(GR_E_INVALID_ARG, "profiling stride must be >= 1");
  e->prof_stride = stride;
  return GR_OK;
}

gr_status gr_engine_profile_read(gr_engine *e, int32_t kind, int32_t level, double *total_ms, int64_t *launches) {
  if (!e || !total_ms || !launches) return fail(GR_E_INVALID_ARG, "null argument");
  if (kind < 0 || kind > GR_PROF_NORM) return fail(GR_E_INVALID_ARG, "unknown profile kind");
  if (level < -1 || level > e->dm.levels) return fail(GR_E_INVALID_ARG, "level out of range");
  gr_status r = prof_fold(e);
  if (r != GR_OK) return r;
  double ms = 0.0;
  int64_t n = 0;
  for (int l = 0; l <= e->dm.levels; ++l)
    if (level < 0 || l == level) {
      ms += e->prof_ms[kind][l];
      n += e->prof_n[kind][l];
    }
  *total_ms = ms;
  *launches = n;
  return GR_OK;
}

gr_status gr_engine_profile_dispatches(gr_engine *e, int32_t kind, int32_t level, int64_t *dispatches) {
  if (!e || !dispatches) return fail(GR_E_INVALID_ARG, "null argument");
  if (kind < 0 || kind > GR_PROF_NORM) return fail(GR_E_INVALID_ARG, "unknown profile kind");
  if (level < -1 || level > e->dm.levels) return fail(GR_E_INVALID_ARG, "level out of range");
  gr_status r = prof_fold(e);
  if (r != GR_OK) return r;
  int64_t n = 0;
  for (int l = 0; l <= e->dm.levels; ++l)
    if (level < 0 || l == level) n += e->prof_d[kind][l];
  *dispatches = n;
  return GR_OK;
}

gr_status gr_engine_graph_stats(const gr_engine *e, int64_t *captures, int64_t *replays) {
  if (!e || !captures || !replays) return fail(GR_E_INVALID_ARG, "null argument");
  *captures = e->graph_captures;
  *replays = e->graph_hits;
  return GR_OK;
}

gr_status gr_engine_profile_reset(gr_engine *e) {
  if (!e) return fail(GR_E_INVALID_ARG, "null engine");
  gr_status r = prof_fold(e);
  if (r != GR_OK) return r;
  std::memset(e->prof_ms, 0, sizeof(e->prof_ms));
  std::memset(e->prof_n, 0, sizeof(e->prof_n));
  std::memset(e->prof_d, 0, sizeof(e->prof_d));
  return GR_OK;
}

gr_status gr_topk_select(const float *cand, int32_t n_rows, int32_t V, int32_t k, int32_t *out_flat,
                         float *out_score, int32_t *n_out, void *stream) {
  g_err.clear();
  if (!cand || !out_flat || !out_score || !n_out) return fail(GR_E_INVALID_ARG, "null argument");
  if (n_rows < 1 || V < 1) return fail(GR_E_INVALID_ARG, "n_rows and V must be >= 1");
  if ((int64_t)n_rows * V > (int64_t)1 << 26) return fail(GR_E_UNSUPPORTED, "n_rows*V must be <= 2**26");
  if (k < 1 || k > gr::kMaxBeam) return fail(GR_E_INVALID_ARG, "k must be in [1, 1024]");
  hipError_t err = gr::launch_topk_select(cand, n_rows, V, k, out_flat, out_score, n_out, (hipStream_t)stream);
  if (err != hipSuccess) return fail(GR_E_DEVICE, std::string("top-k select: ") + hipGetErrorString(err));
  return GR_OK;
}


// ---- continuous batching: host scheduler ---------------------------------------------------
// FIFO admission into free slots, one batched step per call over every decoding request, and a
// one-step lag on results: the call that enqueues step t waits only for the result copy of step
// t-1, which the GPU finished before starting step t.  Result buffers alternate between two
// pinned areas; the device staging area of the engine is reused in stream order.
}  // extern "C"

struct gr_sched {
  gr_engine *e = nullptr;
  hipStream_t st = nullptr;
  int max_active = 1;
  struct Pending {
    int64_t rid;
    int32_t N, W;
    const void *k, *v, *q;
    uint32_t flags;
  };
  std::deque<Pending> queue;
  std::vector<int64_t> active;        // loaded and decoding, in admission order
  std::unordered_set<int64_t> known;  // ids queued, decoding or holding a result
  struct Batch {
    std::vector<int64_t> ids;
    uint8_t *host = nullptr;  // pinned, out_bytes per request
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  Batch batch[2];
  int cur = 0;  // the batch this call fills; the other one belongs to the previous call
  struct Result {
    int32_t n = 0;
    std::vector<int32_t> codes;
    std::vector<float> scores;
  };
  std::unordered_map<int64_t, Result> done;
  std::deque<int64_t> done_order;  // may hold ids already taken (skipped)
  int64_t steps = 0;
};

namespace {

// Results of a finished batch into the store (waits for its copy).
gr_status sched_collect(gr_sched *s, gr_sched::Batch &B, int32_t *n_completed) {
  if (!B.pending) return GR_OK;
  gr_engine *e = s->e;
  gr_status r;
  if ((r = check_dev(e, hipEventSynchronize(B.ev), "result copy")) != GR_OK) return r;
  const int lv = e->dm.levels;
  for (size_t i = 0; i < B.ids.size(); ++i) {
    gr_sched::Result R;
    std::memcpy(&R.n, B.host + e->out_bytes * i, 4);
    R.codes.resize((size_t)R.n * lv);
    R.scores.resize((size_t)R.n);
    if ((r = gr_beams_unpack(e, B.host, (int32_t)i, R.n, R.codes.data(), R.scores.data(), &R.n)) != GR_OK) return r;
    s->done[B.ids[i]] = std::move(R);
    s->done_order.push_back(B.ids[i]);
  }
  if (n_completed) *n_completed += (int32_t)B.ids.size();
  B.ids.clear();
  B.pending = false;
  return GR_OK;
}

}  // namespace

extern "C" {

gr_status gr_sched_create(gr_engine *e, int32_t max_active, void *stream, gr_sched **out) {
  g_err.clear();
  if (!e || !out) return fail(GR_E_INVALID_ARG, "null argument");
  *out = nullptr;
  if (!e->bound) return fail(GR_E_BAD_STATE, "workspace not bound");
  if (max_active < 1 || max_active > e->opts.max_requests)
    return fail(GR_E_INVALID_ARG, "max_active must be in [1, max_requests]");
  auto *s = new gr_sched();
  s->e = e;
  s->st = (hipStream_t)stream;
  s->max_active = max_active;
  gr_status r = GR_OK;
  for (auto &B : s->batch) {
    if (r == GR_OK)
      r = check_dev(e, hipHostMalloc((void **)&B.host, e->out_bytes * (size_t)e->opts.max_requests,
                                     hipHostMallocDefault), "pinned scheduler results");
    if (r == GR_OK) r = check_dev(e, hipEventCreateWithFlags(&B.ev, hipEventDisableTiming), "event");
  }
  if (r != GR_OK) {
    (void)gr_sched_destroy(s);
    return r;
  }
  *out = s;
  return GR_OK;
}

gr_status gr_sched_destroy(gr_sched *s) {
  if (!s) return GR_OK;
  if (s->e && s->e->bound) (void)hipStreamSynchronize(s->st);
  for (int64_t rid : s->active) (void)gr_request_release(s->e, rid);
  for (auto &B : s->batch) {
    if (B.ev) (void)hipEventDestroy(B.ev);
    if (B.host) (void)hipHostFree(B.host);
  }
  delete s;
  return GR_OK;
}

gr_status gr_sched_submit(gr_sched *s, int64_t rid, int32_t N, int32_t W, const void *k, const void *v,
                          const void *q_last, uint32_t flags) {
  g_err.clear();
  if (!s) return fail(GR_E_INVALID_ARG, "null scheduler");
  if (!k || !v || !q_last) return fail(GR_E_INVALID_ARG, "null k, v or q_last");
  if (s->known.count(rid) || s->e->reqs.count(rid))
    return fail(GR_E_INVALID_ARG, "request id queued, decoding or holding a result");
  s->queue.push_back({rid, N, W, k, v, q_last, flags});
  s->known.insert(rid);
  return GR_OK;
}

gr_status gr_sched_advance(gr_sched *s, int32_t *n_completed) {
  g_err.clear();
  if (!s || !n_completed) return fail(GR_E_INVALID_ARG, "null argument");
  *n_completed = 0;
  gr_engine *e = s->e;
  if (e->poisoned) return fail(GR_E_DEVICE, "engine poisoned by an earlier device error");
  gr_status r;
  // 1. admissions, in arrival order, while a slot, pool room and the concurrency cap allow
  while (!s->queue.empty() && (int)s->active.size() < s->max_active && !e->free_slots.empty()) {
    const gr_sched::Pending P = s->queue.front();
    r = gr_ctx_kv_load(e, P.rid, P.N, P.W, P.k, P.v, P.q, P.flags, s->st);
    if (r == GR_E_OUT_OF_MEMORY && !s->active.empty()) break;  // the pool frees as requests finish
    if (r != GR_OK) {  // dropped with the load's error
      s->queue.pop_front();
      s->known.erase(P.rid);
      return r;
    }
    s->queue.pop_front();
    s->active.push_back(P.rid);
  }
  gr_sched::Batch &B = s->batch[s->cur];
  if ((r = sched_collect(s, B, n_completed)) != GR_OK) return r;  // never pending here; kept safe
  // 2. one batched step over every decoding request, each at its own level
  if (!s->active.empty()) {
    if ((r = gr_beam_step(e, s->active.data(), (int32_t)s->active.size(), s->st)) != GR_OK) return r;
    ++s->steps;
    // 3. the requests this step finished: gather, copy to pinned memory, release the slots
    const int lv = e->dm.levels;
    std::vector<int64_t> still;
    for (int64_t rid : s->active) {
      const gr_engine::Req &R = e->reqs.at(rid);
      if (R.level == lv) {
        B.ids.push_back(rid);
      } else {
        still.push_back(rid);
      }
    }
    s->active.swap(still);
    if (!B.ids.empty()) {
      if ((r = gr_beams_get_batch_async(e, B.ids.data(), (int32_t)B.ids.size(), B.host, s->st)) != GR_OK) return r;
      if ((r = check_dev(e, hipEventRecord(B.ev, s->st), "event")) != GR_OK) return r;
      B.pending = true;
      for (int64_t rid : B.ids)
        if ((r = gr_request_release(e, rid)) != GR_OK) return r;
    }
  }
  // 4. the previous call's results: its copy ran before this call's step
  if ((r = sched_collect(s, s->batch[s->cur ^ 1], n_completed)) != GR_OK) return r;
  s->cur ^= 1;
  return GR_OK;
}

gr_status gr_sched_flush(gr_sched *s, int32_t *n_completed) {
  g_err.clear();
  if (!s || !n_completed) return fail(GR_E_INVALID_ARG, "null argument");
  *n_completed = 0;
  gr_status r;
  // the older batch first
  if ((r = sched_collect(s, s->batch[s->cur], n_completed)) != GR_OK) return r;
  return sched_collect(s, s->batch[s->cur ^ 1], n_completed);
}

gr_status gr_sched_completed(gr_sched *s, int32_t cap, int64_t *ids, int32_t *n) {
  g_err.clear();
  if (!s || !n || cap < 0 || (cap > 0 && !ids)) return fail(GR_E_INVALID_ARG, "null argument");
  int32_t k = 0;
  for (int64_t rid : s->done_order) {
    if (k >= cap) break;
    if (s->done.count(rid)) ids[k++] = rid;
  }
  *n = (int32_t)s->done.size();
  return GR_OK;
}

gr_status gr_sched_result(gr_sched *s, int64_t rid, int32_t cap, int32_t *codes, float *scores, int32_t *n_beams) {
  g_err.clear();
  if (!s || !n_beams || cap < 0 || (cap > 0 && (!codes || !scores))) return fail(GR_E_INVALID_ARG, "null output");
  auto it = s->done.find(rid);
  if (it == s->done.end()) return fail(GR_E_NOT_FOUND, "no result for this request id (yet)");
  const gr_sched::Result &R = it->second;
  *n_beams = R.n;
  if (R.n > cap) return fail(GR_E_INVALID_ARG, "capacity smaller than the number of beams");
  if (R.n > 0) {
    std::memcpy(codes, R.codes.data(), R.codes.size() * 4);
    std::memcpy(scores, R.scores.data(), R.scores.size() * 4);
  }
  s->done.erase(it);
  s->known.erase(rid);
  while (!s->done_order.empty() && !s->done.count(s->done_order.front())) s->done_order.pop_front();
  return GR_OK;
}

gr_status gr_sched_counts(const gr_sched *s, int32_t *queued, int32_t *active, int32_t *done, int64_t *steps) {
  g_err.clear();
  if (!s) return fail(GR_E_INVALID_ARG, "null scheduler");
  if (queued) *queued = (int32_t)s->queue.size();
  if (active) *active = (int32_t)s->active.size();
  if (done) *done = (int32_t)s->done.size();
  if (steps) *steps = s->steps;
  return GR_OK;
}

}  // extern "C"
