// Internal structures shared by the host engine (gr_engine.cpp) and the HIP
// kernels (gr_kernels.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gr {

constexpr int kMaxLevels = 8;
constexpr int kMaxGroup = 8;      // query heads per kv head handled by the beam kernel
constexpr int kTileTok = 64;      // context tokens per split granule / padding unit
constexpr int kWaveTimesWgs = 1024;  // workgroups whose waves a GR_WAVE_TIMES build records
constexpr int kWaveTimesFields = 8;  // values per wave
constexpr int kTopkThreads = 1024;
constexpr int kMaxBeam = 1024;
constexpr int kLogitsKS = 4;          // split of the hidden dimension in the logits GEMM
constexpr int kSelectCPT = 64;        // candidates per thread kept in registers by the selection
constexpr int kLsmRows = 16;          // beam rows per log-softmax workgroup (one wave each): a top-K chunk
constexpr int kSel2CPT = 16;          // kept keys per thread in the second top-K stage (chunks x W <= 16384)
constexpr int kTieCap = 1024;         // candidates sharing the cut bin that the fast selection sorts
constexpr int kGatherMax = 64;        // slots per result-gather / root-beam launch

struct Dims {
  int L, Hq, Hkv, g, d, levels, V, MW;  // MW = 32-bit words per trie mask row
  int W_max, S_max;        // S_max: split slots at full beam width (part_rows = Hkv*S_max*W_max*g)
  int dtype;   // 0 f32, 1 bf16
  int norm;    // 0 valid, 1 full
  float scale_log2;  // log2(e) / sqrt(d)
  int debug_attn;
  int chain;         // 1: the layer-chain model (q of a step from the q rows, outputs to the o rows)
  int tl;            // token-table and BeamKV levels: levels - 1, or levels with a label head (the
                     // last level's codes are then tokens too, read by the label step s = levels)
  int n_labels;      // label head outputs (0: none)
};

// Byte offsets of the arrays inside one request slot; slots are slot_bytes apart.
struct SlotLayout {
  size_t slot_bytes;
  size_t beamkv_k, beamkv_v;  // [L][tl][W_max][Hkv][d] elem
  size_t q_last;              // [L][Hq][d] elem
  size_t knmax;               // [L][Hkv] f32: largest context-key norm (bounds the scores)
  size_t vscale;              // [L][Hkv] f32: power of two above the context's largest |v| (taken at load)
  size_t h;                   // [W_max][Hq*d] f32
  size_t logits;              // [W_max][V] f32
  size_t logits_part;         // [kLogitsKS][W_max][V] f32 split-K partial sums
  size_t cand;                // [W_max][V] f32
  size_t lkeys;               // [ceil(W_max / kLsmRows)][W] u64: each chunk's largest candidate keys
  size_t lcnt;                // [ceil(W_max / kLsmRows)] i32: keys kept per chunk
  size_t part_o[2];           // [part_rows][d] f32 unnormalised o, row ((h*splits + sp)*rows_b + row); by layer parity
  size_t part_ml[2];          // [part_rows] float2 (m in log2 units, l)
  size_t codes[2];            // [W_max][levels] i32   (double-buffered by level parity)
  size_t score[2];            // [W_max] f32
  size_t node[2];             // [W_max] i32  trie node of the beam's prefix
  size_t anc[2];              // [W_max][levels] i32  BeamKV slot of each level's token
  size_t parent[2];           // [W_max] i32
  size_t n_live;              // i32[2]: n_live[s & 1] = beams of B_s
  size_t items;               // [W_max][levels] i32: the candidates of a scoring request
  size_t dbg_attn;            // [L][W_max][Hq][d] f32 (only with debug_attn)
  size_t hl;                  // full-context steps: [L][W_max][Hq][d] f32 o/l of each layer (0 when impossible)
};

// The layer chain's weights and per-step activation rows (gr_chain.hip).  Rows: a step's beams
// packed request after request (StepReq::row0), padded to a multiple of 128.
struct ChainDev {
  int D, I;          // hidden (= Hq * d) and MLP width
  float eps;
  const uint16_t *embed;                      // [levels-1][V][D] bf16
  const uint16_t *wq, *wk, *wv, *wo;          // [L][Hq d][D], [L][Hkv d][D] x2, [L][D][Hq d]
  const uint16_t *wg, *wu, *wd;               // [L][I][D] x2, [L][D][I]
  const float *g_attn, *g_mlp, *g_final;      // [L][D], [L][D], [D]
  float *x;                                   // residual rows [rows][D] float32
  uint16_t *xn, *q, *o, *act;                 // bf16 rows: [rows][D], [rows][Hq d] x2, [rows][I]
  float *part;                                // split-K partial sums of a projection over few rows
  size_t part_floats;                         // capacity of part
};
enum { kChainQKV = 0, kChainO = 1, kChainGateUp = 2, kChainDown = 3 };

struct Dev {
  Dims dm;
  SlotLayout sl;
  uint8_t *slots;
  const uint32_t *trie_mask;       // concatenated levels: [nodes_t][MW]
  const int32_t *trie_child;       // concatenated levels: [nodes_t]
  int64_t trie_off[kMaxLevels + 1];  // node offset of level t
  const void *tok_q, *tok_k, *tok_v;  // [L][tl][V][H][d]
  const float *w_sid;
  const float *w_label;  // [Hq*d][n_labels] f32 (label head), or null
  float *label_out;      // [max_requests][W_max][n_labels] f32: a label step's log-probs
  ChainDev ch;
};

// One request of one gr_beam_step call.
struct StepReq {
  const void *ctx_k;    // native K [L][Hkv][Np][d]
  const void *ctx_vt;   // native V^T [L][Hkv][d][Np]
  const void *ctx_vt16; // its float16 copy (launch_load_v16), or null: the wide kernel converts V^T itself
  int64_t ctx_lstride;  // elements per layer = Hkv*Np*d
  int N, Np;
  int slot, level, W;
  int n_bound;          // upper bound of n_s known on the host (device holds the exact n_s)
  int rows_b;           // n_bound * g: row stride of the split-K partials
  int splits, tps;      // split-K: number of token ranges, tokens per range (multiple of 64); range
                        // sp covers [sp*tps, (sp+1)*tps), the last one [(splits-1)*tps, N)
  int lgroups;          // full-context steps: layers per launch (else 0)
  int defer_finish;     // split-K steps: layer l is finished inside layer l+1's launch (else by a merge
                        // launch after each layer)
  int row0;             // the layer chain: first packed row of this request (a multiple of 32)
  int n_items;          // > 0: scoring request, its n_items candidates' codes are forced (no top-K)
  int sel2;             // top-K in two stages: k_lsm keeps each chunk's W largest keys, k_select
                        // selects over them (chunks x W <= kTopkThreads * kSel2CPT)
  int row_blocks;       // context-attention row blocks per kv head
  int wg_ctx, wg_merge, wg_logits, wg_lsm, wg_fin;  // first workgroup of this request in each launch
};

// ---- launchers (gr_kernels.hip) ------------------------------------------
// Optional timing events carried by a dispatch itself (hipExtLaunchKernel): `start` is
// stamped when the first launch of a launcher begins, `stop` when its last one ends.  They
// add no marker packets between kernels; both null means a plain launch.
struct LaunchEv {
  hipEvent_t start = nullptr, stop = nullptr;
};
// Context-attention variants: waves per workgroup (1, 2, 4 or 8; 32 query rows per wave)
// in the low byte.  kCtxHiLo marks P split into two bf16 terms (p = p_hi + p_lo, relative
// error about 2^-17), which the one-, two- and four-wave variants use; the eight-wave (wide)
// kernel takes P as one float16 term against float16 V (relative error 2^-11).  A single bf16
// P perturbs each weight by up to 2^-8, and with a few dominant tokens (large query/key norms)
// that moved log-probs past 1e-3.
constexpr int kCtxHiLo = 0x100;
hipError_t launch_ctx_attn(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                           int ctx_kind, hipStream_t st, LaunchEv ev = {});
// Finish of `layer` for reqs[0..n_reqs): one workgroup per beam (total_wgs of them); wg0 =
// reqs[0].wg_merge when reqs starts past the step's first request.
hipError_t launch_beam_merge(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                             hipStream_t st, LaunchEv ev = {}, int wg0 = 0);
// The same finish for bf16 models with the phased loads of the deferred finish: workgroup
// (request, row block of fin_rows_per_wg(d) rows, kv head); wg0 = reqs[0].wg_fin when reqs starts
// past the step's first request.
hipError_t launch_finish_layer(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                              hipStream_t st, LaunchEv ev = {}, int wg0 = 0);
inline int fin_rows_per_wg(int d) { return 256 / (d / 8); }
// A first-level step of head_dim-128 bf16 requests with every layer in one launch (grid
// [total_wgs][L], partials of layer l at row offset l*Hkv*splits*rows_b of buffer 0), and its
// finish: per-layer outputs into buffer 1, then h = sum over layers in order.
hipError_t launch_ctx_attn_first_level(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs,
                                       hipStream_t st, LaunchEv ev = {});
// A wide step (8-wave variant, head_dim 128, bf16) without split partials: one launch covers
// layers layer0 .. layer0 + lgroups - 1, workgroup (row block, kv head, g) owns layer layer0 + g
// over the whole context and finishes it; its o/l goes to the layer's fp16 hidden partial (hl,
// hl_scale), which launch_sum_hparts adds into h in layer order.
hipError_t launch_ctx_attn_layered(const Dev &dev, const StepReq *reqs, int n_reqs, int layer0, int total_wgs,
                                   int ctx_kind, hipStream_t st, LaunchEv ev = {});
hipError_t launch_sum_hparts(const Dev &dev, const StepReq *reqs, int n_reqs, hipStream_t st, LaunchEv ev = {});
// The context-attention wave timeline of a GR_WAVE_TIMES build (gr_kernels.hip): select the
// (level, layer) whose launch is recorded; read kWaveTimesWgs x 8 waves x kWaveTimesFields
// values (hipErrorNotSupported in the product library).
hipError_t wave_times_select(int level, int layer);
hipError_t wave_times_read(long long *host, size_t count);
hipError_t launch_finish_first_level(const Dev &dev, const StepReq *reqs, int n_reqs, hipStream_t st,
                                     LaunchEv ev = {});
hipError_t launch_logits(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st,
                         LaunchEv ev = {});
hipError_t launch_lsm(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st,
                      LaunchEv ev = {});
// max_cand: largest n_bound*V of the step (selects the register-resident or the streaming variant)
hipError_t launch_topk(const Dev &dev, const StepReq *reqs, int n_reqs, int max_cand, hipStream_t st,
                       LaunchEv ev = {});
// root beam (level 0, empty prefix, score 0) in up to kGatherMax slots
hipError_t launch_init_slots(const Dev &dev, const int32_t *slots, int n, hipStream_t st);
// Copies n_live, codes and scores of level parity `parity` of up to kGatherMax slots into a
// staging area: request i at out + i*out_bytes (n_live at 0, codes at 16, scores after
// W_max*levels codes).
hipError_t launch_gather_results(const Dev &dev, const int32_t *slots, int n, int parity, uint8_t *out,
                                 size_t out_bytes, hipStream_t st);
// Context loading.  copy: caller K, V [L][N][Hkv][d] -> native K nk [L][Hkv][Np][d] and V^T nvt
// [L][Hkv][d][Np] (padding zero); else nk / nvt already hold the native layout and are only
// read.  Both: per (layer, kv head) the largest key norm -> knmax [L][Hkv] and the value
// scale, the power of two 2^e with max |v| < 2^e over the first N tokens -> vscale [L][Hkv].
hipError_t launch_load_ctx(const void *src_k, const void *src_v, void *nk, void *nvt, bool copy, int L, int Hkv,
                           int N, int Np, int d, int elem_bytes, float *knmax, float *vscale, hipStream_t st);
// The float16 copy of a bf16 context's V^T that the eight-wave attention kernel reads: nvt16
// [L][Hkv][d][Np] = float16 of v in the units that kernel computes in (v / vscale, or v itself
// when the head's vscale lies in [2^-10, 2^15]), the same rounding as its in-LDS conversion.
// It must follow the launch that wrote vscale, on the same stream.
hipError_t launch_load_v16(const void *nvt, void *nvt16, const float *vscale, int L, int Hkv, int d, int Np,
                           hipStream_t st);
// Prefill (gr_prefill.hip).  Soft token: e = u * proj [du][de] as kSoftSplit partial sums
// over the user vector in e_buf [kSoftSplit][de], then the
// per-layer projections of e in kSoftSplit partial sums over the embedding dimension,
// part [kSoftSplit][L][cq + 2 ckv] (q columns, then k, then v; cq = Hq d, ckv = Hkv d),
// summed in order by their readers.
constexpr int kSoftSplit = 8;
hipError_t launch_soft_token(const float *u, const float *proj, int du, int de, const float *wq, const float *wk,
                             const float *wv, int L, int cq, int ckv, float *e_buf, float *part, hipStream_t st);
// Context K, V of tokens tok device [N] (table rows of tk / tv [L][vocab][Hkv][d]; position
// soft_pos from part) written in the native layout nk [L][Hkv][Np][d], nvt [L][Hkv][d][Np],
// padding zero, with knmax / vscale [L][Hkv] as launch_load_ctx computes them; it must follow
// launch_prefill_q on the same stream (which clears the maxima).  Token ids must be in
// [0, vocab) (checked by the caller).
hipError_t launch_prefill_ctx(int elem_bytes, const void *tk, const void *tv, const int32_t *tok, int N, int Np,
                              int soft_pos, const float *part, int L, int Hq, int Hkv, int d, int vocab, void *nk,
                              void *nvt, float *knmax, float *vscale, hipStream_t st);
// Query of the last position, [L][Hq][d]: row last_tok of tq [L][vocab][Hq][d] (or of the id
// at last_dev, device memory, clamped into [0, vocab)), or the soft token's q (last_tok < 0 and
// no last_dev), into q_slot and (if set) q_out; clears knmax / vscale [L][Hkv] for the
// launch_prefill_ctx that follows.  Context token ids of launch_prefill_ctx outside [0, vocab)
// are clamped the same way.
hipError_t launch_prefill_q(int elem_bytes, const void *tq, int last_tok, const int32_t *last_dev, const float *part,
                            int L, int Hq, int Hkv, int d, int vocab, void *q_slot, void *q_out, float *knmax,
                            float *vscale, hipStream_t st);
// The allocation-free prefill's fixed device array (soft-token partial sums), the same
// kSoftSplit * (embed_dim + L * (Hq + 2 Hkv) d) floats as gr_engine_set_prefill's staging: at
// most kPrefillScratchFloats.  prefill_scratch returns the current device's address of it
// (hipGetSymbolAddress, once per device).
constexpr size_t kPrefillScratchFloats = (size_t)1 << 20;  // 4 MiB
hipError_t prefill_scratch(float **out);
hipError_t launch_topk_select(const float *cand, int n_rows, int V, int k, int32_t *out_flat,
                              float *out_score, int32_t *n_out_dev, hipStream_t st);

// The layer chain (gr_chain.hip), over `rows` packed rows (a multiple of 128): the new tokens'
// input vectors and their first norm; a norm of the residual rows with gain g; a projection
// (kChainQKV, kChainO, kChainGateUp, kChainDown) of layer `layer` with its epilogue; the final
// norm into each request's hidden rows.
hipError_t launch_chain_start(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, hipStream_t st,
                              LaunchEv ev = {});
// The label head after a label step (s = levels): per live beam row of each request, the
// log-softmax over n_labels of h . w_label, to label_out[i][j][c] (i = the request's index in
// reqs).  One workgroup per (request, beam); total_wgs = the sum of the requests' n_bound.
hipError_t launch_label_head(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st,
                             LaunchEv ev = {});
hipError_t launch_chain_norm(const Dev &dev, const float *g, int rows, hipStream_t st, LaunchEv ev = {});
// few: 0 any step; 2 every request at the first level with one live row (n_bound 1): the
// few-row kernel, and the q/k/v projection computes q only (1, one live row per request at any
// level, is accepted by the kernel but not produced by the engine)
hipError_t launch_chain_gemm(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, int kind, int layer,
                             int few, hipStream_t st, LaunchEv ev = {});
hipError_t launch_chain_final(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, hipStream_t st,
                              LaunchEv ev = {});

// rows per context workgroup for a given variant
inline int ctx_rows_per_wg(int kind) { return (kind & 0xFF) * 32; }

// Variant for one request of a step (bf16 path).
inline int ctx_kind_for(int rows, int N, int d) {
  if (rows <= 32) return 1 | kCtxHiLo;
  if (rows <= 64 || d == 64) return (rows <= 64 ? 2 : 4) | kCtxHiLo;
  if (rows <= 128) return 4 | kCtxHiLo;
  (void)N;
  return 8;
}

}  // namespace gr
