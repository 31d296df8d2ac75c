// HIP kernels of the semantic-ID beam-decode step, written for gfx950 (MI355X).
//
// Sources of the method: the zhiding.cn article on NVIDIA recsys-examples,
// section "语义ID生成式推荐专用推理框架" (ContextKV shared by all beams of a
// request, short BeamKV per beam, BeamPath ancestry, item-constrained top-K,
// a decode-attention backend working directly on that KV layout), and the
// paper-daily summary "Advancing Generative Recommendation Inference",
// section "Background" (beam search over semantic-ID prefixes, all beams
// returned).  Split-K over the context with an online-softmax merge is the
// published online-normaliser / flash-decoding method (Milakov & Gimelshein
// 2018); it is not on the pages.
//
// Kernels of a decode step:
//   shared-context attention on MFMA (bf16 K/V), in one of three shapes:
//     k_ctx_attn_stream<3, true>  first level (one beam): every layer in one launch,
//                                 split partials, then k_finish_first_level and
//                                 k_sum_layers form h
//     k_ctx_attn_wide<.., true>   wide steps that fill the chip: a workgroup owns one
//                                 layer's row block over the whole context, merges the
//                                 beam's own tokens (BeamKV through BeamPath) and stores
//                                 o/l as the layer's fp16 hidden partial; k_sum_hparts
//                                 adds the layers into h
//     split-K per layer           k_ctx_attn_wide<.., false>, k_ctx_attn_bf16_narrow,
//                                 k_ctx_attn_stream<4, false>: (m, l, o) partials per
//                                 token range; the next layer's launch finishes the layer
//                                 (BeamKV append, beam tokens, merge, h += o) and
//                                 k_beam_merge the last one
//   k_ctx_attn_f32    split-K context attention on the vector ALU for float32 models
//   k_logits          h @ w_sid[level], fp32 MFMA, split over the hidden dim (float32 models);
//                     k_logits_x3 the same on bf16 MFMA with three-term bf16 operands
//   k_lsm             sums the split logits, trie-masked log-softmax, candidates
//   k_select          top-K over beams x codes, BeamPath update
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gr_internal.h"

namespace gr {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
#define GR_GLOBAL __attribute__((address_space(1)))

constexpr float kNegInf = -__builtin_inff();

// Loads and stores through the global address space (global_load/store, counted by
// vmcnt only, so waiting for LDS never waits for a prefetch in flight).  T is a scalar or
// a clang vector type.
template <typename T>
__device__ __forceinline__ T gld(const void *p) {
  return *(const GR_GLOBAL T *)(p);
}
template <typename T>
__device__ __forceinline__ void gst(void *p, const T &v) {
  *(GR_GLOBAL T *)(p) = v;
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet); two of them in one word
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }
// two floats as float16 (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)a, (_Float16)b});
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over each aligned group of 16 lanes without LDS permutes (DPP: swap neighbours, swap
// pairs, mirror within 8, mirror within 16); every lane of the group gets the sum.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                                   false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);      // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);      // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);     // row_half_mirror
  return dpp_add<0x140>(v);  // row_mirror
}

// Workgroup -> request: reqs[] is ordered by each first-workgroup field.  Up to 8 requests, the
// fields of requests 1..7 are loaded at once (one round trip instead of a binary search's three);
// more, a binary search.
template <int FIELD>
__device__ __forceinline__ int req_first(const StepReq &r) {
  return FIELD == 0 ? r.wg_ctx : FIELD == 1 ? r.wg_merge : FIELD == 2 ? r.wg_logits : FIELD == 3 ? r.wg_lsm : r.wg_fin;
}
template <int FIELD>
__device__ __forceinline__ int find_req(const StepReq *reqs, int n, int bid) {
  if (n <= 8) {
    int f[7];
#pragma unroll
    for (int i = 1; i < 8; ++i) f[i - 1] = req_first<FIELD>(reqs[min(i, n - 1)]);
    int cnt = 0;
#pragma unroll
    for (int i = 1; i < 8; ++i) cnt += (i < n && f[i - 1] <= bid) ? 1 : 0;
    return cnt;
  }
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (req_first<FIELD>(reqs[mid]) <= bid) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint8_t *slot_base(const Dev &dev, int slot) {
  return dev.slots + (size_t)slot * dev.sl.slot_bytes;
}

// Row r of a K tile is stored at LDS row swap23(r) (bits 2 and 3 exchanged).  Lane l of
// the QK^T MFMA then reads LDS row l%32 and holds token swap23(l%32), which makes the
// score accumulator's register layout equal to the PV MFMA's B-operand layout with 8
// consecutive tokens per lane: no cross-lane shuffle between the two MFMAs.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Split partials: (m, l) and the row's unnormalised o, all float32 (a reader weights split sp by
// exp2(m_sp - M)).  Float32 keeps the merge exact to fp32 rounding whatever the attention's
// sharpness: with a few dominant tokens o/l is close to one value row, the hidden vector and
// the logits grow with it, and a 16-bit partial's rounding reached the 1e-3 log-prob bound.
// Lane (row, hh) of an MFMA output tile holds features db*32 + 8a + 4hh .. +4.
template <int DB>
__device__ __forceinline__ void store_partial(uint8_t *slot, const SlotLayout &sl, int buf, size_t prow, float M,
                                              float ltot, int hh, const f32x16_t (&oacc)[DB]) {
  constexpr int D = DB * 32;
  if (hh == 0) gst<f32x2_t>((float2 *)(slot + sl.part_ml[buf]) + prow, f32x2_t{M, ltot});
  float *po = (float *)(slot + sl.part_o[buf]) + prow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      gst<f32x4_t>(po + db * 32 + 8 * a + 4 * hh,
                   f32x4_t{oacc[db][4 * a], oacc[db][4 * a + 1], oacc[db][4 * a + 2], oacc[db][4 * a + 3]});
  }
}

template <int D, typename T>
__device__ __forceinline__ void merge_elem(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int j,
                                           int gi, int kv, int c8);
template <int D, int E>
__device__ __forceinline__ void finish_rows(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int kv,
                                            int r0, int r1, int tid, int nthreads);

// Rows [r0, r1) of a row block's nr rows that split sp finishes.  The rows go to as few splits
// as one batch per workgroup allows (batch = rows one workgroup finishes at once), taken from
// the last split down: the last token range is the shortest, so a small finish (one beam at the
// first level) lands where it lengthens the launch least.
__device__ __forceinline__ void finish_share(int row0, int nr, int splits, int sp, int batch_rows, int &r0, int &r1) {
  const int k = min(splits, max(1, (nr + batch_rows - 1) / batch_rows));
  const int idx = splits - 1 - sp;
  const int per = (nr + k - 1) / k;
  r0 = row0 + min(nr, idx < k ? idx * per : nr);
  r1 = row0 + min(nr, idx < k ? (idx + 1) * per : nr);
}

// --------------------------------------------------------------------------------------
// Shared-context attention, bf16 K/V, fp32 accumulate, MFMA 32x32x16.
//
// Workgroup = NW waves; wave w owns 32 query rows (beam j = row / g, head hq = h*g + row%g)
// of one kv head h of one request; all waves share the K/V tiles of one token range,
// double-buffered through LDS.  Per 32-token sub-tile and wave:
//   S^T[32 tok][32 q] = K_tile * Q^T     (D/16 MFMAs, A = K from LDS, B = Q in registers)
//   online softmax in the log2 domain with a lazy reference max (rescale only when a
//   column's max grows by more than 8, so p <= 256; exact since m and l share it)
//   O^T[D][32 q] += V^T_tile * P^T        (D/32 * 2 MFMAs, A = V^T from LDS, B = P as bf16)
// Output: unnormalised o, the reference max m (log2 units) and l per row and token range.
//
// Workgroup order: the row blocks of one (kv head, token range) pair get workgroup ids
// 8 apart, so (with workgroups dealt round-robin over the 8 XCDs) they run on one XCD
// and share its L2 for the K/V tiles.
template <int D, int NW, int TT, bool HILO>
__device__ __forceinline__ void ctx_attn_body(const Dev &dev, const StepReq *__restrict__ reqs, int n_reqs,
                                              int layer) {
  constexpr int KB = D / 16;
  constexpr int DB = D / 32;
  constexpr int NSUB = TT / 32;
  constexpr int NT = NW * 64;
  constexpr int KCH = TT * (D / 8);
  constexpr int VCH = D * (TT / 8);
  constexpr int KPT = KCH / NT;
  constexpr int VPT = VCH / NT;
  static_assert(KCH % NT == 0 && VCH % NT == 0, "tile/threads mismatch");
  __shared__ bf16x8_t sK[2][TT][D / 8 + 1];
  __shared__ bf16x8_t sV[2][D][TT / 8 + 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5;
  const int ri = find_req<0>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int local = blockIdx.x - R.wg_ctx;
  const int rest = local >> 3;
  const int rb = rest % R.row_blocks;
  const int pidx = (rest / R.row_blocks) * 8 + (local & 7);
  if (pidx >= dm.Hkv * R.splits) return;  // padding workgroup
  const int h = pidx / R.splits, sp = pidx % R.splits;

  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int rows = n_live * dm.g;
  const int row0 = rb * (NW * 32);
  if (row0 >= rows) return;  // whole workgroup idle

  const int wrow = row0 + w * 32;
  const bool wave_active = wrow < rows;
  const int q_row = wrow + (lane & 31);
  const bool row_ok = q_row < rows;

  // ---- query fragments (B operand of QK^T): lane holds Q[q_row][kb*16 + 8*hh .. +8]
  bf16x8_t qf[KB];
  {
    const uint16_t *qsrc = nullptr;
    if (row_ok) {
      const int j = q_row / dm.g, hq = h * dm.g + q_row % dm.g;
      if (dm.chain) {
        qsrc = dev.ch.q + ((size_t)(R.row0 + j) * dm.Hq + hq) * D;
      } else if (s == 0) {
        qsrc = (const uint16_t *)(slot + dev.sl.q_last) + ((size_t)layer * dm.Hq + hq) * D;
      } else {
        const int *codes = (const int *)(slot + dev.sl.codes[s & 1]);
        const int code = codes[j * dm.levels + (s - 1)];
        qsrc = (const uint16_t *)dev.tok_q +
               ((((size_t)layer * dm.tl + (s - 1)) * dm.V + code) * dm.Hq + hq) * D;
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qf[kb] = __builtin_bit_cast(bf16x8_t, row_ok ? gld<u32x4_t>(qsrc + kb * 16 + 8 * hh) : u32x4_t{0, 0, 0, 0});
  }

  const int t0 = sp * R.tps;
  const int t1 = (sp == R.splits - 1 ? R.N : t0 + R.tps);
  const int ntiles = (t1 - t0 + TT - 1) / TT;
  const uint16_t *gK = (const uint16_t *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const uint16_t *gV = (const uint16_t *)R.ctx_vt + (size_t)layer * R.ctx_lstride + (size_t)h * D * R.Np;

  u32x4_t rk[KPT], rv[VPT];
  auto gload = [&](int tb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT, r = c / (D / 8), cc = c % (D / 8);
      rk[i] = gld<u32x4_t>(gK + (size_t)(tb + r) * D + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT, dd = c / (TT / 8), tc = c % (TT / 8);
      rv[i] = gld<u32x4_t>(gV + (size_t)dd * R.Np + tb + tc * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT, r = c / (D / 8), cc = c % (D / 8);
      sK[buf][swap23(r)][cc] = __builtin_bit_cast(bf16x8_t, rk[i]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT, dd = c / (TT / 8), tc = c % (TT / 8);
      sV[buf][dd][tc] = __builtin_bit_cast(bf16x8_t, rv[i]);
    }
  };

  const float c2 = dm.scale_log2;
  float M = kNegInf, l = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};

  // Score bound (Cauchy-Schwarz): u = q.k*log2(e)/sqrt(d) <= B = |q| max|k| log2(e)/sqrt(d).
  // When every row of the workgroup has B <= 60, the fixed reference M = B - 60 keeps every
  // p = 2^(u - M) <= 2^60 and the row's largest p >= 2^(-2B+60) >= 2^-60: no running max and
  // no rescale are needed (m and l share M, so the result is exact).  Otherwise the loop
  // tracks a running max with a lazy rescale.
  __shared__ float sBound[NW];
  {
    float qn = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) qn = fmaf((float)qf[kb][e], (float)qf[kb][e], qn);
    qn += __shfl_xor(qn, 32);
    const float kn = ((const float *)(slot + dev.sl.knmax))[layer * dm.Hkv + h];
    const float B = row_ok ? sqrtf(qn) * kn * c2 * 1.001f + 1e-3f : 0.f;
    M = B - 60.f;
    const float bw = wave_max(B);
    if (lane == 0) sBound[w] = bw;
  }
  __syncthreads();
  float bmax = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) bmax = fmaxf(bmax, sBound[i]);
  const bool fixed_ref = bmax <= 60.f;  // uniform over the workgroup
  if (!fixed_ref) M = kNegInf;

  // one 32-token sub-tile; MASK handles the tokens >= t1 of the last tile
  auto subtile = [&](int buf, int sub, int tb, auto mask_tag, auto fixed_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool FIXED = decltype(fixed_tag)::value;
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8_t kf = sK[buf][sub * 32 + (lane & 31)][kb * 2 + hh];
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], sacc, 0, 0, 0);
    }
    // accumulator register i of lane (col q, half hh) holds token tb + sub*32 + 16*(i/8) + 8*hh + (i%8)
    if constexpr (MASK) {
      const int tbase = tb + sub * 32 + 8 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tbase + 16 * (i >> 3) + (i & 7) >= t1) sacc[i] = kNegInf;
    }
    if constexpr (!FIXED) {
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * c2;
      if (__ballot(mxs > M + 8.f) != 0ull) {
        const float Mn = fmaxf(M, mxs);
        const float f = fast_exp2(M - Mn);
        l *= f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= f;
        M = Mn;
      }
    }
    bf16x8_t pf[2], pl[2];
    if constexpr (HILO) {
      // p = p_hi + p_lo, both bf16 (relative error ~2^-17); l sums p in fp32
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[i], c2, -M));
        const __bf16 ph = (__bf16)p;
        pf[i >> 3][i & 7] = ph;
        pl[i >> 3][i & 7] = (__bf16)(p - (float)ph);
        l += p;
      }
    } else {
      // p rounded to bf16 feeds the PV MFMA; l sums exactly those rounded values (dot2
      // with (1, 1)), so the output is an exact convex combination of the value rows.
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = (__bf16)fast_exp2(fmaf(sacc[i], c2, -M));
      const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[pp], pf[pp], 0, 1), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[pp], pf[pp], 2, 3), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[pp], pf[pp], 4, 5), ones, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[pp], pf[pp], 6, 7), ones, l, false);
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const bf16x8_t vf = sV[buf][db * 32 + (lane & 31)][sub * 4 + pp * 2 + hh];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pp], oacc[db], 0, 0, 0);
        if constexpr (HILO) oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[pp], oacc[db], 0, 0, 0);
      }
    }
  };

  auto run = [&](auto fixed_tag) {
    gload(t0);
    if (layer > 0 && R.defer_finish) {
      // finish the previous layer for this workgroup's share of the row block (its split
      // partials are complete: that layer's kernel has ended)
      int r0, r1;
      finish_share(row0, min(rows, row0 + NW * 32) - row0, R.splits, sp, NT / (D / 8), r0, r1);
      finish_rows<D, 1>(dev, R, slot, layer - 1, h, r0, r1, tid, NT);
    }
    lstore(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      const int tb = t0 + it * TT;
      if (it + 1 < ntiles) gload(tb + TT);
      if (wave_active) {
        if (tb + TT <= t1) {
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub) subtile(buf, sub, tb, std::false_type{}, fixed_tag);
        } else {
#pragma unroll
          for (int sub = 0; sub < NSUB; ++sub)
            if (tb + sub * 32 < t1) subtile(buf, sub, tb, std::true_type{}, fixed_tag);
        }
      }
      if (it + 1 < ntiles) lstore(buf ^ 1);
      __syncthreads();
    }
  };
  if (fixed_ref)
    run(std::true_type{});
  else
    run(std::false_type{});

  const float ltot = l + __shfl_xor(l, 32);
  if (wave_active && row_ok) {
    const size_t prow = ((size_t)h * R.splits + sp) * R.rows_b + q_row;
    store_partial<DB>(slot, dev.sl, layer & 1, prow, M, ltot, hh, oacc);
  }

}

// Wide steps (many query rows, MFMA-bound): two waves per SIMD so one wave's softmax
// overlaps the other's MFMAs; P is rounded once to bf16.  Narrow steps (HBM- or
// latency-bound) keep their staging registers and spend the idle MFMA time on a second
// bf16 term of P.
template <int D, int NW, int TT, bool HILO>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_ctx_attn_bf16(
    Dev dev, const StepReq *__restrict__ reqs, int n_reqs, int layer) {
  ctx_attn_body<D, NW, TT, HILO>(dev, reqs, n_reqs, layer);
}
template <int D, int NW, int TT>
__global__ __launch_bounds__(NW * 64) void k_ctx_attn_bf16_narrow(Dev dev, const StepReq *__restrict__ reqs,
                                                                  int n_reqs, int layer) {
  ctx_attn_body<D, NW, TT, true>(dev, reqs, n_reqs, layer);
}

// --------------------------------------------------------------------------------------
// Shared-context attention for wide steps, head_dim 128: 8 waves (two per SIMD), 32 query
// rows each, 256 rows per workgroup; the arithmetic is that of ctx_attn_body, the schedule
// is built for a long MFMA-bound token loop:
//   * K and V^T tiles go from global memory straight into LDS (global_load_lds_dwordx4,
//     1 KB of consecutive LDS per wave instruction): no staging registers, no LDS stores.
//     A ring of NST stages of 64 tokens keeps NST-2 tiles in flight.
//   * LDS rows are XOR-swizzled instead of padded: 16-byte column c of K row r sits at
//     c ^ (r & 15), of V^T row r (half as long) at c ^ (r & 7) ^ ((r >> 3) & 1), so the
//     operand reads of 16 consecutive lanes (16 consecutive rows) cover all 64 banks once.
//   * QK^T of the next 32-token sub-tile is interleaved by hand with the softmax and PV of
//     the current one, so the exponentials issue while the matrix core works.
// One barrier per tile, placed before the first QK^T of tile it: tile it has landed in LDS
// and every wave is past its last read of tile it-2, whose stage then receives tile
// it+NST-2.  The barrier is a bare s_barrier behind an explicit vmcnt wait (a full
// workgroup fence would wait for the tiles still in flight).
// The copy is issued from inline assembly: the compiler then neither orders later LDS reads
// behind it nor counts it; the explicit vmcnt waits below do both.  lds_addr is the byte
// address in LDS and must be uniform over the wave (it goes through M0; one wait state
// between the M0 write and the LDS-DMA instruction).
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr) : "memory", "m0");
}
// Wave timeline of the context-attention launch (a build option: GR_WAVE_TIMES, the library
// libgr_beam_timed.so; the product library compiles none of it).  For the launch of the selected
// (level, layer) of each request batch, every wave of the first kWaveTimesWgs workgroups
// writes kWaveTimesFields values: its entry, token-loop start, token-loop end and
// partial-stores-done stamps (s_memrealtime, 100 MHz), and over the token loop the shader-clock
// cycles (s_memtime) spent in the copy waits, in the barriers and in the whole loop, and the
// number of barriers.  The last matching launch's values stay.
#ifdef GR_WAVE_TIMES
constexpr bool kWaveTimes = true;
#else
constexpr bool kWaveTimes = false;
#endif
__device__ long long g_wave_times[kWaveTimes ? kWaveTimesWgs * 8 * kWaveTimesFields : 1];
__device__ int g_wave_times_sel[2] = {-1, -1};

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0 || N == 4 || N == 8, "unsupported wait");
}

// as vm_wait_barrier, and this wave's LDS writes done before the barrier
template <int N>
__device__ __forceinline__ void vm_lgkm_wait_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0 || N == 4, "unsupported wait");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (N == 32) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  else if constexpr (N == 48) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  else static_assert(N % 16 == 0 && N <= 48, "unsupported wait");
}

// --------------------------------------------------------------------------------------
// Shared-context attention for narrow steps (at most 32 query rows per wave, head_dim 128),
// which stream the context once and are bound by HBM.  32-token tiles go from global memory
// straight into a ring of NST LDS stages (NST-1 tiles in flight); P is split into two bf16
// terms.  NW = 1: one wave per workgroup, no barrier (the wave's own vmcnt says when a tile has
// landed).  NW = 2: two waves (rows 0-31, 32-63 of the block) share the ring, each issues half
// of every tile's copies, and one barrier per tile (behind the wave's own vmcnt wait) says that
// the tile has landed and that every wave is done with the stage the next copy overwrites.
// V^T rows are 64 bytes here: 16-byte column c of row r sits at
// c ^ (((r >> 1) ^ (r >> 3)) & 3), which keeps 16 consecutive operand rows on 64 banks.
// FUSED (NW = 1): every layer of a first-level step in one launch (blockIdx.y = layer).  At the
// first level each layer's query is an input (q_last), so no layer waits for another; layer l's
// partials go to partial buffer 0 at row offset l*Hkv*splits*rows_b, and the finish of all
// layers runs afterwards (k_finish_first_level).
template <int N>
__device__ __forceinline__ void vm_wait_barrier8() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
  else static_assert(N % 8 == 0 && N <= 24, "unsupported wait");
}

// The beam's own tokens in the full-context kernels.  A row of beam j at level s attends to
// s tokens of its own besides the context: level t < s-1 from BeamKV slot anc[j][t], level s-1
// (its query token) from the token tables at the code chosen at level s-1.
// Index loads first (issued before the live-beam count is known; j is clamped so that rows
// past the live beams load in bounds, and their values are never used): the code and the
// first ancestor slot (older ones are loaded when their token is).  Unsigned, so that
// widening them to 64 bits waits for nothing.
struct BeamIdx {
  uint32_t code, anc0;
};
template <bool ANC>
__device__ __forceinline__ BeamIdx load_beam_idx(const Dev &dev, const uint8_t *slot, int s, int j) {
  BeamIdx b{0u, 0u};
  const int lvl = dev.dm.levels, jj = min(j, dev.dm.W_max - 1);
  if (s > 0) b.code = ((const uint32_t *)(slot + dev.sl.codes[s & 1]))[jj * lvl + (s - 1)];
  if constexpr (ANC) {
    if (s > 1) b.anc0 = ((const uint32_t *)(slot + dev.sl.anc[s & 1]))[jj * lvl];
  }
  return b;
}
// Keys and values of two own tokens (t0, t0+1) of the lane's row, loaded before any arithmetic
// so that a pair costs one memory round trip.  A lane without the token (row past the live
// beams, or t >= s) reads the token table's first row instead: no branch around the loads,
// and its values are never used.
template <int D, int NTOK = 1>
struct TailPair {
  u32x4_t kr[NTOK][D / 16];
  u32x2_t vr[NTOK][D / 8];
};
template <int D, int NTOK>
__device__ __forceinline__ void tail_load_pair(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                               int j, const BeamIdx &bi, int hh, int t0, TailPair<D, NTOK> &tp);
template <int D, int NTOK>
__device__ __forceinline__ void tail_merge_pair(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                                int j, int gi, int hh, float c2, int t0, const TailPair<D, NTOK> &tp,
                                                const bf16x8_t (&qf)[D / 16], float &M, float &l,
                                                f32x16_t (&oacc)[D / 32], bool append, bool fresh = false);
template <int D>
__device__ __forceinline__ void wide_tail_merge(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                                int j, int gi, const BeamIdx &bi, int hh, float c2, bool fresh,
                                                const bf16x8_t (&qf)[D / 16], float &M, float &l,
                                                f32x16_t (&oacc)[D / 32], bool append);
template <int D>
__device__ __forceinline__ void wide_store_layer(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int j,
                                                 int hq, int hh, float ltot, const f32x16_t (&oacc)[D / 32],
                                                 bool row_ok);

// LAYERED (NW = 2): as in the layered wide kernel, a launch covers layers layer_arg ..
// layer_arg + lgroups - 1 and a workgroup owns its rows over the whole context of one of them;
// the beam's own tokens are merged in the prologue and o/l goes to the layer's hidden partial.
template <int NST, bool FUSED, int NW = 1, bool LAYERED = false>
__global__ __launch_bounds__(NW * 64) void k_ctx_attn_stream(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                             int layer_arg) {
  static_assert(NW == 1 || (NW == 2 && !FUSED), "one wave, or two waves per split-K or layered workgroup");
  static_assert(!(FUSED && LAYERED), "first-level fusion or layer slots, not both");
  constexpr int D = 128, TT = 32, KB = D / 16, DB = D / 32;
  constexpr int P = NST - 1;
  constexpr int NT = NW * 64;
  constexpr int KCH = TT * D / 8, VCH = D * TT / 8;  // 16-byte chunks per stage
  constexpr int KI = KCH / NT, VI = VCH / NT, LPT = KI + VI;  // copies per tile and wave
  static_assert(LPT * NW == 16 && NST >= 2 && NST <= 5, "wait immediates assume 16 copies per tile");
  __shared__ bf16x8_t sK[NST][KCH];
  __shared__ bf16x8_t sV[NST][VCH];

  // the wave index is uniform over the wave (it enters the copies' LDS address, an SGPR)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), hh = lane >> 5;
  const int kx = lane & 15, vx = ((lane >> 1) ^ (lane >> 3)) & 3;
  const int ri = find_req<0>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int local = blockIdx.x - R.wg_ctx;
  const int rest = local >> 3;
  const int rb = rest % R.row_blocks;
  const int pidx = (rest / R.row_blocks) * 8 + (local & 7);
  const int nparts = LAYERED ? R.lgroups : R.splits;  // layer slots, or token ranges
  if (pidx >= dm.Hkv * nparts) return;  // padding workgroup
  const int h = pidx / nparts, sp = pidx % nparts;
  const int layer = FUSED ? (int)blockIdx.y : layer_arg + (LAYERED ? sp : 0);
  if (LAYERED && layer >= dm.L) return;  // past the last layer of the last launch

  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int row0 = rb * (NW * 32);
  const int wrow = row0 + w * 32;
  const int q_row = wrow + (lane & 31);
  // the lane's query row: beam j_row, query head hq_row; its index loads go out before the
  // live-beam count is known
  const int j_row = q_row / dm.g, gi_row = q_row % dm.g, hq_row = h * dm.g + gi_row;
  const BeamIdx bi = load_beam_idx<LAYERED>(dev, slot, s, j_row);
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int rows = n_live * dm.g;
  if (row0 >= rows) return;  // whole workgroup idle
  const bool wave_active = wrow < rows;  // an idle wave still copies its share and meets the barriers
  const bool row_ok = q_row < rows;

  const int t0 = LAYERED ? 0 : sp * R.tps;
  const int t1 = LAYERED ? R.N : (sp == R.splits - 1 ? R.N : t0 + R.tps);
  const int ntiles = (t1 - t0 + TT - 1) / TT;
  const uint16_t *gK = (const uint16_t *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const uint16_t *gV = (const uint16_t *)R.ctx_vt + (size_t)layer * R.ctx_lstride + (size_t)h * D * R.Np;
  // copy i of wave w fills the 1 KB of the stage at (i * NW + w) * 1024: chunk p of the stage
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int p = (i * NW + w) * 64 + lane, rl = p >> 4, c = (p & 15) ^ (rl & 15);
    koff[i] = (uint32_t)(swap23(rl) * D + c * 8);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int p = (i * NW + w) * 64 + lane, row = p >> 2, c = (p & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
    voff[i] = (uint32_t)row * (uint32_t)R.Np + (uint32_t)(c * 8);
  }
  const uint32_t kdst = lds_addr(&sK[0][0]), vdst = lds_addr(&sV[0][0]);
  auto issue = [&](int tile) {
    const int st = tile % NST, tb = t0 + tile * TT;
    const uint16_t *kb = gK + (size_t)tb * D;
    const uint16_t *vb = gV + tb;
#pragma unroll
    for (int i = 0; i < KI; ++i) dma16(kb + koff[i], kdst + st * (KCH * 16) + (i * NW + w) * 1024);
#pragma unroll
    for (int i = 0; i < VI; ++i) dma16(vb + voff[i], vdst + st * (VCH * 16) + (i * NW + w) * 1024);
  };
  bf16x8_t qf[KB];
  const float kn = ((const float *)(slot + dev.sl.knmax))[layer * dm.Hkv + h];
  {
    // a row past the live beams reads the request's own q_last row and is zeroed
    const uint16_t *qsrc = (const uint16_t *)(slot + dev.sl.q_last) + (size_t)layer * dm.Hq * D;
    if (dm.chain)
      qsrc = dev.ch.q + ((size_t)(R.row0 + (row_ok ? j_row : 0)) * dm.Hq + (row_ok ? hq_row : 0)) * D;
    else if (row_ok)
      qsrc = s == 0 ? qsrc + (size_t)hq_row * D
                    : (const uint16_t *)dev.tok_q +
                          ((((size_t)layer * dm.tl + (s - 1)) * dm.V + bi.code) * dm.Hq + hq_row) * D;
    u32x4_t qr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qr[kb] = gld<u32x4_t>(qsrc + kb * 16 + 8 * hh);
    // the tiles the ring holds ahead of the first one, in flight with the query
#pragma unroll
    for (int k = 0; k < P; ++k)
      if (k < ntiles) issue(k);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qf[kb] = __builtin_bit_cast(bf16x8_t, row_ok ? qr[kb] : u32x4_t{0, 0, 0, 0});
  }
  const float c2 = dm.scale_log2;
  float M, l = 0.f;
  f32x16_t oacc[DB];  // zero, or set by the first own token
  float bmax;
  {
    float qn = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) qn = fmaf((float)qf[kb][e], (float)qf[kb][e], qn);
    qn += __shfl_xor(qn, 32);
    const float B = row_ok ? sqrtf(qn) * kn * c2 * 1.001f + 1e-3f : 0.f;
    M = B - 60.f;
    bmax = wave_max(B);
  }
  // the beam's own tokens, against the fixed reference (redone below on the lazy path)
  if (LAYERED && wave_active && s > 0) {
    wide_tail_merge<D>(dev, slot, layer, h, s, row_ok, j_row, gi_row, bi, hh, c2, true, qf, M, l, oacc, true);
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
  }
  if (!FUSED && !LAYERED && layer > 0 && R.defer_finish) {
    int r0, r1;
    finish_share(row0, min(rows, row0 + NW * 32) - row0, R.splits, sp, NT / (D / 8), r0, r1);
    finish_rows<D, 1>(dev, R, slot, layer - 1, h, r0, r1, tid, NT);
  }
  // per wave: both branches meet the same barriers, once per tile
  const bool fixed_ref = bmax <= 60.f;
  if (!fixed_ref) {
    M = kNegInf;
    if (LAYERED && wave_active) {
      l = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
      wide_tail_merge<D>(dev, slot, layer, h, s, row_ok, j_row, gi_row, bi, hh, c2, false, qf, M, l, oacc, false);
    }
  }

  auto tile_step = [&](int it, auto mask_tag, auto fixed_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool FIXED = decltype(fixed_tag)::value;
    const int st = it % NST;
    const bf16x8_t *kr = &sK[st][(lane & 31) * (D / 8)];
    const bf16x8_t *vr = &sV[st][(lane & 31) * (TT / 8)];
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[(kb * 2 + hh) ^ kx], qf[kb], sacc, 0, 0, 0);
    if constexpr (MASK) {
      const int tbase = t0 + it * TT + 8 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tbase + 16 * (i >> 3) + (i & 7) >= t1) sacc[i] = kNegInf;
    }
    if constexpr (!FIXED) {
      float mx = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * c2;
      if (__ballot(mxs > M + 8.f) != 0ull) {
        const float Mn = fmaxf(M, mxs);
        const float f = fast_exp2(M - Mn);
        l *= f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= f;
        M = Mn;
      }
    }
    bf16x8_t pf[2], pl[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(sacc[i], c2, -M));
      const __bf16 ph = (__bf16)p;
      pf[i >> 3][i & 7] = ph;
      pl[i >> 3][i & 7] = (__bf16)(p - (float)ph);
      l += p;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const bf16x8_t vf = vr[db * 32 * (TT / 8) + ((pp * 2 + hh) ^ vx)];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pp], oacc[db], 0, 0, 0);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[pp], oacc[db], 0, 0, 0);
      }
    }
  };
  auto run = [&](auto fixed_tag) {
    using F = decltype(fixed_tag);
    const bool partial = ((t1 - t0) % TT) != 0;
    for (int it = 0; it < ntiles; ++it) {
      // tile it has landed once at most the copies of the later tiles already issued remain
      const int ahead = min(P - 1, ntiles - 1 - it);
      if constexpr (NW == 1) {
        if (ahead >= 3) vm_wait<3 * LPT>();
        else if (ahead == 2) vm_wait<2 * LPT>();
        else if (ahead == 1) vm_wait<LPT>();
        else vm_wait<0>();
      } else {
        // every wave's copies of tile it have landed, and every wave is past tile it-1
        if (ahead >= 3) vm_wait_barrier8<3 * LPT>();
        else if (ahead == 2) vm_wait_barrier8<2 * LPT>();
        else if (ahead == 1) vm_wait_barrier8<LPT>();
        else vm_wait_barrier8<0>();
      }
      if (it + P < ntiles) issue(it + P);  // into the stage of tile it-1, read by now
      if (!wave_active) continue;
      if (it + 1 < ntiles || !partial)
        tile_step(it, std::false_type{}, F{});
      else
        tile_step(it, std::true_type{}, F{});
    }
  };
  if (fixed_ref)
    run(std::true_type{});
  else
    run(std::false_type{});

  const float ltot = l + __shfl_xor(l, 32);
  if (LAYERED) {
    if (wave_active && row_ok)
      wide_store_layer<D>(dev, R, slot, layer, j_row, hq_row, hh, ltot, oacc, true);
  } else if (wave_active && row_ok) {
    const size_t lofs = FUSED ? (size_t)layer * dm.Hkv * R.splits * R.rows_b : 0;
    const int pb = FUSED ? 0 : layer & 1;
    const size_t prow = lofs + ((size_t)h * R.splits + sp) * R.rows_b + q_row;
    store_partial<DB>(slot, dev.sl, pb, prow, M, ltot, hh, oacc);
  }
}

// The beam's own tokens t < s for the lane's query row (beam j, head of kv head kv) in the
// layered wide kernel, merged online into (M, l, o) before the context loop: the newest token
// from the token tables (appended to BeamKV by the gi == 0 row of the beam), older ones from
// BeamKV at the beam's ancestry.  qf holds the lane's features kb*16 + 8hh .. +8; oacc[db][4a + c]
// is feature db*32 + 8a + 4hh + c.  A row's two lanes compute the same scores, and only the
// hh == 0 lane counts p in l (l of the two lanes is summed at the end).  Lanes of rows past the
// live beams load nothing but take part in the shuffles.
template <int D, int NTOK>
__device__ __forceinline__ void tail_load_pair(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                               int j, const BeamIdx &bi, int hh, int t0, TailPair<D, NTOK> &tp) {
  constexpr int KB = D / 16;
  const Dims &dm = dev.dm;
  const int lvl = dm.levels;
  const size_t wstride = (size_t)dm.Hkv * D;  // one BeamKV slot
  const size_t lvstride = (size_t)dm.W_max * wstride;
  const size_t lbase = (size_t)layer * dm.tl * lvstride + (size_t)kv * D;
  const size_t tbase = (size_t)layer * dm.tl * dm.V * dm.Hkv + kv;  // token-table row, level 0, code 0
#pragma unroll
  for (int e = 0; e < NTOK; ++e) {
    const int t = t0 + e;
    // element offset into tok_k/tok_v, or into BeamKV when `own`; selected without branches
    const bool valid = row_ok && t < s, table = t == s - 1;
    uint32_t a = bi.anc0;
    if (t > 0 && t < s - 1)  // uniform: an older own token beyond the first
      a = valid ? ((const uint32_t *)(slot + dev.sl.anc[s & 1]))[j * lvl + t] : 0u;
    const size_t krow_tab = (tbase + ((size_t)t * dm.V + bi.code) * dm.Hkv) * D;
    const size_t krow_own = lbase + (size_t)t * lvstride + (size_t)a * wstride;
    const bool own = valid && !table;
    const size_t krow = own ? krow_own : valid ? krow_tab : tbase * D;
    const uint16_t *kp = (own ? (const uint16_t *)(slot + dev.sl.beamkv_k) : (const uint16_t *)dev.tok_k) + krow;
    const uint16_t *vp = (own ? (const uint16_t *)(slot + dev.sl.beamkv_v) : (const uint16_t *)dev.tok_v) + krow;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) tp.kr[e][kb] = gld<u32x4_t>(kp + kb * 16 + 8 * hh);
#pragma unroll
    for (int q = 0; q < D / 8; ++q) tp.vr[e][q] = gld<u32x2_t>(vp + (q >> 2) * 32 + 8 * (q & 3) + 4 * hh);
  }
}

// Online-softmax update of (M, l, oacc) with the pair's tokens, in level order, against the
// running reference M; the row with gi == 0 appends its query token's key and value to BeamKV.
// fresh: l and oacc are still zero (and M finite or -inf), so the first token sets them, which
// is what the update gives (f <= 1), without reading zero accumulators.
template <int D, int NTOK>
__device__ __forceinline__ void tail_merge_pair(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                                int j, int gi, int hh, float c2, int t0, const TailPair<D, NTOK> &tp,
                                                const bf16x8_t (&qf)[D / 16], float &M, float &l,
                                                f32x16_t (&oacc)[D / 32], bool append, bool fresh) {
  constexpr int KB = D / 16, DB = D / 32;
  const Dims &dm = dev.dm;
  const int lvl = dm.levels;
  uint16_t *bk = (uint16_t *)(slot + dev.sl.beamkv_k);
  uint16_t *bv = (uint16_t *)(slot + dev.sl.beamkv_v);
  const size_t wstride = (size_t)dm.Hkv * D;
  const size_t lvstride = (size_t)dm.W_max * wstride;
  const size_t lbase = (size_t)layer * dm.tl * lvstride + (size_t)kv * D;
#pragma unroll
  for (int e = 0; e < NTOK; ++e) {
    const int t = t0 + e;
    if (t >= s) break;
    const bool app = append && t == s - 1 && row_ok && gi == 0;
    const size_t dst = lbase + (size_t)t * lvstride + (size_t)j * wstride;
    float dot = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        dot = fmaf((float)qf[kb][2 * x], __uint_as_float(tp.kr[e][kb][x] << 16), dot);
        dot = fmaf((float)qf[kb][2 * x + 1], __uint_as_float(tp.kr[e][kb][x] & 0xFFFF0000u), dot);
      }
      if (app) gst<u32x4_t>(bk + dst + kb * 16 + 8 * hh, tp.kr[e][kb]);
    }
    dot += __shfl_xor(dot, 32);
    const float u = dot * c2;
    const float Mn = fmaxf(M, u);
    const float f = fast_exp2(M - Mn);  // M = -inf before the first token of the lazy path: f = 0
    const float p = fast_exp2(u - Mn);
    const bool first = fresh && e == 0;
    l = first ? (hh == 0 ? p : 0.f) : fmaf(l, f, hh == 0 ? p : 0.f);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t wv = tp.vr[e][db * 4 + (i >> 2)][(i & 3) >> 1];
        const float v = __uint_as_float((i & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
        oacc[db][i] = first ? p * v : fmaf(p, v, oacc[db][i] * f);
      }
    }
    if (app) {
#pragma unroll
      for (int q = 0; q < DB * 4; ++q) gst<u32x2_t>(bv + dst + (q >> 2) * 32 + 8 * (q & 3) + 4 * hh, tp.vr[e][q]);
    }
    M = Mn;
  }
}

// The own tokens in level order, each key and value in one round trip; the first of them
// sets l and oacc when fresh (both still zero).
template <int D>
__device__ __forceinline__ void wide_tail_merge(const Dev &dev, uint8_t *slot, int layer, int kv, int s, bool row_ok,
                                                int j, int gi, const BeamIdx &bi, int hh, float c2, bool fresh,
                                                const bf16x8_t (&qf)[D / 16], float &M, float &l,
                                                f32x16_t (&oacc)[D / 32], bool append) {
  for (int t = 0; t < s; ++t) {
    TailPair<D, 1> tp;
    tail_load_pair<D, 1>(dev, slot, layer, kv, s, row_ok, j, bi, hh, t, tp);
    tail_merge_pair<D, 1>(dev, slot, layer, kv, s, row_ok, j, gi, hh, c2, t, tp, qf, M, l, oacc, append,
                          fresh && t == 0);
  }
}

// Layer output o/l of the lane's query row in the full-context kernels: to the debug rows, and
// stored (never read back here) in float32 as the layer's partial of the hidden vector;
// k_sum_hparts adds the layers' rows in layer order.  Lanes (row, hh) and (row, hh ^ 1) hold
// the two halves of the row's features.
template <int D>
__device__ __forceinline__ void wide_store_layer(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int j,
                                                 int hq, int hh, float ltot, const f32x16_t (&oacc)[D / 32],
                                                 bool row_ok) {
  constexpr int DB = D / 32;
  const Dims &dm = dev.dm;
  const float inv = 1.f / ltot;
  if (!row_ok) return;
  const size_t row = ((size_t)layer * dm.W_max + j) * dm.Hq + hq;
  float *hp = (float *)(slot + dev.sl.hl) + row * D;
  float *dg = dm.debug_attn ? (float *)(slot + dev.sl.dbg_attn) + row * D : nullptr;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int f0 = db * 32 + 8 * a + 4 * hh;
      const f32x4_t o = f32x4_t{oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv, oacc[db][4 * a + 2] * inv,
                                oacc[db][4 * a + 3] * inv};
      if (dg) gst<f32x4_t>(dg + f0, o);
      gst<f32x4_t>(hp + f0, o);
    }
}

// The wide context kernel: 8 waves x 32 query rows (256 rows of one kv head) against K and V^T
// tiles of 64 tokens that go from HBM straight into LDS through a ring of five stages.  Each
// V^T tile is rewritten in place, once it has landed, as float16 of v / vscale, where vscale =
// 2^e is the power of two above the head's largest |v| (taken at load; 1 when that lies in
// [2^-10, 2^15], where float16 of v itself is as good); a bf16 value converts exactly while
// |v| >= 2^-14 vscale, and below that to within 2^-25 vscale.  P is then a single
// float16 term (relative rounding 2^-11) and PV one f16 MFMA per 16 tokens.  The softmax keeps
// a running maximum with a lazy rescale: only when a row's maximum grows by more than 8 in log2
// units, so every p stays within (0, 2^8].  A tile is converted while its predecessor is in
// use, one barrier before its first PV.
//
// LAYERED: a launch covers layers layer_arg .. layer_arg + lgroups - 1, and a workgroup owns its
// row block over the whole context of one of them, layer_arg + g (every layer's query comes
// from the token tables or the request, never from another layer's output).  It then finishes
// its rows itself, with no split partials: the beam's own tokens are merged into (m, l, o) in
// the prologue (the newest one appended to BeamKV), the context loop continues from that
// state, and o/l is stored as the layer's float32 hidden partial (k_sum_hparts adds the layers
// in order at the end).  Otherwise: one layer, one token range, split partials out, and the
// previous layer finished in the prologue when the step defers it.
// Units of V in the eight-wave kernel's float16 PV: with the head's values between 2^-11 and
// 2^15 in magnitude (vscale = 2^e above max|v| in [2^-10, 2^15]) float16 of v itself is exact
// for |v| >= 2^-14 and within 2^-25 below, so v is taken as it is (raw); otherwise in units of
// vscale.  Returns the factor v is multiplied by (1, or 1/vscale: exact, a power of two).
__device__ __forceinline__ float v16_factor(float vsc, bool &raw) {
  raw = vsc >= 0x1p-10f && vsc <= 0x1p15f;
  return raw ? 1.f : 1.f / vsc;
}

// Loads of a beam code and of the live-beam count, then the four copies of a wave's share of a
// tile (two K, two V^T chunks of 1 KB), and a wait for the two loads only (vmcnt counts
// outstanding vector memory operations, which complete in issue order): one block, so the two
// results are complete when it ends and the compiler, which does not see the copies, keeps no
// wait of its own on them.  The copies are waited for by the caller.
__device__ __forceinline__ void idx_and_tile0(const uint32_t *code_p, const int *nl_p, const uint16_t *k0,
                                              const uint16_t *k1, const uint16_t *v0, const uint16_t *v1,
                                              uint32_t lk0, uint32_t lk1, uint32_t lv0, uint32_t lv1,
                                              uint32_t &code, uint32_t &nl) {
  asm volatile(
      "global_load_dword %0, %2, off\n\t"
      "global_load_dword %1, %3, off\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, off\n\t"
      "s_mov_b32 m0, %10\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, off\n\t"
      "s_mov_b32 m0, %11\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, off\n\t"
      "s_waitcnt vmcnt(4)"
      : "=&v"(code), "=&v"(nl)
      : "v"(code_p), "v"(nl_p), "v"(k0), "v"(k1), "v"(v0), "v"(v1), "s"(lk0), "s"(lk1), "s"(lv0), "s"(lv1)
      : "memory", "m0");
}

template <bool LAYERED>
__global__ __launch_bounds__(512) void k_ctx_attn_wide(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                       int layer_arg) {
  constexpr int D = 128, NW = 8, TT = 64, KB = D / 16, DB = D / 32, NT = NW * 64, NST = 5;
  constexpr int KCH = TT * D / 8, VCH = D * TT / 8;  // 16-byte chunks per stage
  constexpr int KI = KCH / NT, VI = VCH / NT;        // DMA instructions per wave and tile
  constexpr int LPT = KI + VI;
  static_assert(LPT == 4 && KI == 2 && VI == 2, "wait immediates assume four copies per lane and tile");
  static_assert(TT == kTileTok, "tiles never cross the zero-padded end of the context");
  __shared__ bf16x8_t sK[NST][KCH];   // [token row swap23(r)][column c ^ (row & 15)]
  __shared__ u32x4_t sV[NST][VCH];    // [feature row][token column c ^ (row & 7) ^ (row >> 3 & 1)]

  long long wt[kWaveTimesFields] = {};  // the wave timeline (GR_WAVE_TIMES builds only)
  if constexpr (kWaveTimes) wt[0] = wall_clock64();
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5;
  const int kx = lane & 15, vx = (lane & 7) ^ ((lane >> 3) & 1);  // swizzle of this lane's operand row
  // the model's and then the descriptor's fields that the prologue reads, in SGPRs at once (the
  // first with the request lookup's own loads): a round trip each, not a chain of loads each
  // behind the branch that first needs it
  const Dims &dm = dev.dm;
  asm volatile("" ::"s"(dm.L), "s"(dm.Hq), "s"(dm.Hkv), "s"(dm.g), "s"(dm.levels), "s"(dm.V), "s"(dm.W_max),
               "s"(dm.chain), "s"(dm.tl), "s"(dm.scale_log2), "s"(dev.slots), "s"(dev.sl.slot_bytes),
               "s"(dev.sl.n_live), "s"(dev.sl.codes[0]), "s"(dev.sl.codes[1]), "s"(dev.sl.vscale),
               "s"(dev.sl.q_last), "s"(dev.tok_q), "s"(dev.ch.q));
  const int ri = find_req<0>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  asm volatile("" ::"s"(R.ctx_k), "s"(R.ctx_vt), "s"(R.ctx_vt16), "s"(R.ctx_lstride), "s"(R.N), "s"(R.Np),
               "s"(R.slot), "s"(R.level), "s"(R.rows_b), "s"(R.splits), "s"(R.tps), "s"(R.lgroups),
               "s"(R.defer_finish), "s"(R.row0), "s"(R.row_blocks), "s"(R.wg_ctx));
  const int local = blockIdx.x - R.wg_ctx;
  const int rest = local >> 3;
  const int rb = rest % R.row_blocks;
  const int pidx = (rest / R.row_blocks) * 8 + (local & 7);
  const int nparts = LAYERED ? R.lgroups : R.splits;  // layer groups, or token ranges
  if (pidx >= dm.Hkv * nparts) return;  // padding workgroup
  const int h = pidx / nparts, sp = pidx % nparts;

  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int row0 = rb * (NW * 32);
  const int wrow = row0 + w * 32;
  const int q_row = wrow + (lane & 31);
  // the row's beam j, query head hq and latest code (its query token at steps s >= 1), and
  // the BeamKV slots of its older tokens: loaded before the live-beam count is known
  const int j_row = q_row / dm.g, gi_row = q_row % dm.g, hq_row = h * dm.g + gi_row;

  const int t0 = LAYERED ? 0 : sp * R.tps;
  const int t1 = LAYERED ? R.N : (sp == R.splits - 1 ? R.N : t0 + R.tps);
  const int ntiles = (t1 - t0 + TT - 1) / TT;  // at least one
  const int nsub = (t1 - t0 + 31) / 32;
  const int layer = layer_arg + (LAYERED ? sp : 0);
  if (layer >= dm.L) return;  // past the last layer of the last launch
  // V^T as float16 in the kernel's units when the context has that copy (v16), else bf16
  // converted in LDS after each tile lands
  const bool v16 = R.ctx_vt16 != nullptr;  // uniform
  const uint16_t *gK = (const uint16_t *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const uint16_t *gV = (const uint16_t *)(v16 ? R.ctx_vt16 : R.ctx_vt) + (size_t)layer * R.ctx_lstride +
                       (size_t)h * D * R.Np;

  // per-lane DMA sources (elements from the tile's first token) for this wave's chunks
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int p = (w * KI + i) * 64 + lane, rl = p >> 4, c = (p & 15) ^ (rl & 15);
    koff[i] = (uint32_t)(swap23(rl) * D + c * 8);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int p = (w * VI + i) * 64 + lane, row = p >> 3, c = (p & 7) ^ (row & 7) ^ ((row >> 3) & 1);
    voff[i] = (uint32_t)row * (uint32_t)R.Np + (uint32_t)(c * 8);
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t kdst = lds_addr(&sK[0][0]) + wu * KI * 1024, vdst = lds_addr(&sV[0][0]) + wu * VI * 1024;
  auto issue = [&](int tile) {
    const int st = tile % NST, tb = t0 + tile * TT;
    const uint16_t *kb = gK + (size_t)tb * D;
    const uint16_t *vb = gV + tb;
#pragma unroll
    for (int i = 0; i < KI; ++i) dma16(kb + koff[i], kdst + st * (KCH * 16) + i * 1024);
#pragma unroll
    for (int i = 0; i < VI; ++i) dma16(vb + voff[i], vdst + st * (VCH * 16) + i * 1024);
  };
  // the row's beam index and the live-beam count; per-layer launches load them with tile 0's
  // copies right behind, waiting for the two loads only, so the query gather that depends on
  // them overlaps the tile's fetch
  BeamIdx bi;
  int n_live;
  if constexpr (LAYERED) {
    bi = load_beam_idx<true>(dev, slot, s, j_row);
    n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  } else {
    const int jj = min(j_row, dm.W_max - 1);
    const size_t codes = (s & 1) ? dev.sl.codes[1] : dev.sl.codes[0];  // both in SGPRs already
    const uint32_t *cp = (const uint32_t *)(slot + codes) + jj * dm.levels + max(s - 1, 0);
    uint32_t code, nl;
    idx_and_tile0(cp, (const int *)(slot + dev.sl.n_live) + (s & 1), gK + t0 * D + koff[0], gK + t0 * D + koff[1],
                  gV + t0 + voff[0], gV + t0 + voff[1], kdst, kdst + 1024, vdst, vdst + 1024, code, nl);
    bi.code = s > 0 ? code : 0u;
    bi.anc0 = 0u;
    n_live = __builtin_amdgcn_readfirstlane((int)nl);
  }
  const int rows = n_live * dm.g;
  if (row0 >= rows) {  // whole workgroup idle; tile 0 lands before the LDS is released
    if (!LAYERED) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  const bool wave_active = wrow < rows;  // an idle wave still copies and converts its share
  const bool row_ok = q_row < rows;
  const float vsc = ((const float *)(slot + dev.sl.vscale))[layer * dm.Hkv + h];
  bool vraw;
  const float ivs = v16_factor(vsc, vraw);
  const float vs = vraw ? 1.f : vsc;
  // V^T of a landed tile -> float16 of v / vscale, in place (each thread two 16-byte chunks)
  auto convert_v = [&](int tile) {
    u32x4_t *sv = &sV[tile % NST][0];
#pragma unroll
    for (int i = 0; i < VCH / NT; ++i) {
      const u32x4_t x = sv[i * NT + tid];
      u32x4_t y;
      if (vraw) {  // uniform over the workgroup
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = pack_f16(__uint_as_float(x[e] << 16), __uint_as_float(x[e] & 0xFFFF0000u));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = pack_f16(__uint_as_float(x[e] << 16) * ivs, __uint_as_float(x[e] & 0xFFFF0000u) * ivs);
      }
      sv[i * NT + tid] = y;
    }
  };
  const float c2 = dm.scale_log2;
  bf16x8_t qf[KB];  // B operand of QK^T: lane holds Q[q_row][kb*16 + 8*hh .. +8]
  float M = kNegInf, l = 0.f;
  f32x16_t oacc[DB];

  auto qk = [&](int tile, int sub) {
    const bf16x8_t *kr = &sK[tile % NST][(sub * 32 + (lane & 31)) * (D / 8)];
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[(kb * 2 + hh) ^ kx], qf[kb], acc, 0, 0, 0);
    return acc;
  };
  // lazy rescale before the sub-tile whose lane maxima of the scores are mx: a row's maximum
  // (x log2 e / sqrt(d)) outgrows M + 8 exactly when one of its two lanes' does, so the lanes
  // exchange their maxima only on that (rare) path
  auto rescale = [&](float mx) {
    if (__ballot(mx * c2 > M + 8.f) != 0ull) {  // uniform over the wave
      const float mxs = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
      const float Mn = fmaxf(M, mxs);
      const float f = fast_exp2(M - Mn);  // 0 before the first sub-tile (M = -inf)
      l *= f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= f;
      M = Mn;
    }
  };
  auto smax = [&](const f32x16_t &sc) {
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    return mx;
  };
  // The token loop carries a sub-tile's scores as exponent arguments a = s x log2 e / sqrt(d) - M
  // (converted once, right after the QK^T: the maximum is then taken over arithmetic results,
  // which need no quieting, three at a time).  The lazy rescale on arguments whose lane maximum
  // is mx: a row whose arguments exceed 8 moves M up by its largest argument, its l and o scale
  // by exp2 of the difference, and its arguments shift by the same difference.
  auto rescale_args = [&](float mx, f32x16_t &a) {
    if (__ballot(mx > 8.f) != 0ull) {  // uniform over the wave
      const float Mn = M + fmaxf(fmaxf(mx, __shfl_xor(mx, 32)), 0.f);
      const float e = M - Mn;
      const float f = fast_exp2(e);
      l *= f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a[i] += e;
      M = Mn;
    }
  };
  auto to_args = [&](f32x16_t &a) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = fmaf(a[i], c2, -M);
  };
  const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  // softmax of sub-tile u (first token t0 + 32u) and PV with its tile's V^T (tail sub-tiles);
  // sacc holds exponent arguments (ARGS, rescaled already) or raw scores
  auto soft_pv = [&](f32x16_t sacc, int u, auto mask_tag, auto args_tag) {
    constexpr bool MASK = decltype(mask_tag)::value, ARGS = decltype(args_tag)::value;
    if constexpr (MASK) {
      const int tbase = t0 + u * 32 + 8 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tbase + 16 * (i >> 3) + (i & 7) >= t1) sacc[i] = kNegInf;
    }
    if constexpr (!ARGS) {
      rescale(smax(sacc));
      to_args(sacc);
    }
    f16x8_t pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pf[i >> 3][i & 7] = (_Float16)fast_exp2(sacc[i]);
#pragma unroll
    for (int i = 0; i < 16; i += 2)
      l = __builtin_amdgcn_fdot2(f16x2_t{pf[i >> 3][i & 7], pf[i >> 3][(i & 7) + 1]}, ones, l, false);
    const int tile = u >> 1, sub = u & 1;
    const u32x4_t *vr = &sV[tile % NST][(lane & 31) * (TT / 8)];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const f16x8_t vf = __builtin_bit_cast(f16x8_t, vr[db * 32 * (TT / 8) + ((sub * 4 + pp * 2 + hh) ^ vx)]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[pp], oacc[db], 0, 0, 0);
      }
  };
  // Steady-state step, sub-tile u unmasked: QK^T of sub-tile u+1 and softmax + PV of sub-tile
  // u, interleaved by hand.  Issue is in order within a wave, so the softmax is spread over the
  // wave's own MFMAs, giving each wave independent VALU work between its MFMAs (the two waves of
  // a SIMD then keep the matrix core fed): element k (k < 8) after the k-th QK^T MFMA, elements
  // 8..15 two at a time after the first four PV MFMAs (those use the first eight only), and
  // sub-tile u+1's scores turned into arguments, with their maxima, over the last four, for its
  // lazy rescale at the end.  LDS
  // operands are fetched two MFMAs ahead; sched_barrier keeps the order.  kr: the K rows of the
  // QK^T sub-tile, vr: the V^T tile of the PV sub-tile spv.  With compile-time stages
  // (block_st) every operand address is a per-lane register plus an immediate offset.
  auto block_p = [&](const bf16x8_t *kr, const u32x4_t *vr, int spv, const f32x16_t &sc) {
    auto kfrag = [&](int kb) { return kr[(kb * 2 + hh) ^ kx]; };
    auto vfrag = [&](int j) {  // j = pp*4 + db
      return __builtin_bit_cast(f16x8_t, vr[(j & 3) * 32 * (TT / 8) + ((spv * 4 + (j >> 2) * 2 + hh) ^ vx)]);
    };
    bf16x8_t kf[3];
    f16x8_t vf[3], pf[2];
    float pr[8], mx = 0.f;
    // the pair (i, i+1) of P and its share of l (exactly the float16 weights the MFMAs use)
    auto pair = [&](float p0, float p1, int i) {
      const f16x2_t h2 = {(_Float16)p0, (_Float16)p1};
      pf[i >> 3][i & 7] = h2[0];
      pf[i >> 3][(i + 1) & 7] = h2[1];
      l = __builtin_amdgcn_fdot2(h2, ones, l, false);
    };
    kf[0] = kfrag(0);
    kf[1] = kfrag(1);
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (kb + 2 < KB) kf[(kb + 2) % 3] = kfrag(kb + 2);
      else vf[(kb + 2 - KB) % 3] = vfrag(kb + 2 - KB);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb % 3], qf[kb], acc, 0, 0, 0);
      pr[kb] = fast_exp2(sc[kb]);
      if (kb & 1) pair(pr[kb - 1], pr[kb], kb - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 2 < 8) vf[(j + 2) % 3] = vfrag(j + 2);
      oacc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[j % 3], pf[j >> 2], oacc[j & 3], 0, 0, 0);
      if (j < 4) {
        pair(fast_exp2(sc[8 + 2 * j]), fast_exp2(sc[9 + 2 * j]), 8 + 2 * j);
      } else {
        // sub-tile u+1's scores to arguments, four per step, and their maximum
        const int b = 4 * (j - 4);
#pragma unroll
        for (int i = b; i < b + 4; ++i) acc[i] = fmaf(acc[i], c2, -M);
        const float m4 = fmaxf(fmaxf(acc[b], acc[b + 1]), fmaxf(acc[b + 2], acc[b + 3]));
        mx = j == 4 ? m4 : fmaxf(mx, m4);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    rescale_args(mx, acc);
    return acc;
  };
  static_assert(KB == 8, "the interleave assumes eight QK^T MFMAs per sub-tile");
  auto block = [&](int u, const f32x16_t &sc) {
    const int tq = (u + 1) >> 1, sq = (u + 1) & 1, tp = u >> 1;
    return block_p(&sK[tq % NST][(sq * 32 + (lane & 31)) * (D / 8)], &sV[tp % NST][(lane & 31) * (TT / 8)], u & 1,
                   sc);
  };
  // sub-tile u = 2*it + SPV with it % NST == ST (QK^T of sub-tile u+1, PV of sub-tile u)
  auto block_st = [&](auto st_tag, auto spv_tag, const f32x16_t &sc) {
    constexpr int ST = decltype(st_tag)::value, SPV = decltype(spv_tag)::value;
    constexpr int KST = SPV ? (ST + 1) % NST : ST, SQ = SPV ? 0 : 1;
    return block_p(&sK[KST][(SQ * 32 + (lane & 31)) * (D / 8)], &sV[ST][(lane & 31) * (TT / 8)], SPV, sc);
  };

  // between the blocks of sub-tiles 2T-2 and 2T-1 (T >= 1): tile T+1 has landed (only tile T+2
  // may still be in flight), then the barrier (every wave is past sub-tile 2T-3, the last use
  // of tile T-2, and the V^T of tile T, converted before, is visible), tile T+3 goes into the
  // stage of tile T-2, and tile T+1's V^T is converted
  auto advance = [&](int T) {
    if constexpr (kWaveTimes) {
      const long long ta = __builtin_amdgcn_s_memtime();
      if (T + 2 < ntiles) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      const long long tb = __builtin_amdgcn_s_memtime();
      asm volatile("s_barrier" ::: "memory");
      wt[4] += tb - ta;
      wt[5] += __builtin_amdgcn_s_memtime() - tb;
      wt[7] += 1;
    } else if (T + 2 < ntiles) {
      vm_lgkm_wait_barrier<LPT>();
    } else {
      vm_lgkm_wait_barrier<0>();
    }
    if (T + 3 < ntiles) issue(T + 3);
    if (!v16 && T + 1 < ntiles) convert_v(T + 1);
  };

  {
    // a row past the live beams reads the request's own q_last row and is zeroed
    const uint16_t *qsrc = (const uint16_t *)(slot + dev.sl.q_last) + (size_t)layer * dm.Hq * D;
    if (dm.chain)
      qsrc = dev.ch.q + ((size_t)(R.row0 + (row_ok ? j_row : 0)) * dm.Hq + (row_ok ? hq_row : 0)) * D;
    else if (row_ok)
      qsrc = s == 0 ? qsrc + (size_t)hq_row * D
                    : (const uint16_t *)dev.tok_q +
                          ((((size_t)layer * dm.tl + (s - 1)) * dm.V + bi.code) * dm.Hq + hq_row) * D;
    u32x4_t qr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qr[kb] = gld<u32x4_t>(qsrc + kb * 16 + 8 * hh);
    // the tiles the prologue needs in flight with the query (tile 0, out already in per-layer
    // launches, and tile 1 when its V^T is converted here); the rest of the ring's tiles once
    // those have landed: at the start of a launch every workgroup waits only for its first
    // tiles, not for the whole chip's first four
    const int first = v16 ? 1 : 2;
    for (int k = LAYERED ? 0 : 1; k < first; ++k)
      if (k < ntiles) issue(k);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      qf[kb] = __builtin_bit_cast(bf16x8_t, row_ok ? qr[kb] : u32x4_t{0, 0, 0, 0});
      asm volatile("" ::"v"(qf[kb]));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int k = first; k < NST - 1; ++k)
      if (k < ntiles) issue(k);
  }
  if (LAYERED && s > 0) {
    // the beam's own tokens (the first sets (M, l, o)), then o in units of vscale like the
    // context's contributions
    wide_tail_merge<D>(dev, slot, layer, h, s, row_ok, j_row, gi_row, bi, hh, c2, true, qf, M, l, oacc, true);
    if (!vraw) {
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= ivs;
    }
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
  }
  if (!LAYERED && layer > 0 && R.defer_finish) {
    // finish the previous layer for this workgroup's share of the row block
    int r0, r1;
    finish_share(row0, min(rows, row0 + NW * 32) - row0, R.splits, sp, 2 * NT / (D / 8), r0, r1);
    finish_rows<D, 2>(dev, R, slot, layer - 1, h, r0, r1, tid, NT);
  }
  // every wave's first tiles have landed (tile 0, and tile 1 when it is converted here; the
  // later ones may be in flight; after prologue work with memory accesses of its own,
  // everything is waited for, so that the ring's waits count copies only); the barrier makes
  // every wave's copies visible.  Tiles 0 and 1 are converted here (without the float16 copy),
  // every later one in advance(); tile 1 is in LDS by the first advance() (which waits for tile
  // 2), before sub-tile 2 reads it
  if (LAYERED ? s > 0 : layer > 0 && R.defer_finish)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (!v16) {
    convert_v(0);
    if (ntiles > 1) convert_v(1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if constexpr (kWaveTimes) {
    wt[1] = wall_clock64();
    wt[6] = __builtin_amdgcn_s_memtime();
  }
  // s0 holds the exponent arguments of even sub-tiles, s1 of odd ones
  f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
  if (wave_active) {
    s0 = qk(0, 0);
    rescale(smax(s0));
    to_args(s0);
  }
  // steady state: both sub-tiles of tile it are unmasked and tile it+1 exists; NST tiles at a
  // time with compile-time stages, then one at a time
  int it = 0;
  auto step = [&](auto st_tag) {
    if (wave_active) s1 = block_st(st_tag, std::integral_constant<int, 0>{}, s0);
    advance(it + 1);
    if (wave_active) s0 = block_st(st_tag, std::integral_constant<int, 1>{}, s1);
    ++it;
  };
  while (2 * (it + NST - 1) + 2 < nsub) {
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
  }
  for (; 2 * it + 2 < nsub; ++it) {
    if (wave_active) s1 = block(2 * it, s0);
    advance(it + 1);
    if (wave_active) s0 = block(2 * it + 1, s1);
  }
  // tail: one or two sub-tiles of the last tile; only the very last one can be partial
  const bool partial = ((t1 - t0) & 31) != 0;
  if (wave_active) {
    if (2 * it + 1 < nsub) {
      s1 = qk(it, 1);
      soft_pv(s0, 2 * it, std::false_type{}, std::true_type{});
      if (partial)
        soft_pv(s1, nsub - 1, std::true_type{}, std::false_type{});
      else
        soft_pv(s1, nsub - 1, std::false_type{}, std::false_type{});
    } else if (partial) {
      soft_pv(s0, nsub - 1, std::true_type{}, std::true_type{});
    } else {
      soft_pv(s0, nsub - 1, std::false_type{}, std::true_type{});
    }
  }

  if constexpr (kWaveTimes) {
    wt[2] = wall_clock64();
    wt[6] = __builtin_amdgcn_s_memtime() - wt[6];
  }
  // back to units of v
  if (!vraw) {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= vs;
  }
  const float ltot = l + __shfl_xor(l, 32);
  if constexpr (!LAYERED) {
    if (wave_active && row_ok) {
      const size_t prow = ((size_t)h * R.splits + sp) * R.rows_b + q_row;
      store_partial<DB>(slot, dev.sl, layer & 1, prow, M, ltot, hh, oacc);
    }
    if constexpr (kWaveTimes) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      wt[3] = wall_clock64();
      if (lane == 0 && wave_active && s == g_wave_times_sel[0] && layer == g_wave_times_sel[1] &&
          blockIdx.x < kWaveTimesWgs) {
        long long *o = g_wave_times + ((size_t)blockIdx.x * 8 + w) * kWaveTimesFields;
#pragma unroll
        for (int f = 0; f < kWaveTimesFields; ++f) o[f] = wt[f];
      }
    }
  } else {
    if (row_ok) wide_store_layer<D>(dev, R, slot, layer, j_row, hq_row, hh, ltot, oacc, true);
  }
}

// --------------------------------------------------------------------------------------
// Shared-context attention for float32 models (vector ALU).  One wave per
// (request, kv head, query row, token range); lane = token for the scores,
// lane = feature for the output.
template <int D>
__global__ __launch_bounds__(256) void k_ctx_attn_f32(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                      int layer) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ri = find_req<0>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  int lw = (blockIdx.x - R.wg_ctx) * 4 + w;
  const int sp = lw % R.splits;
  lw /= R.splits;
  const int q_row = lw % R.rows_b;
  const int h = lw / R.rows_b;
  if (h >= dm.Hkv) return;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  if (q_row >= n_live * dm.g) return;
  const int j = q_row / dm.g, hq = h * dm.g + q_row % dm.g;
  const float *q;
  if (s == 0) {
    q = (const float *)(slot + dev.sl.q_last) + ((size_t)layer * dm.Hq + hq) * D;
  } else {
    const int code = ((const int *)(slot + dev.sl.codes[s & 1]))[j * dm.levels + (s - 1)];
    q = (const float *)dev.tok_q + ((((size_t)layer * dm.tl + (s - 1)) * dm.V + code) * dm.Hq + hq) * D;
  }
  const float *gK = (const float *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const float *gV = (const float *)R.ctx_vt + (size_t)layer * R.ctx_lstride + (size_t)h * D * R.Np;
  const int t0 = sp * R.tps, t1 = (sp == R.splits - 1 ? R.N : t0 + R.tps);
  const float c2 = dm.scale_log2;
  float M = kNegInf, l = 0.f, o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    float u = kNegInf;
    if (t < t1) {
      float acc = 0.f;
      for (int dd = 0; dd < D; ++dd) acc = fmaf(q[dd], gK[(size_t)t * D + dd], acc);
      u = acc * c2;
    }
    const float Mn = fmaxf(M, wave_max(u));
    const float f = fast_exp2(M - Mn);
    const float p = fast_exp2(u - Mn);
    l = l * f + wave_sum(p);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= f;
    M = Mn;
    const int nt = min(64, t1 - tb);
    for (int tt = 0; tt < nt; ++tt) {
      const float pt = __shfl(p, tt);
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(pt, gV[(size_t)(lane + 64 * e) * R.Np + tb + tt], o[e]);
    }
  }
  const size_t prow = ((size_t)h * R.splits + sp) * R.rows_b + q_row;
  if (lane == 0) ((float2 *)(slot + dev.sl.part_ml[layer & 1]))[prow] = make_float2(M, l);
  float *po = (float *)(slot + dev.sl.part_o[layer & 1]) + prow * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) po[lane + 64 * e] = o[e];
}

// --------------------------------------------------------------------------------------
// 8 consecutive elements of a bf16 or f32 row: raw copy and float conversion.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4_t u;
  __device__ __forceinline__ void load(const uint16_t *p) { u = gld<u32x4_t>(p); }
  __device__ __forceinline__ void store(uint16_t *p) const { gst<u32x4_t>(p, u); }
  __device__ __forceinline__ void to_float(float *f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Raw8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = gld<f32x4_t>(p);
    b = gld<f32x4_t>(p + 4);
  }
  __device__ __forceinline__ void store(float *p) const {
    gst<f32x4_t>(p, a);
    gst<f32x4_t>(p + 4, b);
  }
  __device__ __forceinline__ void to_float(float *f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
};

// One (beam j, query head h*g+gi, 8-feature chunk c8) element of the per-layer finish:
//   step s >= 1: the new token's k/v (code c_{s-1}) are written to BeamKV slot
//   [layer][s-1][j] (by gi == 0); the beam's earlier tokens t < s-1 are read from BeamKV
//   slot anc[j][t] (BeamPath) -- never re-looked-up from the tables -- and attended to;
//   then the split-K context partials are merged in split order with that beam partial and
//   the layer output is added to h (written at layer 0).
// The D/8 lanes of one (j, head) must be consecutive and active together (their dot
// products are reduced with lane shuffles).
template <int D, typename T>
__device__ __forceinline__ void merge_elem(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int j,
                                           int gi, int kv, int c8) {
  constexpr int C8 = D / 8;
  const Dims &dm = dev.dm;
  const int s = R.level, g = dm.g, lvl = dm.levels, hq = kv * g + gi;
  const float c2 = dm.scale_log2;
  float Mb = kNegInf, lb = 0.f, ob[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ob[i] = 0.f;
  if (s > 0) {
    const int *codes = (const int *)(slot + dev.sl.codes[s & 1]);
    const int *anc = (const int *)(slot + dev.sl.anc[s & 1]);
    const int code = codes[j * lvl + (s - 1)];
    const size_t trow = ((size_t)layer * dm.tl + (s - 1)) * dm.V + code;
    float q[8];
    {
      Raw8<T> rq;
      rq.load((const T *)dev.tok_q + (trow * dm.Hq + hq) * D + c8 * 8);
      rq.to_float(q);
    }
    Raw8<T> kn, vn;
    kn.load((const T *)dev.tok_k + (trow * dm.Hkv + kv) * D + c8 * 8);
    vn.load((const T *)dev.tok_v + (trow * dm.Hkv + kv) * D + c8 * 8);
    T *bk = (T *)(slot + dev.sl.beamkv_k);
    T *bv = (T *)(slot + dev.sl.beamkv_v);
    const size_t wstride = (size_t)dm.Hkv * D;  // one BeamKV slot
    const size_t lvstride = (size_t)dm.W_max * wstride;
    const size_t base = (size_t)layer * dm.tl * lvstride + (size_t)kv * D + c8 * 8;
    if (gi == 0) {
      kn.store(bk + base + (size_t)(s - 1) * lvstride + (size_t)j * wstride);
      vn.store(bv + base + (size_t)(s - 1) * lvstride + (size_t)j * wstride);
    }
    for (int t = 0; t < s; ++t) {
      float kt[8], vt[8];
      if (t == s - 1) {
        kn.to_float(kt);
        vn.to_float(vt);
      } else {
        const size_t off = base + (size_t)t * lvstride + (size_t)anc[j * lvl + t] * wstride;
        Raw8<T> a, b;
        a.load(bk + off);
        b.load(bv + off);
        a.to_float(kt);
        b.to_float(vt);
      }
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(q[i], kt[i], dot);
#pragma unroll
      for (int o = C8 / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
      const float u = dot * c2;
      const float Mn = fmaxf(Mb, u);
      const float f = fast_exp2(Mb - Mn);
      const float p = fast_exp2(u - Mn);
      lb = lb * f + p;
#pragma unroll
      for (int i = 0; i < 8; ++i) ob[i] = fmaf(p, vt[i], ob[i] * f);
      Mb = Mn;
    }
  }
  // split partials: unnormalised o in float32, weight exp2(m - Ms)
  const float2 *pml = (const float2 *)(slot + dev.sl.part_ml[layer & 1]);
  const float *po = (const float *)(slot + dev.sl.part_o[layer & 1]);
  const int row = j * g + gi;
  const size_t pbase = (size_t)kv * R.splits * R.rows_b + row;
  float Ms = Mb;
  for (int sp = 0; sp < R.splits; ++sp) Ms = fmaxf(Ms, gld<f32x2_t>(pml + pbase + (size_t)sp * R.rows_b)[0]);
  const float fb = fast_exp2(Mb - Ms);
  float Ls = lb * fb, O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = ob[i] * fb;
  for (int sp = 0; sp < R.splits; ++sp) {
    const size_t prow = pbase + (size_t)sp * R.rows_b;
    const f32x2_t ml = gld<f32x2_t>(pml + prow);
    const float f = fast_exp2(ml[0] - Ms);
    Ls = fmaf(ml[1], f, Ls);
    const f32x4_t x = gld<f32x4_t>(po + prow * D + c8 * 8);
    const f32x4_t y = gld<f32x4_t>(po + prow * D + c8 * 8 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      O[i] = fmaf(x[i], f, O[i]);
      O[4 + i] = fmaf(y[i], f, O[4 + i]);
    }
  }
  const float inv = 1.f / Ls;
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] *= inv;
  float *hr = (float *)(slot + dev.sl.h) + ((size_t)j * dm.Hq + hq) * D + c8 * 8;
  f32x4_t a = f32x4_t{O[0], O[1], O[2], O[3]}, b = f32x4_t{O[4], O[5], O[6], O[7]};
  if (dm.debug_attn) {
    float *dg = (float *)(slot + dev.sl.dbg_attn) + (((size_t)layer * dm.W_max + j) * dm.Hq + hq) * D + c8 * 8;
    gst<f32x4_t>(dg, a);
    gst<f32x4_t>(dg + 4, b);
  }
  if (layer > 0) {
    a += gld<f32x4_t>(hr);
    b += gld<f32x4_t>(hr + 4);
  }
  gst<f32x4_t>(hr, a);
  gst<f32x4_t>(hr + 4, b);
}

// Finishes rows [r0, r1) of kv head kv for `layer` (bf16 caches); thread = (row, 8-feature
// chunk).  The arithmetic is merge_elem's, in the same order; the memory accesses are arranged
// for parallelism, E elements of a thread at a time: first every load that needs only indices
// (the beam's code, the first two splits' partials, h), then the token-table and BeamKV loads
// that need the code or the ancestry, then the arithmetic and the stores.  The finish is
// bound by these round trips, not by bandwidth: its data sits in the L2 / Infinity Cache.
template <int D, int E>
__device__ __forceinline__ void finish_rows(const Dev &dev, const StepReq &R, uint8_t *slot, int layer, int kv,
                                            int r0, int r1, int tid, int nthreads) {
  constexpr int C8 = D / 8;
  const Dims &dm = dev.dm;
  const int s = R.level, g = dm.g, lvl = dm.levels, S = R.splits;
  const float c2 = dm.scale_log2;
  const int total = (r1 - r0) * C8;
  const float2 *pml = (const float2 *)(slot + dev.sl.part_ml[layer & 1]);
  const float *po = (const float *)(slot + dev.sl.part_o[layer & 1]);  // unnormalised o, float32
  const int *codes = (const int *)(slot + dev.sl.codes[s & 1]);
  const int *anc = (const int *)(slot + dev.sl.anc[s & 1]);
  uint16_t *bk = (uint16_t *)(slot + dev.sl.beamkv_k);
  uint16_t *bv = (uint16_t *)(slot + dev.sl.beamkv_v);
  float *hb = (float *)(slot + dev.sl.h);
  const size_t wstride = (size_t)dm.Hkv * D;  // one BeamKV slot
  const size_t lvstride = (size_t)dm.W_max * wstride;
  const size_t lbase = (size_t)layer * dm.tl * lvstride + (size_t)kv * D;
  for (int e0 = tid; e0 < total; e0 += E * nthreads) {
    int j[E], gi[E], c8[E], code[E];
    bool ok[E];
    size_t pbase[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const int e = e0 + k * nthreads;
      ok[k] = e < total;  // uniform over the C8 lanes of a row
      const int row = r0 + (ok[k] ? e / C8 : 0);
      j[k] = row / g;
      gi[k] = row % g;
      c8[k] = e % C8;
      pbase[k] = (size_t)kv * S * R.rows_b + row;
    }
    // ---- phase 1: index-only loads
    f32x2_t ml0[E], ml1[E];
    f32x4_t pa0[E], pb0[E], pa1[E], pb1[E];
    f32x4_t ha[E], hc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if (!ok[k]) continue;
      code[k] = s > 0 ? codes[j[k] * lvl + (s - 1)] : 0;
      const float *p0 = po + pbase[k] * D + c8[k] * 8;
      ml0[k] = gld<f32x2_t>(pml + pbase[k]);
      pa0[k] = gld<f32x4_t>(p0);
      pb0[k] = gld<f32x4_t>(p0 + 4);
      if (S > 1) {
        ml1[k] = gld<f32x2_t>(pml + pbase[k] + R.rows_b);
        pa1[k] = gld<f32x4_t>(p0 + (size_t)R.rows_b * D);
        pb1[k] = gld<f32x4_t>(p0 + (size_t)R.rows_b * D + 4);
      }
      if (layer > 0 && !dm.chain) {
        const float *hr = hb + ((size_t)j[k] * dm.Hq + kv * g + gi[k]) * D + c8[k] * 8;
        ha[k] = gld<f32x4_t>(hr);
        hc[k] = gld<f32x4_t>(hr + 4);
      }
    }
    // ---- phase 2: the beam's own tokens (step s >= 1)
    float Mb[E], lb[E], ob[E][8];
#pragma unroll
    for (int k = 0; k < E; ++k) {
      Mb[k] = kNegInf;
      lb[k] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ob[k][i] = 0.f;
    }
    if (s > 0) {
      Raw8<uint16_t> rq[E], kn[E], vn[E];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (!ok[k]) continue;
        if (dm.chain) {
          // the layer chain: the step's q row, and the newest token's key and value already in
          // BeamKV slot [layer][s-1][j] (written by the q/k/v projection)
          const size_t own = lbase + (size_t)(s - 1) * lvstride + (size_t)j[k] * wstride + c8[k] * 8;
          rq[k].load(dev.ch.q + ((size_t)(R.row0 + j[k]) * dm.Hq + kv * g + gi[k]) * D + c8[k] * 8);
          kn[k].load(bk + own);
          vn[k].load(bv + own);
          continue;
        }
        const size_t trow = ((size_t)layer * dm.tl + (s - 1)) * dm.V + code[k];
        rq[k].load((const uint16_t *)dev.tok_q + (trow * dm.Hq + kv * g + gi[k]) * D + c8[k] * 8);
        kn[k].load((const uint16_t *)dev.tok_k + (trow * dm.Hkv + kv) * D + c8[k] * 8);
        vn[k].load((const uint16_t *)dev.tok_v + (trow * dm.Hkv + kv) * D + c8[k] * 8);
      }
      float q[E][8];
#pragma unroll
      for (int k = 0; k < E; ++k) {
        rq[k].to_float(q[k]);
        if (ok[k] && gi[k] == 0 && !dm.chain) {
          const size_t dst = lbase + (size_t)(s - 1) * lvstride + (size_t)j[k] * wstride + c8[k] * 8;
          kn[k].store(bk + dst);
          vn[k].store(bv + dst);
        }
      }
      for (int t = 0; t < s; ++t) {
        float kt[E][8], vt[E][8];
        if (t == s - 1) {
#pragma unroll
          for (int k = 0; k < E; ++k) {
            kn[k].to_float(kt[k]);
            vn[k].to_float(vt[k]);
          }
        } else {
          Raw8<uint16_t> a[E], b[E];
#pragma unroll
          for (int k = 0; k < E; ++k) {
            if (!ok[k]) continue;
            const size_t off = lbase + (size_t)t * lvstride + (size_t)anc[j[k] * lvl + t] * wstride + c8[k] * 8;
            a[k].load(bk + off);
            b[k].load(bv + off);
          }
#pragma unroll
          for (int k = 0; k < E; ++k) {
            a[k].to_float(kt[k]);
            b[k].to_float(vt[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < E; ++k) {
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) dot = fmaf(q[k][i], kt[k][i], dot);
          if constexpr (C8 == 16) {
            dot = row16_sum(dot);
          } else {
#pragma unroll
            for (int o = C8 / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
          }
          const float u = dot * c2;
          const float Mn = fmaxf(Mb[k], u);
          const float f = fast_exp2(Mb[k] - Mn);
          const float p = fast_exp2(u - Mn);
          lb[k] = lb[k] * f + p;
#pragma unroll
          for (int i = 0; i < 8; ++i) ob[k][i] = fmaf(p, vt[k][i], ob[k][i] * f);
          Mb[k] = Mn;
        }
      }
    }
    // ---- phase 3: merge the splits in order with the beam partial, h += o
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if (!ok[k]) continue;
      float Ms = fmaxf(Mb[k], ml0[k][0]);
      if (S > 1) Ms = fmaxf(Ms, ml1[k][0]);
      for (int sp = 2; sp < S; ++sp) Ms = fmaxf(Ms, gld<f32x2_t>(pml + pbase[k] + (size_t)sp * R.rows_b)[0]);
      const float fb = fast_exp2(Mb[k] - Ms);
      float Ls = lb[k] * fb, O[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] = ob[k][i] * fb;
      {
        const float f = fast_exp2(ml0[k][0] - Ms);
        Ls = fmaf(ml0[k][1], f, Ls);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[i] = fmaf(pa0[k][i], f, O[i]);
          O[4 + i] = fmaf(pb0[k][i], f, O[4 + i]);
        }
      }
      if (S > 1) {
        const float f = fast_exp2(ml1[k][0] - Ms);
        Ls = fmaf(ml1[k][1], f, Ls);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[i] = fmaf(pa1[k][i], f, O[i]);
          O[4 + i] = fmaf(pb1[k][i], f, O[4 + i]);
        }
      }
      for (int sp = 2; sp < S; ++sp) {
        const size_t prow = pbase[k] + (size_t)sp * R.rows_b;
        const f32x2_t ml = gld<f32x2_t>(pml + prow);
        const float f = fast_exp2(ml[0] - Ms);
        Ls = fmaf(ml[1], f, Ls);
        const f32x4_t x = gld<f32x4_t>(po + prow * D + c8[k] * 8);
        const f32x4_t y = gld<f32x4_t>(po + prow * D + c8[k] * 8 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[i] = fmaf(x[i], f, O[i]);
          O[4 + i] = fmaf(y[i], f, O[4 + i]);
        }
      }
      const float inv = 1.f / Ls;
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] *= inv;
      const int hq = kv * g + gi[k];
      float *hr = hb + ((size_t)j[k] * dm.Hq + hq) * D + c8[k] * 8;
      f32x4_t a = f32x4_t{O[0], O[1], O[2], O[3]}, b = f32x4_t{O[4], O[5], O[6], O[7]};
      if (dm.debug_attn) {
        float *dg = (float *)(slot + dev.sl.dbg_attn) + (((size_t)layer * dm.W_max + j[k]) * dm.Hq + hq) * D + c8[k] * 8;
        gst<f32x4_t>(dg, a);
        gst<f32x4_t>(dg + 4, b);
      }
      if (dm.chain) {
        // the attention output, rounded to bf16, is the output projection's input row
        gst<u32x4_t>(dev.ch.o + ((size_t)(R.row0 + j[k]) * dm.Hq + hq) * D + c8[k] * 8,
                     u32x4_t{pack_bf16(O[0], O[1]), pack_bf16(O[2], O[3]), pack_bf16(O[4], O[5]),
                             pack_bf16(O[6], O[7])});
        continue;
      }
      if (layer > 0) {
        a += ha[k];
        b += hc[k];
      }
      gst<f32x4_t>(hr, a);
      gst<f32x4_t>(hr + 4, b);
    }
  }
}

// Separate finish kernel: the float32 path after every layer, the bf16 path after the last
// layer.  One workgroup per (request, beam j); thread = (query head, 8-feature chunk).
// thread = (query head, 8-feature chunk).
template <int D, typename T>
__global__ __launch_bounds__(256) void k_beam_merge(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                    int layer, int wg0) {
  constexpr int C8 = D / 8;
  const int bid = (int)blockIdx.x + wg0;  // reqs may start past the step's first request
  const int ri = find_req<1>(reqs, n_reqs, bid);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int j = bid - R.wg_merge;
  uint8_t *slot = slot_base(dev, R.slot);
  const int n_live = ((const int *)(slot + dev.sl.n_live))[R.level & 1];
  if (j >= n_live) return;
  const int nchunk = dm.Hq * C8;  // a multiple of C8: a head's lanes are all active or all idle
  for (int e = threadIdx.x; e < nchunk; e += 256) {
    const int hq = e / C8;
    merge_elem<D, T>(dev, R, slot, layer, j, hq % dm.g, hq / dm.g, e % C8);
  }
}

// Finish of one layer of a split-K step of a bf16 model as a launch of its own (the merge that
// otherwise runs in the next layer's prologue): workgroup (request, 16- or 32-row block, kv
// head), finish_rows with one element per thread (BeamKV append, the beam's own tokens, the
// split merge in split order, h += o).  Its time is the round trips of its dependent loads;
// many small workgroups keep more of them in flight (one element per thread: 13.6 us per
// layer of the 256-beam headline, two: 16.0).
template <int D>
__global__ __launch_bounds__(256) void k_finish_layer(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                      int layer, int wg0) {
  constexpr int RPW = 256 / (D / 8);  // rows per workgroup
  const int bid = (int)blockIdx.x + wg0;
  const StepReq R = reqs[find_req<4>(reqs, n_reqs, bid)];
  const Dims &dm = dev.dm;
  const int local = bid - R.wg_fin;
  const int kv = local % dm.Hkv, r0 = (local / dm.Hkv) * RPW;
  uint8_t *slot = slot_base(dev, R.slot);
  const int rows = ((const int *)(slot + dev.sl.n_live))[R.level & 1] * dm.g;
  if (r0 >= rows) return;
  finish_rows<D, 1>(dev, R, slot, layer, kv, r0, min(rows, r0 + RPW), (int)threadIdx.x, 256);
}

// Finish of a first-level step whose layers ran in one launch (k_ctx_attn_stream<.., true>).
// The first level has one live beam and no beam tokens, so a layer's output is the merge of
// its split partials.  k_finish_first_level: workgroup (request, layer), thread = (query
// head, 8-feature chunk); the layer's output goes to the scratch rows [layer][Hq*d] of
// partial buffer 1 (unused by the fused launch).  k_sum_layers then forms h = sum over layers
// in layer order, the additions of the per-layer finish.
template <int D>
__global__ __launch_bounds__(256) void k_finish_first_level(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  constexpr int C8 = D / 8;
  const StepReq R = reqs[blockIdx.x];
  const int layer = blockIdx.y;
  const Dims &dm = dev.dm;
  uint8_t *slot = slot_base(dev, R.slot);
  const float2 *pml = (const float2 *)(slot + dev.sl.part_ml[0]);
  const float *po = (const float *)(slot + dev.sl.part_o[0]);  // unnormalised o, float32
  float *tmp = (float *)(slot + dev.sl.part_o[1]);
  const size_t lofs = (size_t)layer * dm.Hkv * R.splits * R.rows_b;
  for (int e = threadIdx.x; e < dm.Hq * C8; e += blockDim.x) {
    const int hq = e / C8, c8 = e % C8, kv = hq / dm.g, row = hq % dm.g;  // beam 0: row = gi
    const size_t pbase = lofs + (size_t)kv * R.splits * R.rows_b + row;
    float Ms = kNegInf;
    for (int sp = 0; sp < R.splits; ++sp) Ms = fmaxf(Ms, gld<f32x2_t>(pml + pbase + (size_t)sp * R.rows_b)[0]);
    float Ls = 0.f, O[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) O[i] = 0.f;
    for (int sp = 0; sp < R.splits; ++sp) {
      const size_t prow = pbase + (size_t)sp * R.rows_b;
      const f32x2_t ml = gld<f32x2_t>(pml + prow);
      const float f = fast_exp2(ml[0] - Ms);
      Ls = fmaf(ml[1], f, Ls);
      const f32x4_t x = gld<f32x4_t>(po + prow * D + c8 * 8);
      const f32x4_t y = gld<f32x4_t>(po + prow * D + c8 * 8 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        O[i] = fmaf(x[i], f, O[i]);
        O[4 + i] = fmaf(y[i], f, O[4 + i]);
      }
    }
    const float inv = 1.f / Ls;
    const f32x4_t a = f32x4_t{O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv};
    const f32x4_t b = f32x4_t{O[4] * inv, O[5] * inv, O[6] * inv, O[7] * inv};
    float *t = tmp + ((size_t)layer * dm.Hq + hq) * D + c8 * 8;
    gst<f32x4_t>(t, a);
    gst<f32x4_t>(t + 4, b);
    if (dm.debug_attn) {
      float *dg = (float *)(slot + dev.sl.dbg_attn) + ((size_t)layer * dm.W_max * dm.Hq + hq) * D + c8 * 8;
      gst<f32x4_t>(dg, a);
      gst<f32x4_t>(dg + 4, b);
    }
  }
}

__global__ __launch_bounds__(256) void k_sum_layers(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  const StepReq R = reqs[blockIdx.x];
  const Dims &dm = dev.dm;
  uint8_t *slot = slot_base(dev, R.slot);
  const float *tmp = (const float *)(slot + dev.sl.part_o[1]);
  float *hb = (float *)(slot + dev.sl.h);
  const int n = dm.Hq * dm.d;
  for (int e = blockIdx.y * blockDim.x + threadIdx.x; e < n; e += gridDim.y * blockDim.x) {
    float acc = tmp[e];
    for (int l = 1; l < dm.L; ++l) acc = tmp[(size_t)l * n + e] + acc;
    hb[e] = acc;
  }
}

// h of every live beam after a full-context step: the sum over layers, in layer order, of the
// rows' stored float32 o/l.  One thread per 8 features of a (beam, query head) row.
__global__ __launch_bounds__(256) void k_sum_hparts(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  const StepReq R = reqs[blockIdx.y];
  if (R.lgroups < 1) return;
  const Dims &dm = dev.dm;
  uint8_t *slot = slot_base(dev, R.slot);
  const int n_live = ((const int *)(slot + dev.sl.n_live))[R.level & 1];
  const int per_row = dm.d / 8;
  const size_t n8 = (size_t)n_live * dm.Hq * per_row;
  const size_t lrows = (size_t)dm.W_max * dm.Hq;  // rows per layer
  const f32x4_t *hp = (const f32x4_t *)(slot + dev.sl.hl);
  f32x4_t *hb = (f32x4_t *)(slot + dev.sl.h);
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += (size_t)gridDim.x * blockDim.x) {
    f32x4_t a0 = gld<f32x4_t>(hp + 2 * e), a1 = gld<f32x4_t>(hp + 2 * e + 1);
#pragma unroll 4
    for (int l = 1; l < dm.L; ++l) {
      a0 += gld<f32x4_t>(hp + 2 * ((size_t)l * lrows * per_row + e));
      a1 += gld<f32x4_t>(hp + 2 * ((size_t)l * lrows * per_row + e) + 1);
    }
    gst<f32x4_t>(hb + 2 * e, a0);
    gst<f32x4_t>(hb + 2 * e + 1, a1);
  }
}

// Label head ([TRT] "Background" and "Scoring many candidates at once": given candidates are
// ranked by the log-probabilities of label tokens read after each candidate).  After a label
// step (s = levels: each candidate's last code run as a token), beam j of request i has the
// hidden vector h_j; z_c = h_j . w_label[:, c] in float32 and label_out[i][j][c] = z_c -
// logsumexp(z).  One workgroup per (request, beam), workgroups numbered as the merge launch's.
constexpr int kMaxLabels = 16;
__global__ __launch_bounds__(256) void k_label_head(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  const int ri = find_req<1>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int j = (int)blockIdx.x - R.wg_merge;
  uint8_t *slot = slot_base(dev, R.slot);
  const int n_live = ((const int *)(slot + dev.sl.n_live))[R.level & 1];
  if (j >= n_live) return;
  const int D = dm.Hq * dm.d, nl = dm.n_labels;
  const float *h = (const float *)(slot + dev.sl.h) + (size_t)j * D;
  float acc[kMaxLabels];
#pragma unroll
  for (int c = 0; c < kMaxLabels; ++c) acc[c] = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) {
    const float hv = h[i];
    const float *w = dev.w_label + (size_t)i * nl;
#pragma unroll
    for (int c = 0; c < kMaxLabels; ++c)
      if (c < nl) acc[c] = fmaf(hv, w[c], acc[c]);
  }
  __shared__ float red[kMaxLabels][4];
#pragma unroll
  for (int c = 0; c < kMaxLabels; ++c) {
    if (c >= nl) break;
    const float v = wave_sum(acc[c]);
    if ((threadIdx.x & 63) == 0) red[c][threadIdx.x >> 6] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float z[kMaxLabels], m = kNegInf;
    for (int c = 0; c < nl; ++c) {
      z[c] = (red[c][0] + red[c][1]) + (red[c][2] + red[c][3]);
      m = fmaxf(m, z[c]);
    }
    float se = 0.f;
    for (int c = 0; c < nl; ++c) se += expf(z[c] - m);
    const float lse = m + logf(se);
    float *out = dev.label_out + ((size_t)ri * dm.W_max + j) * nl;
    for (int c = 0; c < nl; ++c) out[c] = z[c] - lse;
  }
}


// --------------------------------------------------------------------------------------
// logits_part[ks][j][c] = sum over the ks-th quarter of the hidden dim of h[j][k] w_sid[level][k][c]
// fp32 MFMA 32x32x2 (exact fp32 products, fp32 accumulate).  Workgroup: 64 beams x 64 codes
// of one hidden-dim slice; wave w owns the 32x32 block (w/2, w%2).  Tiles of 32 hidden
// features are double-buffered through LDS.
__global__ __launch_bounds__(256) void k_logits(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ri = find_req<2>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int V = dm.V, H = dm.Hq * dm.d, KSL = H / kLogitsKS;
  const int nct = (V + 63) / 64;
  int local = blockIdx.x - R.wg_logits;
  const int ks = local % kLogitsKS;
  local /= kLogitsKS;
  const int ct = local % nct, rt = local / nct;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int row0 = rt * 64;
  if (row0 >= n_live) return;
  const float *hb = (const float *)(slot + dev.sl.h);
  const float *Wt = dev.w_sid + (size_t)s * H * V;
  const int k0 = ks * KSL;
  __shared__ float sA[2][64][33];
  __shared__ float sB[2][32][65];
  float ra[8], rbv[8];
  const int ar = tid >> 2, ak = (tid & 3) * 8;   // A tile: 64 rows x 32 features
  const int br = tid >> 3, bc = (tid & 7) * 8;   // B tile: 32 features x 64 codes
  auto gl = [&](int kc) {
    if (row0 + ar < n_live) {
      const f32x4_t a = gld<f32x4_t>(hb + (size_t)(row0 + ar) * H + k0 + kc + ak);
      const f32x4_t b = gld<f32x4_t>(hb + (size_t)(row0 + ar) * H + k0 + kc + ak + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = a[i];
        ra[4 + i] = b[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int col = ct * 64 + bc + i;
      rbv[i] = col < V ? gld<float>(Wt + (size_t)(k0 + kc + br) * V + col) : 0.f;
    }
  };
  auto ls = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sA[buf][ar][ak + i] = ra[i];
      sB[buf][br][bc + i] = rbv[i];
    }
  };
  const int rbk = w >> 1, cbk = w & 1;
  f32x16_t acc = f32x16_t{};
  gl(0);
  ls(0);
  __syncthreads();
  for (int kc = 0, it = 0; kc < KSL; kc += 32, ++it) {
    const int buf = it & 1;
    if (kc + 32 < KSL) gl(kc + 32);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float a = sA[buf][rbk * 32 + (lane & 31)][kk * 2 + (lane >> 5)];
      const float b = sB[buf][kk * 2 + (lane >> 5)][cbk * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    if (kc + 32 < KSL) ls(buf ^ 1);
    __syncthreads();
  }
  float *out = (float *)(slot + dev.sl.logits_part) + (size_t)ks * dm.W_max * V;
  const int col = ct * 64 + cbk * 32 + (lane & 31);
  if (col < V) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = row0 + rbk * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (row < n_live) gst<float>(out + (size_t)row * V + col, acc[i]);
    }
  }
}

// --------------------------------------------------------------------------------------
// Top-K selection over a candidate array.  Keys are unique 64-bit integers
//   key = order-preserving bits of the score << 32 | (0xFFFFFFFF - flat index)
// so "larger key" = higher score, then lower flat index; -0 is folded to +0 first.
__device__ __forceinline__ uint32_t f2ord(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t cand_key(float v, uint32_t i) {
  const float vc = (v == 0.f) ? 0.f : v;
  return ((uint64_t)f2ord(vc) << 32) | (uint64_t)(0xFFFFFFFFu - i);
}

constexpr int kBins = 2048;

struct SelectSmem {
  uint64_t sel[kMaxBeam];
  uint64_t tie[kTieCap];
  int hist[kBins];
  int wsum[kTopkThreads / 64];
  int wcnt[kTopkThreads / 64];
  float wmin[kTopkThreads / 64], wmax[kTopkThreads / 64];
  uint64_t prefix;
  int need, cut, cnt, tcnt, nvalid;
  float vmin, vmax;
};

__device__ void select_stream(const float *__restrict__ cand, int n_total, uint32_t ibase, int k, SelectSmem &sm);

// Sorts a[0..n) descending (n <= 1024); every thread of the workgroup calls it.
static_assert(kMaxBeam <= kTopkThreads && kTieCap <= kTopkThreads, "one key per thread");
__device__ void block_sort_desc(uint64_t *a, int n) {
  // n <= kTopkThreads distinct keys (each holds its candidate's flat index): a key's place in
  // descending order is the number of keys above it, so the places form a permutation.  With
  // n <= kTopkThreads / 4 four adjacent lanes count a key's rank over a quarter of the keys
  // each; the reads a[j] are LDS broadcasts.  Two barriers in all.
  const int tid = threadIdx.x;
  uint64_t key = 0;
  int rank = 0;
  if (n <= kTopkThreads / 4) {
    const int me = tid >> 2, q = tid & 3;
    if (me < n) {
      key = a[me];
      const int j0 = q * ((n + 3) >> 2), j1 = min(n, j0 + ((n + 3) >> 2));
      for (int j = j0; j < j1; ++j) rank += (int)(a[j] > key);
    }
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    __syncthreads();
    if (me < n && q == 0) a[rank] = key;
  } else {
    if (tid < n) {
      key = a[tid];
      int j = 0;
      for (; j + 4 <= n; j += 4)
        rank += (int)(a[j] > key) + (int)(a[j + 1] > key) + (int)(a[j + 2] > key) + (int)(a[j + 3] > key);
      for (; j < n; ++j) rank += (int)(a[j] > key);
    }
    __syncthreads();
    if (tid < n) a[rank] = key;
  }
  __syncthreads();
}

// Block reduction of the per-thread statistics of the finite (> -inf) candidates into
// sm.nvalid / vmin / vmax.
__device__ void reduce_stats(int cnt, float mn, float mx, SelectSmem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o);
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    sm.wcnt[w] = cnt;
    sm.wmin[w] = mn;
    sm.wmax[w] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    float a = __builtin_inff(), b = kNegInf;
    for (int i = 0; i < kTopkThreads / 64; ++i) {
      c += sm.wcnt[i];
      a = fminf(a, sm.wmin[i]);
      b = fmaxf(b, sm.wmax[i]);
    }
    sm.nvalid = c;
    sm.vmin = a;
    sm.vmax = b;
  }
  __syncthreads();
}

// Streaming statistics of cand[0..total): eight loads in flight per thread at a time.
__device__ void scan_cands(const float *__restrict__ cand, int total, SelectSmem &sm) {
  const int tid = threadIdx.x;
  int cnt = 0;
  float mn = __builtin_inff(), mx = kNegInf;
  for (int base = 0; base < total; base += 8 * kTopkThreads) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + tid + u * kTopkThreads;
      x[u] = i < total ? gld<float>(cand + i) : kNegInf;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (x[u] > kNegInf) {
        ++cnt;
        mn = fminf(mn, x[u]);
        mx = fmaxf(mx, x[u]);
      }
  }
  reduce_stats(cnt, mn, mx, sm);
}

// Flat index of a thread's m-th register candidate: four consecutive candidates per 16-byte
// load, 4096 apart between loads.
__device__ __forceinline__ int reg_cand(int m) { return 4 * (int)threadIdx.x + 4 * kTopkThreads * (m >> 2) + (m & 3); }

// cand[0..total) into the registers v[m] (flat index reg_cand(m)), -inf past the end: every
// load is issued before the first is used (one round trip, not CPT/4), then their statistics.
// total is a multiple of 4 (rows x codebook with 4 | codebook) or the loads of the last
// group go element by element.
template <int CPT>
__device__ void load_cands(const float *__restrict__ cand, int total, float (&v)[CPT], SelectSmem &sm) {
  static_assert(CPT % 4 == 0, "four candidates per load");
#pragma unroll
  for (int m4 = 0; m4 < CPT / 4; ++m4) {
    const int i = reg_cand(4 * m4);
    if (i + 4 <= total) {
      const f32x4_t x = gld<f32x4_t>(cand + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * m4 + e] = x[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * m4 + e] = i + e < total ? gld<float>(cand + i + e) : kNegInf;
    }
  }
  int cnt = 0;
  float mn = __builtin_inff(), mx = kNegInf;
#pragma unroll
  for (int m = 0; m < CPT; ++m)
    if (v[m] > kNegInf) {
      ++cnt;
      mn = fminf(mn, v[m]);
      mx = fmaxf(mx, v[m]);
    }
  reduce_stats(cnt, mn, mx, sm);
}

// Top-k of the candidates a thread holds in v[m] (flat index idx(m); -inf = none) with their
// statistics in sm (1 <= k <= nvalid).  A monotone linear map of the score to 2048 bins;
// the histogram picks the bin holding the k-th best, everything above it is selected, and the
// candidates of that bin are ordered exactly by their 64-bit keys.  When the cut bin holds
// more than kTieCap candidates the exact streaming radix select runs instead, over the same
// candidates in memory: cand[0..total), flat index ibase + i.  Leaves the k best keys in
// sm.sel[0..k), sorted descending when `sorted` (the streaming select always sorts).
template <int CPT, typename IDX>
__device__ void select_bins(const float *__restrict__ cand, int total, uint32_t ibase, const float (&v)[CPT], IDX idx,
                            int k, bool sorted, SelectSmem &sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float vmin = sm.vmin, span = sm.vmax - sm.vmin;
  float scale = (float)(kBins - 1) / span;
  if (!(scale > 0.f) || !(scale < 3.0e38f)) scale = 0.f;
  auto bin = [&](float x) { return min(kBins - 1, (int)((x - vmin) * scale)); };
  for (int b = tid; b < kBins; b += kTopkThreads) sm.hist[b] = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < CPT; ++m)
    if (v[m] > kNegInf) atomicAdd(&sm.hist[bin(v[m])], 1);
  __syncthreads();
  // suffix sums: thread t owns bins 2t and 2t+1
  const int h0 = sm.hist[2 * tid], h1 = sm.hist[2 * tid + 1];
  const int loc = h0 + h1;
  int suf = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(suf, o);
    if (lane + o < 64) suf += y;
  }
  if (lane == 0) sm.wsum[w] = suf;
  __syncthreads();
  int above = suf - loc;
  for (int ww = w + 1; ww < kTopkThreads / 64; ++ww) above += sm.wsum[ww];
  if (above < k && k <= above + h1) {
    sm.cut = 2 * tid + 1;
    sm.need = k - above;
  } else if (above + h1 < k && k <= above + h1 + h0) {
    sm.cut = 2 * tid;
    sm.need = k - above - h1;
  }
  if (tid == 0) {
    sm.cnt = 0;
    sm.tcnt = 0;
  }
  __syncthreads();
  const int cut = sm.cut, need = sm.need, cutcnt = sm.hist[cut];
  __syncthreads();  // every thread has read hist[cut] before anything reuses hist
  if (cutcnt > kTieCap) {  // uniform branch
    select_stream(cand, total, ibase, k, sm);
    return;
  }
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    if (!(v[m] > kNegInf)) continue;
    const int b = bin(v[m]);
    if (b >= cut) {
      const uint64_t key = cand_key(v[m], (uint32_t)idx(m));
      if (b > cut)
        sm.sel[atomicAdd(&sm.cnt, 1)] = key;
      else
        sm.tie[atomicAdd(&sm.tcnt, 1)] = key;
    }
  }
  __syncthreads();
  const int ntie = sm.tcnt, base = sm.cnt;  // base == k - need
  if (ntie > 1) block_sort_desc(sm.tie, ntie);
  for (int i = tid; i < need; i += kTopkThreads) sm.sel[base + i] = sm.tie[i];
  __syncthreads();
  if (sorted) block_sort_desc(sm.sel, k);
}

// Streaming variant for candidate arrays larger than the registers hold: exact radix
// select reading the array from memory each pass (flat index ibase + i).  Leaves the k largest
// keys sorted.
__device__ void select_stream(const float *__restrict__ cand, int n_total, uint32_t ibase, int k, SelectSmem &sm) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int need = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int b = tid; b < 256; b += kTopkThreads) sm.hist[b] = 0;
    __syncthreads();
    for (int base = 0; base < n_total; base += 8 * kTopkThreads) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + tid + u * kTopkThreads;
        x[u] = i < n_total ? gld<float>(cand + i) : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!(x[u] > kNegInf)) continue;
        const uint64_t key = cand_key(x[u], ibase + (uint32_t)(base + tid + u * kTopkThreads));
        if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255], 1);
      }
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0;
      for (int b = 255; b >= 0; --b) {
        const int hb = sm.hist[b];
        if (cum + hb >= need) {
          sm.prefix = (prefix << 8) | (uint64_t)b;
          sm.need = need - cum;
          break;
        }
        cum += hb;
      }
    }
    __syncthreads();
    prefix = sm.prefix;
    need = sm.need;
    __syncthreads();
  }
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  for (int base = 0; base < n_total; base += 8 * kTopkThreads) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + tid + u * kTopkThreads;
      x[u] = i < n_total ? gld<float>(cand + i) : kNegInf;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!(x[u] > kNegInf)) continue;
      const uint64_t key = cand_key(x[u], ibase + (uint32_t)(base + tid + u * kTopkThreads));
      if (key >= prefix) sm.sel[atomicAdd(&sm.cnt, 1)] = key;
    }
  }
  __syncthreads();
  block_sort_desc(sm.sel, k);
}

// --------------------------------------------------------------------------------------
// The same logit partials for bf16 models, on the bf16 matrix cores: each fp32 operand is
// split into bf16 terms x = hi + lo + r (hi and lo rounded to nearest, |r| <= 2^-16 |x|) and
// the product taken as hi*hi + hi*lo + lo*hi with fp32 accumulation (the dropped lo*lo and
// the residuals leave at most 3 * 2^-16 relative error per product, typically 2e-5 on a
// 2048-term logit of rms 1, far below the decode's 1e-3 log-prob bound).  Tiles as in k_logits; chunks of 32 hidden
// features are staged through LDS already split, A as [row][k] and B transposed to [col][k],
// so every MFMA operand is one 16-byte read.
__global__ __launch_bounds__(256) void k_logits_x3(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  constexpr int KC = 32, LS = KC + 8;  // chunk of hidden features, LDS row stride (elements)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ri = find_req<2>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int V = dm.V, H = dm.Hq * dm.d, KSL = H / kLogitsKS;
  const int nct = (V + 63) / 64;
  int local = blockIdx.x - R.wg_logits;
  const int ks = local % kLogitsKS;
  local /= kLogitsKS;
  const int ct = local % nct, rt = local / nct;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int row0 = rt * 64;
  if (row0 >= n_live) return;
  const float *hb = (const float *)(slot + dev.sl.h);
  const float *Wt = dev.w_sid + (size_t)s * H * V;
  const int k0 = ks * KSL;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][2][64 * LS];  // [buf][hi, lo][row][k]
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][2][64 * LS];  // [buf][hi, lo][col][k]
  // staging: A row ar, features ak..ak+8; B column bc, features bk..bk+8
  const int ar = tid >> 2, ak = (tid & 3) * 8;
  const int bc = tid & 63, bk = w * 8;
  const bool a_ok = row0 + ar < n_live, b_ok = ct * 64 + bc < V;
  f32x4_t ra[2];
  float rb[8];
  auto gl = [&](int kc) {
    const float *ap = hb + (size_t)(row0 + (a_ok ? ar : 0)) * H + k0 + kc + ak;
    ra[0] = a_ok ? gld<f32x4_t>(ap) : f32x4_t{};
    ra[1] = a_ok ? gld<f32x4_t>(ap + 4) : f32x4_t{};
    const float *bp = Wt + (size_t)(k0 + kc + bk) * V + ct * 64 + (b_ok ? bc : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[i] = b_ok ? gld<float>(bp + (size_t)i * V) : 0.f;
  };
  // x -> (hi, lo) bf16, eight at a time, as two 16-byte words
  auto split8 = [](const float (&x)[8], u32x4_t &hi, u32x4_t &lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t v = {x[2 * i], x[2 * i + 1]};
      const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
      const f32x2_t hf = __builtin_convertvector(h, f32x2_t);
      const bf16x2_t l = __builtin_convertvector(v - hf, bf16x2_t);
      hi[i] = __builtin_bit_cast(uint32_t, h);
      lo[i] = __builtin_bit_cast(uint32_t, l);
    }
  };
  auto ls = [&](int buf) {
    float a8[8] = {ra[0][0], ra[0][1], ra[0][2], ra[0][3], ra[1][0], ra[1][1], ra[1][2], ra[1][3]};
    u32x4_t h, l;
    split8(a8, h, l);
    *(u32x4_t *)&sA[buf][0][ar * LS + ak] = h;
    *(u32x4_t *)&sA[buf][1][ar * LS + ak] = l;
    split8(rb, h, l);
    *(u32x4_t *)&sB[buf][0][bc * LS + bk] = h;
    *(u32x4_t *)&sB[buf][1][bc * LS + bk] = l;
  };
  const int rbk = w >> 1, cbk = w & 1;
  const int ao = (rbk * 32 + (lane & 31)) * LS + 8 * (lane >> 5);
  const int bo = (cbk * 32 + (lane & 31)) * LS + 8 * (lane >> 5);
  f32x16_t acc = f32x16_t{};
  gl(0);
  ls(0);
  __syncthreads();
  for (int kc = 0, it = 0; kc < KSL; kc += KC, ++it) {
    const int buf = it & 1;
    if (kc + KC < KSL) gl(kc + KC);
#pragma unroll
    for (int kb = 0; kb < KC / 16; ++kb) {
      const bf16x8_t ah = *(const bf16x8_t *)&sA[buf][0][ao + 16 * kb];
      const bf16x8_t al = *(const bf16x8_t *)&sA[buf][1][ao + 16 * kb];
      const bf16x8_t bh = *(const bf16x8_t *)&sB[buf][0][bo + 16 * kb];
      const bf16x8_t bl = *(const bf16x8_t *)&sB[buf][1][bo + 16 * kb];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
    }
    if (kc + KC < KSL) ls(buf ^ 1);
    __syncthreads();
  }
  float *out = (float *)(slot + dev.sl.logits_part) + (size_t)ks * dm.W_max * V;
  const int col = ct * 64 + cbk * 32 + (lane & 31);
  if (col < V) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = row0 + rbk * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (row < n_live) gst<float>(out + (size_t)row * V + col, acc[i]);
    }
  }
}

// --------------------------------------------------------------------------------------
// Per beam row (one wave, kLsmRows rows per workgroup): logits = sum of the split partials
// (fixed order), trie mask of the beam's node, log-softmax over the valid codes (or the whole
// codebook), candidates cand[j][c] = score_j + logit - lse (valid) or -inf.  For a request
// whose top-K runs in two stages (StepReq::sel2) the workgroup then keeps the W largest
// candidate keys of its rows (a chunk) in lkeys[chunk][0..lcnt[chunk]): keys are unique, so
// the request's W largest are among the union of its chunks' W largest, and k_select selects
// over those.
__global__ __launch_bounds__(kTopkThreads) void k_lsm(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  constexpr int MAXC = 1024 / 64;
  static_assert(kLsmRows * 64 == kTopkThreads, "one wave per row");
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ri = find_req<3>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int chunk = blockIdx.x - R.wg_lsm, row0 = chunk * kLsmRows, j = row0 + w;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level, cur = s & 1, V = dm.V;
  const int n = ((const int *)(slot + dev.sl.n_live))[cur];
  if (row0 >= n) return;  // the whole chunk past the live beams
  float *cand = (float *)(slot + dev.sl.cand);
  float cv[MAXC];  // this lane's candidates (codes lane + 64 e); -inf: invalid, or no row
#pragma unroll
  for (int e = 0; e < MAXC; ++e) cv[e] = kNegInf;
  if (j < n) {
    const uint32_t *mrow = dev.trie_mask + (dev.trie_off[s] + ((const int *)(slot + dev.sl.node[cur]))[j]) * dm.MW;
    const float sc = ((const float *)(slot + dev.sl.score[cur]))[j];
    const float *part = (const float *)(slot + dev.sl.logits_part);
    const size_t pstride = (size_t)dm.W_max * V;
    float *logits = (float *)(slot + dev.sl.logits);
    float xs[MAXC];
    uint32_t vbits = 0;
    float mx = kNegInf;
#pragma unroll
    for (int e = 0; e < MAXC; ++e) {
      const int c = lane + 64 * e;
      xs[e] = 0.f;
      if (c < V) {
        float x = 0.f;
#pragma unroll
        for (int ks = 0; ks < kLogitsKS; ++ks) x += gld<float>(part + ks * pstride + (size_t)j * V + c);
        xs[e] = x;
        gst<float>(logits + (size_t)j * V + c, x);
        const bool valid = (mrow[c >> 5] >> (c & 31)) & 1u;
        vbits |= (uint32_t)valid << e;
        if (dm.norm == 1 || valid) mx = fmaxf(mx, x);
      }
    }
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < MAXC; ++e) {
      const int c = lane + 64 * e;
      if (c < V && (dm.norm == 1 || ((vbits >> e) & 1u))) sum += expf(xs[e] - mx);
    }
    sum = wave_sum(sum);
    const float lse = mx + logf(sum);
#pragma unroll
    for (int e = 0; e < MAXC; ++e) {
      const int c = lane + 64 * e;
      if (c < V) {
        cv[e] = ((vbits >> e) & 1u) ? sc + (xs[e] - lse) : kNegInf;
        gst<float>(cand + (size_t)j * V + c, cv[e]);
      }
    }
  }
  if (!R.sel2) return;  // uniform over the workgroup
  int cnt = 0;
  float mn = __builtin_inff(), mxv = kNegInf;
#pragma unroll
  for (int e = 0; e < MAXC; ++e)
    if (cv[e] > kNegInf) {
      ++cnt;
      mn = fminf(mn, cv[e]);
      mxv = fmaxf(mxv, cv[e]);
    }
  reduce_stats(cnt, mn, mxv, sm);  // its barriers also publish the chunk's cand stores
  const int k = min(R.W, sm.nvalid);
  if (k > 0) {
    const int rows = min(kLsmRows, n - row0);
    select_bins<MAXC>(cand + (size_t)row0 * V, rows * V, (uint32_t)(row0 * V), cv,
                      [&](int e) { return j * V + lane + 64 * e; }, k, false, sm);
    uint64_t *lk = (uint64_t *)(slot + dev.sl.lkeys) + (size_t)chunk * R.W;
    for (int i = tid; i < k; i += kTopkThreads) lk[i] = sm.sel[i];
  }
  if (tid == 0) ((int *)(slot + dev.sl.lcnt))[chunk] = k;
}

// Scoring step: candidate i (of the n_items given) takes its own code at level s instead of a
// top-K choice.  At level 0 every candidate extends the root beam; later, beam i is candidate
// i's prefix.  Its score is the candidate array's entry (previous score + log-prob, -inf when
// the code is not a valid child of the prefix); an invalid prefix keeps -inf and continues
// from the first trie node of the next level, so every index stays in range.
__device__ void force_codes(const Dev &dev, const StepReq &R, uint8_t *slot) {
  const Dims &dm = dev.dm;
  const int s = R.level, V = dm.V, lvl = dm.levels, MW = dm.MW, n = R.n_items;
  const int cur = s & 1, nxt = cur ^ 1;
  const float *cand = (const float *)(slot + dev.sl.cand);
  const int *items = (const int *)(slot + dev.sl.items);
  const int *node_cur = (const int *)(slot + dev.sl.node[cur]);
  const int *codes_cur = (const int *)(slot + dev.sl.codes[cur]);
  const int *anc_cur = (const int *)(slot + dev.sl.anc[cur]);
  int *codes_nxt = (int *)(slot + dev.sl.codes[nxt]);
  int *anc_nxt = (int *)(slot + dev.sl.anc[nxt]);
  float *score_nxt = (float *)(slot + dev.sl.score[nxt]);
  int *node_nxt = (int *)(slot + dev.sl.node[nxt]);
  int *parent_nxt = (int *)(slot + dev.sl.parent[nxt]);
  const uint32_t *mask = dev.trie_mask + dev.trie_off[s] * MW;
  const int32_t *child = dev.trie_child + dev.trie_off[s];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int j = s == 0 ? 0 : i;  // parent beam
    const int c = items[i * lvl + s];
    for (int t = 0; t < s; ++t) {
      codes_nxt[i * lvl + t] = codes_cur[j * lvl + t];
      anc_nxt[i * lvl + t] = anc_cur[j * lvl + t];
    }
    codes_nxt[i * lvl + s] = c;
    anc_nxt[i * lvl + s] = i;
    parent_nxt[i] = j;
    const int nj = node_cur[j];
    const uint32_t *mrow = mask + (size_t)nj * MW;
    const bool valid = (mrow[c >> 5] >> (c & 31)) & 1u;
    score_nxt[i] = valid ? cand[(size_t)j * V + c] : kNegInf;
    int below = 0;
    for (int wd = 0; wd < (c >> 5); ++wd) below += __popc(mrow[wd]);
    below += __popc(mrow[c >> 5] & ((1u << (c & 31)) - 1u));
    node_nxt[i] = valid ? child[nj] + below : 0;
  }
  if (threadIdx.x == 0) ((int *)(slot + dev.sl.n_live))[nxt] = n;
}

// Top-K over beams x codes + BeamPath update (or the forced codes of a scoring request).  One
// workgroup per request.
template <bool REGS>
__global__ __launch_bounds__(kTopkThreads) void k_select(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x;
  const StepReq R = reqs[blockIdx.x];
  const Dims &dm = dev.dm;
  uint8_t *slot = slot_base(dev, R.slot);
  if (R.n_items > 0) {
    force_codes(dev, R, slot);
    return;
  }
  const int s = R.level, V = dm.V, lvl = dm.levels, MW = dm.MW;
  const int cur = s & 1, nxt = cur ^ 1;
  const int n = ((const int *)(slot + dev.sl.n_live))[cur];
  const float *cand = (const float *)(slot + dev.sl.cand);
  int k;
  if (R.sel2) {
    // second stage: the chunks' kept keys (chunk g's at lkeys[g * W], lcnt[g] of them); the
    // streaming fallback runs over the whole candidate array
    const int G = (n + kLsmRows - 1) / kLsmRows, P = G * R.W;
    const uint64_t *lk = (const uint64_t *)(slot + dev.sl.lkeys);
    const int *lc = (const int *)(slot + dev.sl.lcnt);
    float v[kSel2CPT];
    uint32_t ix[kSel2CPT];
    int cnt = 0;
    float mn = __builtin_inff(), mx = kNegInf;
#pragma unroll
    for (int m = 0; m < kSel2CPT; ++m) {
      const int p = tid + kTopkThreads * m, g = p / R.W;
      v[m] = kNegInf;
      ix[m] = 0;
      if (p < P && p - g * R.W < lc[g]) {
        const uint64_t key = lk[p];
        v[m] = ord2f((uint32_t)(key >> 32));
        ix[m] = 0xFFFFFFFFu - (uint32_t)key;
        ++cnt;
        mn = fminf(mn, v[m]);
        mx = fmaxf(mx, v[m]);
      }
    }
    reduce_stats(cnt, mn, mx, sm);
    k = min(R.W, sm.nvalid);
    if (k > 0) select_bins<kSel2CPT>(cand, n * V, 0u, v, [&](int m) { return ix[m]; }, k, true, sm);
  } else if constexpr (REGS) {
    float v[kSelectCPT];
    load_cands<kSelectCPT>(cand, n * V, v, sm);
    k = min(R.W, sm.nvalid);
    if (k > 0) select_bins<kSelectCPT>(cand, n * V, 0u, v, [](int m) { return reg_cand(m); }, k, true, sm);
  } else {
    scan_cands(cand, n * V, sm);
    k = min(R.W, sm.nvalid);
    if (k > 0) select_stream(cand, n * V, 0u, k, sm);
  }
  __syncthreads();
  const int *node_cur = (const int *)(slot + dev.sl.node[cur]);
  const int *codes_cur = (const int *)(slot + dev.sl.codes[cur]);
  const int *anc_cur = (const int *)(slot + dev.sl.anc[cur]);
  int *codes_nxt = (int *)(slot + dev.sl.codes[nxt]);
  int *anc_nxt = (int *)(slot + dev.sl.anc[nxt]);
  float *score_nxt = (float *)(slot + dev.sl.score[nxt]);
  int *node_nxt = (int *)(slot + dev.sl.node[nxt]);
  int *parent_nxt = (int *)(slot + dev.sl.parent[nxt]);
  const uint32_t *mask = dev.trie_mask + dev.trie_off[s] * MW;
  const int32_t *child = dev.trie_child + dev.trie_off[s];
  for (int i = tid; i < k; i += kTopkThreads) {
    const uint64_t key = sm.sel[i];
    const uint32_t flat = 0xFFFFFFFFu - (uint32_t)key;
    const int j = flat / V, c = flat % V;
    for (int t = 0; t < s; ++t) {
      codes_nxt[i * lvl + t] = codes_cur[j * lvl + t];
      anc_nxt[i * lvl + t] = anc_cur[j * lvl + t];
    }
    codes_nxt[i * lvl + s] = c;
    anc_nxt[i * lvl + s] = i;
    score_nxt[i] = ord2f((uint32_t)(key >> 32));
    parent_nxt[i] = j;
    const int nj = node_cur[j];
    const uint32_t *mrow = mask + (size_t)nj * MW;
    int below = 0;
    for (int wd = 0; wd < (c >> 5); ++wd) below += __popc(mrow[wd]);
    below += __popc(mrow[c >> 5] & ((1u << (c & 31)) - 1u));
    node_nxt[i] = child[nj] + below;
  }
  if (tid == 0) ((int *)(slot + dev.sl.n_live))[nxt] = k;
}

template <bool REGS>
__global__ __launch_bounds__(kTopkThreads) void k_topk_select(const float *__restrict__ cand, int n_rows, int V,
                                                              int k, int32_t *out_flat, float *out_score,
                                                              int32_t *n_out) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x;
  const int n_total = n_rows * V;
  int ke;
  if constexpr (REGS) {
    float v[kSelectCPT];
    load_cands<kSelectCPT>(cand, n_total, v, sm);
    ke = min(k, sm.nvalid);
    if (ke > 0) select_bins<kSelectCPT>(cand, n_total, 0u, v, [](int m) { return reg_cand(m); }, ke, true, sm);
  } else {
    scan_cands(cand, n_total, sm);
    ke = min(k, sm.nvalid);
    if (ke > 0) select_stream(cand, n_total, 0u, ke, sm);
  }
  __syncthreads();
  for (int i = tid; i < ke; i += kTopkThreads) {
    const uint64_t key = sm.sel[i];
    out_flat[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    out_score[i] = ord2f((uint32_t)(key >> 32));
  }
  if (tid == 0) *n_out = ke;
}

// --------------------------------------------------------------------------------------
// Context loading: one workgroup per (layer, kv head, 64-token tile), 16-byte chunks.
// COPY: the caller's K and V [L][N][Hkv][d] go to native K [L][Hkv][Np][d] (a permutation of
// whole token rows, copied chunk for chunk) and V^T [L][Hkv][d][Np] (transposed through
// LDS), padding tokens N..Np-1 zero.  Otherwise the native arrays are only read.  Either
// way the tile's tokens t < N are folded into the maxima of its (layer, kv head): squared
// key norm and |v|, kept as float bits (non-negative floats order like their bit patterns)
// by an atomic max into kn_bits / vm_bits, which k_load_finish turns into the key-norm bound
// and the value scale.
template <int S> struct UIntOf;
template <> struct UIntOf<2> { using type = uint16_t; };
template <> struct UIntOf<4> { using type = uint32_t; };

// element i of a 16-byte chunk as float (bf16 or f32 payload)
template <typename T>
__device__ __forceinline__ float chunk_elem(const u32x4_t &x, int i) {
  if (sizeof(T) == 2) return __uint_as_float((i & 1) ? (x[i >> 1] & 0xFFFF0000u) : (x[i >> 1] << 16));
  return __uint_as_float(x[i]);
}

constexpr int kLoadTile = 64;

template <typename T, int D, bool COPY>
__global__ __launch_bounds__(256) void k_load_ctx(const T *__restrict__ src_k, const T *__restrict__ src_v,
                                                  T *__restrict__ nk, T *__restrict__ nvt, int N, int Np, int Hkv,
                                                  uint32_t *__restrict__ kn_bits, uint32_t *__restrict__ vm_bits) {
  using U = typename UIntOf<sizeof(T)>::type;
  constexpr int EPC = 16 / sizeof(T);          // elements per chunk
  constexpr int TT = kLoadTile;
  constexpr int CPR = D / EPC;                 // chunks per token row: 8, 16 or 32, divides 64
  constexpr int CPT = TT / EPC;                // chunks per V^T row segment of the tile
  constexpr int NI = TT * CPR / 256;           // token-row chunks per thread
  constexpr int NO = D * CPT / 256;            // V^T chunks per thread
  static_assert(NI * 256 == TT * CPR && NO * 256 == D * CPT && 64 % CPR == 0, "tile shape");
  __shared__ U sv[COPY ? D : 1][TT + 4 / sizeof(T)];  // one dword of padding per row
  const int tid = threadIdx.x;
  const int n_tiles = Np / TT;
  const int lh = blockIdx.x / n_tiles, t0 = (blockIdx.x - lh * n_tiles) * TT;
  const int l = lh / Hkv, h = lh - l * Hkv;
  T *krows = nk + ((size_t)lh * Np + t0) * D;  // the tile's native K rows are contiguous
  const size_t src_row = (size_t)Hkv * D;      // caller layout: token stride
  const size_t src0 = ((size_t)l * N * Hkv + h) * D;
  constexpr int GI = NI < 4 ? NI : 4, GO = NO < 4 ? NO : 4;  // chunks in flight per thread per group
  float kmax = 0.f, vmax = 0.f;
#pragma unroll 1
  for (int i0 = 0; i0 < NI; i0 += GI) {
    u32x4_t xk[GI], xv[COPY ? GI : 1];
    // every load of the group is issued before the first use
#pragma unroll
    for (int j = 0; j < GI; ++j) {
      const int c = tid + 256 * (i0 + j), r = c / CPR, q = c % CPR, t = t0 + r;
      xk[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (COPY) {
        xv[j] = u32x4_t{0u, 0u, 0u, 0u};
        if (t < N) {
          xk[j] = gld<u32x4_t>(src_k + src0 + (size_t)t * src_row + q * EPC);
          xv[j] = gld<u32x4_t>(src_v + src0 + (size_t)t * src_row + q * EPC);
        }
      } else if (t < N) {
        xk[j] = gld<u32x4_t>(krows + (size_t)r * D + q * EPC);
      }
    }
#pragma unroll
    for (int j = 0; j < GI; ++j) {
      const int c = tid + 256 * (i0 + j), r = c / CPR, q = c % CPR;
      if (COPY) gst<u32x4_t>(krows + (size_t)r * D + q * EPC, xk[j]);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float x = chunk_elem<T>(xk[j], e);
        ss = fmaf(x, x, ss);
      }
#pragma unroll
      for (int o = CPR / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);  // the row's lanes are aligned
      kmax = fmaxf(kmax, ss);
      if (COPY) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float x = chunk_elem<T>(xv[j], e);
          vmax = fmaxf(vmax, fabsf(x));
          sv[q * EPC + e][r] = (U)(sizeof(T) == 2 ? (__float_as_uint(x) >> 16) : __float_as_uint(x));
        }
      }
    }
  }
  if (COPY) __syncthreads();
#pragma unroll 1
  for (int i0 = 0; i0 < NO; i0 += GO) {
    u32x4_t y[GO];
#pragma unroll
    for (int j = 0; j < GO; ++j) {
      const int c = tid + 256 * (i0 + j), dd = c / CPT, q = c % CPT, tb = t0 + q * EPC;
      if (COPY) {
        const uint32_t *p = (const uint32_t *)&sv[dd][0] + q * 4;
        y[j] = u32x4_t{p[0], p[1], p[2], p[3]};
      } else {
        y[j] = u32x4_t{0u, 0u, 0u, 0u};
        if (tb < N) y[j] = gld<u32x4_t>(nvt + ((size_t)lh * D + dd) * Np + tb);
      }
    }
#pragma unroll
    for (int j = 0; j < GO; ++j) {
      const int c = tid + 256 * (i0 + j), dd = c / CPT, q = c % CPT, tb = t0 + q * EPC;
      if (COPY) {
        gst<u32x4_t>(nvt + ((size_t)lh * D + dd) * Np + tb, y[j]);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (tb + e < N) vmax = fmaxf(vmax, fabsf(chunk_elem<T>(y[j], e)));
      }
    }
  }
  // one atomic pair per workgroup: atomics of many workgroups on the same few lines serialise
  __shared__ float sred[2][4];
  kmax = wave_max(kmax);
  vmax = wave_max(vmax);
  if ((tid & 63) == 0) {
    sred[0][tid >> 6] = kmax;
    sred[1][tid >> 6] = vmax;
  }
  __syncthreads();
  if (tid == 0) {
    atomicMax(kn_bits + lh, __float_as_uint(fmaxf(fmaxf(sred[0][0], sred[0][1]), fmaxf(sred[0][2], sred[0][3]))));
    atomicMax(vm_bits + lh, __float_as_uint(fmaxf(fmaxf(sred[1][0], sred[1][1]), fmaxf(sred[1][2], sred[1][3]))));
  }
}

__global__ void k_load_init(uint32_t *kn_bits, uint32_t *vm_bits, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    kn_bits[i] = 0u;
    vm_bits[i] = 0u;
  }
}

// In place: kn = sqrt(largest squared key norm); vs = 2^e with max|v| < 2^e (frexp: max|v| =
// m 2^e, m in [0.5, 1)), kept a normal float.
// V^T [L][Hkv][d][Np] bf16 -> its float16 copy in the wide kernel's units (v16_factor), one
// 16-byte chunk per thread; grid (chunks of one (layer, kv head), L*Hkv).
__global__ __launch_bounds__(256) void k_load_v16(const u32x4_t *__restrict__ vt, u32x4_t *__restrict__ vt16,
                                                  const float *__restrict__ vscale, int chunks) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const size_t i = (size_t)blockIdx.y * chunks + c;
  bool raw;
  const float f = v16_factor(vscale[blockIdx.y], raw);
  const u32x4_t x = vt[i];
  u32x4_t y;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = __uint_as_float(x[e] << 16), b = __uint_as_float(x[e] & 0xFFFF0000u);
    y[e] = raw ? pack_f16(a, b) : pack_f16(a * f, b * f);
  }
  vt16[i] = y;
}

__global__ void k_load_finish(float *kn, float *vs, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    kn[i] = sqrtf(__uint_as_float(((const uint32_t *)kn)[i]));
    int ex = 0;
    (void)frexpf(__uint_as_float(((const uint32_t *)vs)[i]), &ex);
    vs[i] = ldexpf(1.f, min(max(ex, -126), 127));
  }
}

struct GatherSlots {
  int32_t slot[kGatherMax];
};

// one workgroup per listed slot: the root beam (level 0, empty prefix, score 0)
__global__ void k_init_slot(Dev dev, GatherSlots gs, int n) {
  if ((int)blockIdx.x >= n) return;
  uint8_t *sb = slot_base(dev, gs.slot[blockIdx.x]);
  if (threadIdx.x == 0) {
    ((int *)(sb + dev.sl.n_live))[0] = 1;
    ((int *)(sb + dev.sl.n_live))[1] = 0;
    ((float *)(sb + dev.sl.score[0]))[0] = 0.f;
    ((int *)(sb + dev.sl.node[0]))[0] = 0;
    ((int *)(sb + dev.sl.parent[0]))[0] = -1;
  }
  for (int t = threadIdx.x; t < dev.dm.levels; t += blockDim.x) {
    ((int *)(sb + dev.sl.codes[0]))[t] = 0;
    ((int *)(sb + dev.sl.anc[0]))[t] = 0;
  }
}

// one workgroup per request: final n_live, codes and scores into the staging area
__global__ __launch_bounds__(256) void k_gather_results(Dev dev, GatherSlots gs, int n, int parity, uint8_t *out,
                                                        size_t out_bytes) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const uint8_t *sb = slot_base(dev, gs.slot[i]);
  const int lv = dev.dm.levels;
  const int nl = ((const int *)(sb + dev.sl.n_live))[parity];
  uint8_t *o = out + (size_t)i * out_bytes;
  if (threadIdx.x == 0) *(int32_t *)o = nl;
  int32_t *oc = (int32_t *)(o + 16);
  float *os = (float *)(o + 16 + (size_t)dev.dm.W_max * lv * 4);
  const int32_t *codes = (const int32_t *)(sb + dev.sl.codes[parity]);
  const float *score = (const float *)(sb + dev.sl.score[parity]);
  for (int e = threadIdx.x; e < nl * lv; e += blockDim.x) oc[e] = codes[e];
  for (int e = threadIdx.x; e < nl; e += blockDim.x) os[e] = score[e];
}

}  // namespace

// ---------------------------------------------------------------------------- launchers
namespace {
template <typename K, typename... Args>
void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, LaunchEv ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}
}  // namespace

hipError_t launch_ctx_attn(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs, int ctx_kind,
                           hipStream_t st, LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  const dim3 grid(total_wgs);
  if (dev.dm.dtype == 0) {
    if (dev.dm.d == 64)
      launch(k_ctx_attn_f32<64>, grid, dim3(256), st, ev, dev, reqs, n_reqs, layer);
    else
      launch(k_ctx_attn_f32<128>, grid, dim3(256), st, ev, dev, reqs, n_reqs, layer);
    return hipGetLastError();
  }
  const int nw = ctx_kind & 0xFF;
  const dim3 blk(nw * 64);
  if (dev.dm.d == 128) {
    if (nw == 8)
      launch(k_ctx_attn_wide<false>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
    else if (nw == 4)
      launch(k_ctx_attn_bf16_narrow<128, 4, 64>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
    else if (nw == 2)
      launch(k_ctx_attn_stream<4, false, 2>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
    else
      launch(k_ctx_attn_stream<4, false>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
  } else {
    if (nw == 4)
      launch(k_ctx_attn_bf16_narrow<64, 4, 64>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
    else if (nw == 2)
      launch(k_ctx_attn_bf16_narrow<64, 2, 32>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
    else
      launch(k_ctx_attn_bf16_narrow<64, 1, 32>, grid, blk, st, ev, dev, reqs, n_reqs, layer);
  }
  return hipGetLastError();
}

hipError_t launch_ctx_attn_layered(const Dev &dev, const StepReq *reqs, int n_reqs, int layer0, int total_wgs,
                                   int ctx_kind, hipStream_t st, LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.dtype != 1 || dev.dm.d != 128) return hipErrorInvalidValue;
  if ((ctx_kind & 0xFF) == 2) {
    launch(k_ctx_attn_stream<4, false, 2, true>, dim3(total_wgs), dim3(128), st, ev, dev, reqs, n_reqs, layer0);
    return hipGetLastError();
  }
  if ((ctx_kind & 0xFF) != 8) return hipErrorInvalidValue;
  launch(k_ctx_attn_wide<true>, dim3(total_wgs), dim3(512), st, ev, dev, reqs, n_reqs, layer0);
  return hipGetLastError();
}

hipError_t launch_sum_hparts(const Dev &dev, const StepReq *reqs, int n_reqs, hipStream_t st, LaunchEv ev) {
  if (n_reqs <= 0) return hipSuccess;
  launch(k_sum_hparts, dim3(128, n_reqs), dim3(256), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_ctx_attn_first_level(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs,
                                       hipStream_t st, LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  launch(k_ctx_attn_stream<3, true>, dim3(total_wgs, dev.dm.L), dim3(64), st, ev, dev, reqs, n_reqs, 0);
  return hipGetLastError();
}

hipError_t launch_finish_first_level(const Dev &dev, const StepReq *reqs, int n_reqs, hipStream_t st, LaunchEv ev) {
  if (n_reqs <= 0) return hipSuccess;
  launch(k_finish_first_level<128>, dim3(n_reqs, dev.dm.L), dim3(256), st, LaunchEv{ev.start, nullptr}, dev, reqs,
         n_reqs);
  launch(k_sum_layers, dim3(n_reqs, 8), dim3(256), st, LaunchEv{nullptr, ev.stop}, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_beam_merge(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                             hipStream_t st, LaunchEv ev, int wg0) {
  if (total_wgs <= 0) return hipSuccess;
  const dim3 grid(total_wgs), blk(256);
  if (dev.dm.dtype == 0) {
    if (dev.dm.d == 64)
      launch(k_beam_merge<64, float>, grid, blk, st, ev, dev, reqs, n_reqs, layer, wg0);
    else
      launch(k_beam_merge<128, float>, grid, blk, st, ev, dev, reqs, n_reqs, layer, wg0);
  } else {
    if (dev.dm.d == 64)
      launch(k_beam_merge<64, uint16_t>, grid, blk, st, ev, dev, reqs, n_reqs, layer, wg0);
    else
      launch(k_beam_merge<128, uint16_t>, grid, blk, st, ev, dev, reqs, n_reqs, layer, wg0);
  }
  return hipGetLastError();
}

hipError_t launch_finish_layer(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                              hipStream_t st, LaunchEv ev, int wg0) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.dtype != 1) return hipErrorInvalidValue;
  if (dev.dm.d == 64)
    launch(k_finish_layer<64>, dim3(total_wgs), dim3(256), st, ev, dev, reqs, n_reqs, layer, wg0);
  else
    launch(k_finish_layer<128>, dim3(total_wgs), dim3(256), st, ev, dev, reqs, n_reqs, layer, wg0);
  return hipGetLastError();
}

hipError_t launch_logits(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st,
                         LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.dtype == 1)
    launch(k_logits_x3, dim3(total_wgs), dim3(256), st, ev, dev, reqs, n_reqs);
  else
    launch(k_logits, dim3(total_wgs), dim3(256), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_label_head(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st,
                             LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.n_labels < 1 || dev.dm.n_labels > kMaxLabels || !dev.w_label || !dev.label_out)
    return hipErrorInvalidValue;
  launch(k_label_head, dim3(total_wgs), dim3(256), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_lsm(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st, LaunchEv ev) {
  if (total_wgs <= 0) return hipSuccess;
  launch(k_lsm, dim3(total_wgs), dim3(kTopkThreads), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_topk(const Dev &dev, const StepReq *reqs, int n_reqs, int max_cand, hipStream_t st, LaunchEv ev) {
  if (n_reqs <= 0) return hipSuccess;
  if (max_cand <= kTopkThreads * kSelectCPT)
    launch(k_select<true>, dim3(n_reqs), dim3(kTopkThreads), st, ev, dev, reqs, n_reqs);
  else
    launch(k_select<false>, dim3(n_reqs), dim3(kTopkThreads), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float *cand, int n_rows, int V, int k, int32_t *out_flat, float *out_score,
                              int32_t *n_out_dev, hipStream_t st) {
  // the register path reads 16-byte groups: the array must start on a 16-byte boundary
  if ((int64_t)n_rows * V <= (int64_t)kTopkThreads * kSelectCPT && ((uintptr_t)cand & 15) == 0)
    hipLaunchKernelGGL(k_topk_select<true>, dim3(1), dim3(kTopkThreads), 0, st, cand, n_rows, V, k, out_flat,
                       out_score, n_out_dev);
  else
    hipLaunchKernelGGL(k_topk_select<false>, dim3(1), dim3(kTopkThreads), 0, st, cand, n_rows, V, k, out_flat,
                       out_score, n_out_dev);
  return hipGetLastError();
}

hipError_t launch_load_v16(const void *nvt, void *nvt16, const float *vscale, int L, int Hkv, int d, int Np,
                           hipStream_t st) {
  if (Np % kLoadTile != 0 || Np < kLoadTile || d != 128 || L < 1 || Hkv < 1) return hipErrorInvalidValue;
  const int chunks = d * Np / 8;  // 16-byte chunks of one (layer, kv head)
  hipLaunchKernelGGL(k_load_v16, dim3((unsigned)((chunks + 255) / 256), (unsigned)(L * Hkv)), dim3(256), 0, st,
                     (const u32x4_t *)nvt, (u32x4_t *)nvt16, vscale, chunks);
  return hipGetLastError();
}

hipError_t launch_load_ctx(const void *src_k, const void *src_v, void *nk, void *nvt, bool copy, int L, int Hkv,
                           int N, int Np, int d, int elem_bytes, float *knmax, float *vscale, hipStream_t st) {
  if (Np % kLoadTile != 0 || N < 1 || N > Np || (d != 64 && d != 128) || (elem_bytes != 2 && elem_bytes != 4))
    return hipErrorInvalidValue;
  const int n = L * Hkv;
  uint32_t *kb = (uint32_t *)knmax, *vb = (uint32_t *)vscale;
  hipLaunchKernelGGL(k_load_init, dim3((n + 255) / 256), dim3(256), 0, st, kb, vb, n);
  const dim3 grid((unsigned)((size_t)n * (Np / kLoadTile)));
  auto go = [&](auto tag, auto dtag) {
    using T = decltype(tag);
    constexpr int D = decltype(dtag)::value;
    if (copy)
      hipLaunchKernelGGL((k_load_ctx<T, D, true>), grid, dim3(256), 0, st, (const T *)src_k, (const T *)src_v,
                         (T *)nk, (T *)nvt, N, Np, Hkv, kb, vb);
    else
      hipLaunchKernelGGL((k_load_ctx<T, D, false>), grid, dim3(256), 0, st, nullptr, nullptr, (T *)nk, (T *)nvt, N,
                         Np, Hkv, kb, vb);
  };
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (elem_bytes == 2) {
    if (d == 64) go(uint16_t{}, D64{});
    else go(uint16_t{}, D128{});
  } else {
    if (d == 64) go(float{}, D64{});
    else go(float{}, D128{});
  }
  hipLaunchKernelGGL(k_load_finish, dim3((n + 255) / 256), dim3(256), 0, st, knmax, vscale, n);
  return hipGetLastError();
}

hipError_t launch_gather_results(const Dev &dev, const int32_t *slots, int n, int parity, uint8_t *out,
                                 size_t out_bytes, hipStream_t st) {
  if (n <= 0 || n > kGatherMax) return hipErrorInvalidValue;
  GatherSlots gs{};
  for (int i = 0; i < n; ++i) gs.slot[i] = slots[i];
  hipLaunchKernelGGL(k_gather_results, dim3(n), dim3(256), 0, st, dev, gs, n, parity, out, out_bytes);
  return hipGetLastError();
}

hipError_t launch_init_slots(const Dev &dev, const int32_t *slots, int n, hipStream_t st) {
  if (n <= 0 || n > kGatherMax) return hipErrorInvalidValue;
  GatherSlots gs{};
  for (int i = 0; i < n; ++i) gs.slot[i] = slots[i];
  hipLaunchKernelGGL(k_init_slot, dim3(n), dim3(64), 0, st, dev, gs, n);
  return hipGetLastError();
}


hipError_t wave_times_select(int level, int layer) {
  const int sel[2] = {level, layer};
  return hipMemcpyToSymbol(HIP_SYMBOL(g_wave_times_sel), sel, sizeof sel, 0, hipMemcpyHostToDevice);
}

hipError_t wave_times_read(long long *host, size_t count) {
  if (!kWaveTimes) return hipErrorNotSupported;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_wave_times), count * sizeof(long long), 0, hipMemcpyDeviceToHost);
}

}  // namespace gr
