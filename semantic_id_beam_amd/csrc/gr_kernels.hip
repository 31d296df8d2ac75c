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
// Kernels per decode step (one launch sequence per layer, then logits/top-K):
//   k_ctx_attn_bf16   shared-context attention on MFMA, one (request, kv head,
//                     row block, token range) per workgroup -> (m, l, o) partials
//   k_ctx_attn_f32    the same on the vector ALU for float32 models
//   k_beam_merge      appends the new token to BeamKV, attends over the beam's
//                     own tokens found through BeamPath, merges with the
//                     context partials and adds the layer output to h
//   k_logits          h @ w_sid[level]
//   k_topk            trie-masked log-softmax, top-K over beams x codes,
//                     BeamPath update
#include <hip/hip_runtime.h>

#include "gr_internal.h"

namespace gr {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float ldf(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t *p, size_t i) { return bf2f(p[i]); }

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
__device__ __forceinline__ int wave_isum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup -> request: reqs[] is ordered by its first-workgroup field.
template <int FIELD>
__device__ __forceinline__ int find_req(const StepReq *reqs, int n, int bid) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const int first = FIELD == 0 ? reqs[mid].wg_ctx : FIELD == 1 ? reqs[mid].wg_merge : reqs[mid].wg_logits;
    if (first <= bid) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint8_t *slot_base(const Dev &dev, int slot) {
  return dev.slots + (size_t)slot * dev.sl.slot_bytes;
}

// Row r of a 64-token K tile is stored at LDS row swap23(r) (bits 2 and 3 exchanged).
// Lane l of the QK^T MFMA then reads LDS row l%32 and holds token swap23(l%32), which
// makes the score accumulator's layout equal to the PV MFMA's B-operand layout with
// 8 consecutive tokens per lane (no cross-lane shuffle between the two MFMAs).
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// --------------------------------------------------------------------------------------
// Shared-context attention, bf16 K/V, fp32 accumulate, MFMA 32x32x16.
//
// Workgroup = NW waves; wave w owns 32 query rows (beam j = row / g, head hq = h*g + row % g)
// of one kv head h of one request; all waves share the K/V tiles of one token range,
// double-buffered through LDS.  Per 32-token sub-tile and wave:
//   S^T[32 tok][32 q] = K_tile * Q^T     (D/16 MFMAs, A = K from LDS, B = Q in registers)
//   online softmax in the log2 domain with a lazy reference max (rescale only when a
//   column's max grows by more than 8, so p <= 256; exact since m and l share it)
//   O^T[D][32 q] += V^T_tile * P^T        (D/32 * 2 MFMAs, A = V^T from LDS, B = P as bf16)
// Output: unnormalised o, the reference max m (log2 units) and l per row and token range.
template <int D, int NW, int TT>
__global__ __launch_bounds__(NW * 64) void k_ctx_attn_bf16(Dev dev, const StepReq *__restrict__ reqs,
                                                           int n_reqs, int layer) {
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
  int local = blockIdx.x - R.wg_ctx;
  const int sp = local % R.splits;
  local /= R.splits;
  const int rb = local % R.row_blocks;
  const int h = local / R.row_blocks;

  const Dims &dm = dev.dm;
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
      if (s == 0) {
        qsrc = (const uint16_t *)(slot + dev.sl.q_last) + ((size_t)layer * dm.Hq + hq) * D;
      } else {
        const int *codes = (const int *)(slot + dev.sl.codes[s & 1]);
        const int code = codes[j * dm.levels + (s - 1)];
        qsrc = (const uint16_t *)dev.tok_q +
               ((((size_t)layer * (dm.levels - 1) + (s - 1)) * dm.V + code) * dm.Hq + hq) * D;
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (row_ok) {
        const uint4 u = *(const uint4 *)(qsrc + kb * 16 + 8 * hh);
        qf[kb] = __builtin_bit_cast(bf16x8_t, u);
      } else {
        qf[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      }
    }
  }

  const int t0 = sp * R.tps;
  const int t1 = min(R.N, t0 + R.tps);
  const int ntiles = (t1 - t0 + TT - 1) / TT;
  const uint16_t *gK = (const uint16_t *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const uint16_t *gV = (const uint16_t *)R.ctx_vt + (size_t)layer * R.ctx_lstride + (size_t)h * D * R.Np;

  uint4 rk[KPT], rv[VPT];
  auto gload = [&](int tb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT, r = c / (D / 8), cc = c % (D / 8);
      rk[i] = *(const uint4 *)(gK + (size_t)(tb + r) * D + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT, dd = c / (TT / 8), tc = c % (TT / 8);
      rv[i] = *(const uint4 *)(gV + (size_t)dd * R.Np + tb + tc * 8);
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

  gload(t0);
  lstore(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int tb = t0 + it * TT;
    if (it + 1 < ntiles) gload(tb + TT);
    if (wave_active) {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        if (tb + sub * 32 >= t1) break;
        f32x16_t sacc = f32x16_t{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8_t kf = sK[buf][sub * 32 + (lane & 31)][kb * 2 + hh];
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kb], sacc, 0, 0, 0);
        }
        // accumulator register i of lane (col q, half hh) holds token
        // tb + sub*32 + 16*(i/8) + 8*hh + (i%8)
        float mx = kNegInf;
        const int tbase = tb + sub * 32 + 8 * hh;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = tbase + 16 * (i >> 3) + (i & 7);
          if (tok >= t1) sacc[i] = kNegInf;
          mx = fmaxf(mx, sacc[i]);
        }
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
        float ls = 0.f;
        bf16x8_t pf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[i], c2, -M));
          ls += p;
          pf[i >> 3][i & 7] = (__bf16)p;
        }
        l += ls;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const bf16x8_t vf = sV[buf][db * 32 + (lane & 31)][sub * 4 + pp * 2 + hh];
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[pp], oacc[db], 0, 0, 0);
          }
        }
      }
    }
    if (it + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float ltot = l + __shfl_xor(l, 32);
  if (wave_active && row_ok) {
    const size_t prow = ((size_t)h * dm.S_max + sp) * ((size_t)dm.W_max * dm.g) + q_row;
    if (hh == 0) ((float2 *)(slot + dev.sl.part_ml))[prow] = make_float2(M, ltot);
    float *po = (float *)(slot + dev.sl.part_o) + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = db * 32 + 8 * a + 4 * hh;
        *(float4 *)(po + d0) =
            make_float4(oacc[db][4 * a], oacc[db][4 * a + 1], oacc[db][4 * a + 2], oacc[db][4 * a + 3]);
      }
    }
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
  const int rows_b = R.n_bound * dm.g;
  const int sp = lw % R.splits;
  lw /= R.splits;
  const int q_row = lw % rows_b;
  const int h = lw / rows_b;
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
    q = (const float *)dev.tok_q + ((((size_t)layer * (dm.levels - 1) + (s - 1)) * dm.V + code) * dm.Hq + hq) * D;
  }
  const float *gK = (const float *)R.ctx_k + (size_t)layer * R.ctx_lstride + (size_t)h * R.Np * D;
  const float *gV = (const float *)R.ctx_vt + (size_t)layer * R.ctx_lstride + (size_t)h * D * R.Np;
  const int t0 = sp * R.tps, t1 = min(R.N, t0 + R.tps);
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
  const size_t prow = ((size_t)h * dm.S_max + sp) * ((size_t)dm.W_max * dm.g) + q_row;
  if (lane == 0) ((float2 *)(slot + dev.sl.part_ml))[prow] = make_float2(M, l);
  float *po = (float *)(slot + dev.sl.part_o) + prow * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) po[lane + 64 * e] = o[e];
}

// --------------------------------------------------------------------------------------
// BeamKV append + beam-token attention + split-K merge + layer sum.  One wave per
// (request, beam j, kv head h), covering the g query heads of h.
//   step s >= 1: the new token's k/v (code c_{s-1}) are written to BeamKV slot
//   [layer][s-1][j]; the beam's earlier tokens t < s-1 are read from BeamKV slot
//   anc[j][t] (BeamPath) -- the beam never re-reads the tables for them.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_beam_merge(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                    int layer) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ri = find_req<1>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int lw = (blockIdx.x - R.wg_merge) * 4 + w;
  const int j = lw / dm.Hkv, h = lw % dm.Hkv;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  if (j >= n_live) return;
  const int g = dm.g, lvl = dm.levels;
  const float c2 = dm.scale_log2;

  float Mb[kMaxGroup], lb[kMaxGroup], ob[kMaxGroup][DPL];
#pragma unroll
  for (int gi = 0; gi < kMaxGroup; ++gi) {
    Mb[gi] = kNegInf;
    lb[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) ob[gi][e] = 0.f;
  }

  if (s > 0) {
    const int *codes = (const int *)(slot + dev.sl.codes[s & 1]);
    const int *anc = (const int *)(slot + dev.sl.anc[s & 1]);
    const int code = codes[j * lvl + (s - 1)];
    const size_t trow = ((size_t)layer * (lvl - 1) + (s - 1)) * dm.V + code;
    const T *kn = (const T *)dev.tok_k + (trow * dm.Hkv + h) * D;
    const T *vn = (const T *)dev.tok_v + (trow * dm.Hkv + h) * D;
    T *bk = (T *)(slot + dev.sl.beamkv_k);
    T *bv = (T *)(slot + dev.sl.beamkv_v);
    const size_t wstride = (size_t)dm.Hkv * D;  // one BeamKV slot
    const size_t lvstride = (size_t)dm.W_max * wstride;
    const size_t base_l = (size_t)layer * (lvl - 1) * lvstride;
    // append: BeamKV[layer][s-1][j][h]
    T kraw[DPL], vraw[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kraw[e] = kn[lane * DPL + e];
      vraw[e] = vn[lane * DPL + e];
      bk[base_l + (size_t)(s - 1) * lvstride + j * wstride + (size_t)h * D + lane * DPL + e] = kraw[e];
      bv[base_l + (size_t)(s - 1) * lvstride + j * wstride + (size_t)h * D + lane * DPL + e] = vraw[e];
    }
    float q[kMaxGroup][DPL];
#pragma unroll
    for (int gi = 0; gi < kMaxGroup; ++gi) {
      if (gi < g) {
        const T *qp = (const T *)dev.tok_q + (trow * dm.Hq + h * g + gi) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) q[gi][e] = ldf(qp, lane * DPL + e);
      }
    }
    for (int t = 0; t < s; ++t) {
      float kt[DPL], vt[DPL];
      if (t == s - 1) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          kt[e] = ldf(kraw, e);
          vt[e] = ldf(vraw, e);
        }
      } else {
        const int a = anc[j * lvl + t];
        const size_t off = base_l + (size_t)t * lvstride + a * wstride + (size_t)h * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          kt[e] = ldf(bk, off + e);
          vt[e] = ldf(bv, off + e);
        }
      }
#pragma unroll
      for (int gi = 0; gi < kMaxGroup; ++gi) {
        if (gi < g) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc = fmaf(q[gi][e], kt[e], acc);
          const float u = wave_sum(acc) * c2;
          const float Mn = fmaxf(Mb[gi], u);
          const float f = fast_exp2(Mb[gi] - Mn);
          const float p = fast_exp2(u - Mn);
          lb[gi] = lb[gi] * f + p;
#pragma unroll
          for (int e = 0; e < DPL; ++e) ob[gi][e] = fmaf(p, vt[e], ob[gi][e] * f);
          Mb[gi] = Mn;
        }
      }
    }
  }

  const float2 *pml = (const float2 *)(slot + dev.sl.part_ml);
  const float *po = (const float *)(slot + dev.sl.part_o);
  float *hbuf = (float *)(slot + dev.sl.h);
  const size_t wg = (size_t)dm.W_max * g;
#pragma unroll
  for (int gi = 0; gi < kMaxGroup; ++gi) {
    if (gi >= g) break;
    const int row = j * g + gi;
    float Ms = Mb[gi];
    for (int sp = 0; sp < R.splits; ++sp) Ms = fmaxf(Ms, pml[((size_t)h * dm.S_max + sp) * wg + row].x);
    const float fb = fast_exp2(Mb[gi] - Ms);
    float Ls = lb[gi] * fb, O[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) O[e] = ob[gi][e] * fb;
    for (int sp = 0; sp < R.splits; ++sp) {
      const size_t prow = ((size_t)h * dm.S_max + sp) * wg + row;
      const float2 ml = pml[prow];
      const float f = fast_exp2(ml.x - Ms);
      Ls = fmaf(ml.y, f, Ls);
#pragma unroll
      for (int e = 0; e < DPL; ++e) O[e] = fmaf(po[prow * D + lane * DPL + e], f, O[e]);
    }
    const float inv = 1.f / Ls;
    const int hq = h * g + gi;
    float *hr = hbuf + ((size_t)j * dm.Hq + hq) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float o = O[e] * inv;
      hr[e] = (layer == 0 ? 0.f : hr[e]) + o;
      if (dm.debug_attn)
        ((float *)(slot + dev.sl.dbg_attn))[(((size_t)layer * dm.W_max + j) * dm.Hq + hq) * D + lane * DPL + e] = o;
    }
  }
}

// --------------------------------------------------------------------------------------
// logits[j][c] = h[j] . w_sid[level][:, c]   (fp32, LDS-tiled, 32 rows x 64 codes per workgroup)
__global__ __launch_bounds__(256) void k_logits(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  const int tid = threadIdx.x;
  const int ri = find_req<2>(reqs, n_reqs, blockIdx.x);
  const StepReq R = reqs[ri];
  const Dims &dm = dev.dm;
  const int V = dm.V, H = dm.Hq * dm.d;
  const int nct = (V + 63) / 64;
  const int local = blockIdx.x - R.wg_logits;
  const int rt = local / nct, ct = local % nct;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int row0 = rt * 32;
  if (row0 >= n_live) return;
  const float *hb = (const float *)(slot + dev.sl.h);
  const float *W = dev.w_sid + (size_t)s * H * V;
  float *out = (float *)(slot + dev.sl.logits);
  __shared__ float sh[32][33];
  __shared__ float sw[32][65];
  const int ty = tid >> 4, tx = tid & 15;
  float acc[2][4] = {};
  for (int k0 = 0; k0 < H; k0 += 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256, r = e >> 5, kk = e & 31;
      sh[r][kk] = (row0 + r < n_live) ? hb[(size_t)(row0 + r) * H + k0 + kk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + i * 256, kk = e >> 6, cc = e & 63;
      const int col = ct * 64 + cc;
      sw[kk][cc] = col < V ? W[(size_t)(k0 + kk) * V + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float a0 = sh[ty * 2][kk], a1 = sh[ty * 2 + 1][kk];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float b = sw[kk][tx * 4 + c];
        acc[0][c] = fmaf(a0, b, acc[0][c]);
        acc[1][c] = fmaf(a1, b, acc[1][c]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = row0 + ty * 2 + r;
    if (row >= n_live) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = ct * 64 + tx * 4 + c;
      if (col < V) out[(size_t)row * V + col] = acc[r][c];
    }
  }
}

// --------------------------------------------------------------------------------------
// Top-K over a candidate array by radix select on unique 64-bit keys
//   key = order-preserving bits of the score << 32 | (0xFFFFFFFF - flat index)
// so "larger key" = higher score, then lower flat index.  The k largest keys are
// gathered and bitonic-sorted in LDS (descending).  1024 threads.
__device__ __forceinline__ uint32_t f2ord(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord2f(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t cand_key(float v, uint32_t i) {
  const float vc = (v == 0.f) ? 0.f : v;  // -0 ranks equal to +0
  return ((uint64_t)f2ord(vc) << 32) | (uint64_t)(0xFFFFFFFFu - i);
}

struct SelectSmem {
  uint64_t sel[kMaxBeam];
  int hist[256];
  uint64_t prefix;
  int need;
  int cnt;
  int nvalid;
};

// Leaves the k largest keys, sorted descending, in sm.sel[0..k).  k >= 1, k <= kMaxBeam,
// and at least k finite candidates.
__device__ void wg_select(const float *__restrict__ cand, int n_total, int k, SelectSmem &sm) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int need = k;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int b = tid; b < 256; b += kTopkThreads) sm.hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n_total; i += kTopkThreads) {
      const float v = cand[i];
      if (!(v > kNegInf)) continue;
      const uint64_t key = cand_key(v, (uint32_t)i);
      if (pass == 0 || (key >> (shift + 8)) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255], 1);
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
  const uint64_t kstar = prefix;
  if (tid == 0) sm.cnt = 0;
  __syncthreads();
  for (int i = tid; i < n_total; i += kTopkThreads) {
    const float v = cand[i];
    if (!(v > kNegInf)) continue;
    const uint64_t key = cand_key(v, (uint32_t)i);
    if (key >= kstar) {
      const int pos = atomicAdd(&sm.cnt, 1);
      sm.sel[pos] = key;
    }
  }
  __syncthreads();
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = tid; i < P; i += kTopkThreads)
    if (i >= k) sm.sel[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kTopkThreads) {
        const int pj = i ^ stride;
        if (pj > i) {
          const uint64_t a = sm.sel[i], b = sm.sel[pj];
          const bool desc = (i & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            sm.sel[i] = b;
            sm.sel[pj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Trie-masked log-softmax, top-K over beams x codes, BeamPath update.  One workgroup
// per request.
__global__ __launch_bounds__(kTopkThreads) void k_topk(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const StepReq R = reqs[blockIdx.x];
  const Dims &dm = dev.dm;
  uint8_t *slot = slot_base(dev, R.slot);
  const int s = R.level, V = dm.V, lvl = dm.levels, MW = dm.MW;
  const int cur = s & 1, nxt = cur ^ 1;
  const int n = ((const int *)(slot + dev.sl.n_live))[cur];
  const float *logits = (const float *)(slot + dev.sl.logits);
  float *cand = (float *)(slot + dev.sl.cand);
  const int *node_cur = (const int *)(slot + dev.sl.node[cur]);
  const float *score_cur = (const float *)(slot + dev.sl.score[cur]);
  const uint32_t *mask = dev.trie_mask + dev.trie_off[s] * MW;
  const int32_t *child = dev.trie_child + dev.trie_off[s];
  if (tid == 0) sm.nvalid = 0;
  __syncthreads();
  for (int j = w; j < n; j += kTopkThreads / 64) {
    const uint32_t *mrow = mask + (size_t)node_cur[j] * MW;
    const float sc = score_cur[j];
    float mx = kNegInf;
    for (int c = lane; c < V; c += 64) {
      const bool valid = (mrow[c >> 5] >> (c & 31)) & 1u;
      if (dm.norm == 1 || valid) mx = fmaxf(mx, logits[(size_t)j * V + c]);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int c = lane; c < V; c += 64) {
      const bool valid = (mrow[c >> 5] >> (c & 31)) & 1u;
      if (dm.norm == 1 || valid) sum += expf(logits[(size_t)j * V + c] - mx);
    }
    sum = wave_sum(sum);
    const float lse = mx + logf(sum);
    int cnt = 0;
    for (int c = lane; c < V; c += 64) {
      const bool valid = (mrow[c >> 5] >> (c & 31)) & 1u;
      cand[(size_t)j * V + c] = valid ? sc + (logits[(size_t)j * V + c] - lse) : kNegInf;
      cnt += valid;
    }
    cnt = wave_isum(cnt);
    if (lane == 0) atomicAdd(&sm.nvalid, cnt);
  }
  __syncthreads();
  const int k = min(R.W, sm.nvalid);
  if (k > 0) wg_select(cand, n * V, k, sm);
  __syncthreads();
  const int *codes_cur = (const int *)(slot + dev.sl.codes[cur]);
  const int *anc_cur = (const int *)(slot + dev.sl.anc[cur]);
  int *codes_nxt = (int *)(slot + dev.sl.codes[nxt]);
  int *anc_nxt = (int *)(slot + dev.sl.anc[nxt]);
  float *score_nxt = (float *)(slot + dev.sl.score[nxt]);
  int *node_nxt = (int *)(slot + dev.sl.node[nxt]);
  int *parent_nxt = (int *)(slot + dev.sl.parent[nxt]);
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

__global__ __launch_bounds__(kTopkThreads) void k_topk_select(const float *__restrict__ cand, int n_rows, int V,
                                                              int k, int32_t *out_flat, float *out_score,
                                                              int32_t *n_out) {
  __shared__ SelectSmem sm;
  const int tid = threadIdx.x;
  const int n_total = n_rows * V;
  if (tid == 0) sm.nvalid = 0;
  __syncthreads();
  int cnt = 0;
  for (int i = tid; i < n_total; i += kTopkThreads) cnt += (cand[i] > kNegInf) ? 1 : 0;
  atomicAdd(&sm.nvalid, cnt);
  __syncthreads();
  const int ke = min(k, sm.nvalid);
  if (ke > 0) wg_select(cand, n_total, ke, sm);
  __syncthreads();
  for (int i = tid; i < ke; i += kTopkThreads) {
    const uint64_t key = sm.sel[i];
    out_flat[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    out_score[i] = ord2f((uint32_t)(key >> 32));
  }
  if (tid == 0) *n_out = ke;
}

// --------------------------------------------------------------------------------------
// caller layout [L][N][Hkv][d] -> native K [L][Hkv][Np][d] and V^T [L][Hkv][d][Np], zero pad.
template <typename T>
__global__ void k_relayout_k(const T *__restrict__ src, T *__restrict__ dst, int L, int N, int Np, int Hkv, int d) {
  const size_t total = (size_t)L * Hkv * Np * d;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int dd = e % d;
    const size_t r = e / d;
    const int t = r % Np;
    const size_t r2 = r / Np;
    const int h = r2 % Hkv;
    const int l = r2 / Hkv;
    dst[e] = t < N ? src[(((size_t)l * N + t) * Hkv + h) * d + dd] : T(0);
  }
}
template <typename T>
__global__ void k_relayout_vt(const T *__restrict__ src, T *__restrict__ dst, int L, int N, int Np, int Hkv, int d) {
  const size_t total = (size_t)L * Hkv * d * Np;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const int t = e % Np;
    const size_t r = e / Np;
    const int dd = r % d;
    const size_t r2 = r / d;
    const int h = r2 % Hkv;
    const int l = r2 / Hkv;
    dst[e] = t < N ? src[(((size_t)l * N + t) * Hkv + h) * d + dd] : T(0);
  }
}

__global__ void k_init_slot(Dev dev, int slot) {
  uint8_t *sb = slot_base(dev, slot);
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

}  // namespace

// ---------------------------------------------------------------------------- launchers
hipError_t launch_ctx_attn(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs, int ctx_nw,
                           hipStream_t st) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.dtype == 0) {
    if (dev.dm.d == 64)
      hipLaunchKernelGGL(k_ctx_attn_f32<64>, dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    else
      hipLaunchKernelGGL(k_ctx_attn_f32<128>, dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    return hipGetLastError();
  }
  if (dev.dm.d == 128) {
    if (ctx_nw == 4)
      hipLaunchKernelGGL((k_ctx_attn_bf16<128, 4, 64>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    else if (ctx_nw == 2)
      hipLaunchKernelGGL((k_ctx_attn_bf16<128, 2, 32>), dim3(total_wgs), dim3(128), 0, st, dev, reqs, n_reqs, layer);
    else
      hipLaunchKernelGGL((k_ctx_attn_bf16<128, 1, 32>), dim3(total_wgs), dim3(64), 0, st, dev, reqs, n_reqs, layer);
  } else {
    if (ctx_nw == 4)
      hipLaunchKernelGGL((k_ctx_attn_bf16<64, 4, 64>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    else if (ctx_nw == 2)
      hipLaunchKernelGGL((k_ctx_attn_bf16<64, 2, 32>), dim3(total_wgs), dim3(128), 0, st, dev, reqs, n_reqs, layer);
    else
      hipLaunchKernelGGL((k_ctx_attn_bf16<64, 1, 32>), dim3(total_wgs), dim3(64), 0, st, dev, reqs, n_reqs, layer);
  }
  return hipGetLastError();
}

hipError_t launch_beam_merge(const Dev &dev, const StepReq *reqs, int n_reqs, int layer, int total_wgs,
                             hipStream_t st) {
  if (total_wgs <= 0) return hipSuccess;
  if (dev.dm.dtype == 0) {
    if (dev.dm.d == 64)
      hipLaunchKernelGGL((k_beam_merge<64, float>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    else
      hipLaunchKernelGGL((k_beam_merge<128, float>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
  } else {
    if (dev.dm.d == 64)
      hipLaunchKernelGGL((k_beam_merge<64, uint16_t>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
    else
      hipLaunchKernelGGL((k_beam_merge<128, uint16_t>), dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs, layer);
  }
  return hipGetLastError();
}

hipError_t launch_logits(const Dev &dev, const StepReq *reqs, int n_reqs, int total_wgs, hipStream_t st) {
  if (total_wgs <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_logits, dim3(total_wgs), dim3(256), 0, st, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_topk(const Dev &dev, const StepReq *reqs, int n_reqs, hipStream_t st) {
  if (n_reqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3(n_reqs), dim3(kTopkThreads), 0, st, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float *cand, int n_rows, int V, int k, int32_t *out_flat, float *out_score,
                              int32_t *n_out_dev, hipStream_t st) {
  hipLaunchKernelGGL(k_topk_select, dim3(1), dim3(kTopkThreads), 0, st, cand, n_rows, V, k, out_flat, out_score,
                     n_out_dev);
  return hipGetLastError();
}

hipError_t launch_relayout(const void *src_k, const void *src_v, void *dst_k, void *dst_vt, int L, int N, int Np,
                           int Hkv, int d, int elem_bytes, hipStream_t st) {
  const size_t total = (size_t)L * Hkv * Np * d;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(k_relayout_k<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t *)src_k,
                       (uint16_t *)dst_k, L, N, Np, Hkv, d);
    hipLaunchKernelGGL(k_relayout_vt<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t *)src_v,
                       (uint16_t *)dst_vt, L, N, Np, Hkv, d);
  } else {
    hipLaunchKernelGGL(k_relayout_k<float>, dim3(blocks), dim3(256), 0, st, (const float *)src_k, (float *)dst_k, L,
                       N, Np, Hkv, d);
    hipLaunchKernelGGL(k_relayout_vt<float>, dim3(blocks), dim3(256), 0, st, (const float *)src_v, (float *)dst_vt,
                       L, N, Np, Hkv, d);
  }
  return hipGetLastError();
}

hipError_t launch_init_slot(const Dev &dev, int slot, hipStream_t st) {
  hipLaunchKernelGGL(k_init_slot, dim3(1), dim3(64), 0, st, dev, slot);
  return hipGetLastError();
}

}  // namespace gr
