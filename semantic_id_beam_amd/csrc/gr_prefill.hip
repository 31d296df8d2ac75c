// Prefill of a request's ContextKV from context token ids, written for gfx950 (MI355X).
//
// The step before the decode path.  A context token's key and value at layer l are rows of
// per-layer tables indexed by token id (the stand-in for the projections of its embedding,
// as the fed-back code tables are in the decode step).  One position may instead hold a
// soft token: the paper-daily summary "Advancing Generative Recommendation Inference",
// section "Getting the user vector into the prompt: three approaches" (the third approach),
// maps a user vector through one linear layer to a token-sized embedding that takes a
// placeholder's place before the first forward pass; here that embedding is projected to
// the soft position's query, key and value per layer.
//
//   k_soft_embed    e = u * proj                       (one thread per embedding element)
//   k_soft_proj     e * w_{q,k,v}[l], split in kSoftSplit ranges of the embedding
//                   dimension (partial sums, added in order by the readers)
//   k_prefill_ctx   table rows (or the soft row, rounded to the model dtype) into the
//                   native layout: K rows copied as 16-byte chunks, V transposed through
//                   LDS; padding tokens zero
//   k_prefill_q     the last position's query into the request's slot
//
// All of it is HBM-bound gather and GEMV work: no matrix cores.
#include <hip/hip_runtime.h>

#include "gr_internal.h"

namespace gr {
namespace {

constexpr int kPfTile = 64;    // tokens per prefill workgroup (the native layout pads to it)
constexpr int kMaxEmbed = 8192;

// float -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ inline T from_f32(float f);
template <>
__device__ inline uint16_t from_f32<uint16_t>(float f) { return bf16_rne(f); }
template <>
__device__ inline float from_f32<float>(float f) { return f; }

// sum of the soft token's partials for column c of layer l
__device__ inline float soft_col(const float *part, int L, int ct, int l, int c) {
  float a = 0.f;
#pragma unroll
  for (int s = 0; s < kSoftSplit; ++s) a += part[((size_t)s * L + l) * ct + c];
  return a;
}

__global__ __launch_bounds__(256) void k_soft_embed(const float *__restrict__ u, const float *__restrict__ proj,
                                                    int du, int de, float *__restrict__ e) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= de) return;
  float a = 0.f;
  for (int i = 0; i < du; ++i) a = fmaf(u[i], proj[(size_t)i * de + j], a);
  e[j] = a;
}

// grid (ceil(ct / 256), L, kSoftSplit): thread = one output column of one layer over one
// range of the embedding dimension; consecutive threads read consecutive weight columns
__global__ __launch_bounds__(256) void k_soft_proj(const float *__restrict__ e, const float *__restrict__ wq,
                                                   const float *__restrict__ wk, const float *__restrict__ wv,
                                                   int de, int L, int cq, int ckv, float *__restrict__ part) {
  __shared__ float se[kMaxEmbed / kSoftSplit];
  const int chunk = (de + kSoftSplit - 1) / kSoftSplit;
  const int i0 = blockIdx.z * chunk, i1 = min(de, i0 + chunk);
  for (int i = i0 + (int)threadIdx.x; i < i1; i += 256) se[i - i0] = e[i];
  __syncthreads();
  const int l = blockIdx.y, ct = cq + 2 * ckv;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ct) return;
  const float *w;
  int cols, cc;
  if (c < cq) {
    w = wq + (size_t)l * de * cq;
    cols = cq;
    cc = c;
  } else if (c < cq + ckv) {
    w = wk + (size_t)l * de * ckv;
    cols = ckv;
    cc = c - cq;
  } else {
    w = wv + (size_t)l * de * ckv;
    cols = ckv;
    cc = c - cq - ckv;
  }
  float a = 0.f;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) a = fmaf(se[i - i0], w[(size_t)i * cols + cc], a);
  part[((size_t)blockIdx.z * L + l) * ct + c] = a;
}

// grid (Np / 64, Hkv, L), 256 threads
template <typename T>
__global__ __launch_bounds__(256) void k_prefill_ctx(const T *__restrict__ tk, const T *__restrict__ tv,
                                                     const int32_t *__restrict__ tok, int N, int Np, int soft_pos,
                                                     const float *__restrict__ part, int L, int cq, int Hkv, int d,
                                                     int vocab, T *__restrict__ nk, T *__restrict__ nvt) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int PITCH = 128 + EPC;          // LDS row pitch (elements), 16-byte multiple
  __shared__ __align__(16) T sv[kPfTile * PITCH];
  const int tile = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int cpr = d / EPC, ckv = Hkv * d, ct = cq + 2 * ckv;
  const size_t head = (size_t)l * Hkv + h;
  for (int idx = threadIdx.x; idx < kPfTile * cpr; idx += 256) {
    const int t = idx / cpr, ch = idx - t * cpr;
    const int n = tile * kPfTile + t;
    uint4 kc = make_uint4(0, 0, 0, 0), vc = make_uint4(0, 0, 0, 0);
    if (n < N) {
      if (n == soft_pos) {
        T kt[EPC], vt[EPC];
#pragma unroll
        for (int q = 0; q < EPC; ++q) {
          const int col = h * d + ch * EPC + q;
          kt[q] = from_f32<T>(soft_col(part, L, ct, l, cq + col));
          vt[q] = from_f32<T>(soft_col(part, L, ct, l, cq + ckv + col));
        }
        __builtin_memcpy(&kc, kt, 16);
        __builtin_memcpy(&vc, vt, 16);
      } else {
        const size_t row = (((size_t)l * vocab + (size_t)tok[n]) * Hkv + h) * d + (size_t)ch * EPC;
        kc = *reinterpret_cast<const uint4 *>(tk + row);
        vc = *reinterpret_cast<const uint4 *>(tv + row);
      }
    }
    *reinterpret_cast<uint4 *>(nk + (head * Np + n) * d + (size_t)ch * EPC) = kc;
    *reinterpret_cast<uint4 *>(sv + t * PITCH + ch * EPC) = vc;
  }
  __syncthreads();
  // V^T: row c of this head holds the tile's 64 tokens; a thread writes EPC of them
  constexpr int GPR = kPfTile / EPC;
  for (int idx = threadIdx.x; idx < d * GPR; idx += 256) {
    const int c = idx / GPR, g = idx - c * GPR;
    T v[EPC];
#pragma unroll
    for (int q = 0; q < EPC; ++q) v[q] = sv[(g * EPC + q) * PITCH + c];
    uint4 w;
    __builtin_memcpy(&w, v, 16);
    *reinterpret_cast<uint4 *>(nvt + (head * d + c) * Np + (size_t)tile * kPfTile + g * EPC) = w;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prefill_q(const T *__restrict__ tq, int last_tok,
                                                   const float *__restrict__ part, int L, int Hq, int Hkv, int d,
                                                   int vocab, T *__restrict__ q_slot, T *__restrict__ q_out) {
  const int cq = Hq * d, ct = cq + 2 * Hkv * d;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= L * cq) return;
  const int l = i / cq, c = i - l * cq;
  const T v = last_tok >= 0 ? tq[((size_t)l * vocab + (size_t)last_tok) * cq + c]
                            : from_f32<T>(soft_col(part, L, ct, l, c));
  q_slot[i] = v;
  if (q_out) q_out[i] = v;
}

}  // namespace

hipError_t launch_soft_token(const float *u, const float *proj, int du, int de, const float *wq, const float *wk,
                             const float *wv, int L, int cq, int ckv, float *e_buf, float *part, hipStream_t st) {
  if (du < 1 || de < 1 || de > kMaxEmbed || L < 1 || cq < 1 || ckv < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_soft_embed, dim3((unsigned)((de + 255) / 256)), dim3(256), 0, st, u, proj, du, de, e_buf);
  const int ct = cq + 2 * ckv;
  hipLaunchKernelGGL(k_soft_proj, dim3((unsigned)((ct + 255) / 256), (unsigned)L, kSoftSplit), dim3(256), 0, st,
                     e_buf, wq, wk, wv, de, L, cq, ckv, part);
  return hipGetLastError();
}

hipError_t launch_prefill_ctx(int elem_bytes, const void *tk, const void *tv, const int32_t *tok, int N, int Np,
                              int soft_pos, const float *part, int L, int Hq, int Hkv, int d, int vocab, void *nk,
                              void *nvt, hipStream_t st) {
  if (N < 1 || Np % kPfTile != 0 || N > Np || (d != 64 && d != 128) || (elem_bytes != 2 && elem_bytes != 4) ||
      soft_pos >= N || (soft_pos >= 0 && !part))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(Np / kPfTile), (unsigned)Hkv, (unsigned)L);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_prefill_ctx<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)tk, (const uint16_t *)tv,
                       tok, N, Np, soft_pos, part, L, Hq * d, Hkv, d, vocab, (uint16_t *)nk, (uint16_t *)nvt);
  else
    hipLaunchKernelGGL(k_prefill_ctx<float>, grid, dim3(256), 0, st, (const float *)tk, (const float *)tv, tok, N,
                       Np, soft_pos, part, L, Hq * d, Hkv, d, vocab, (float *)nk, (float *)nvt);
  return hipGetLastError();
}

hipError_t launch_prefill_q(int elem_bytes, const void *tq, int last_tok, const float *part, int L, int Hq, int Hkv,
                            int d, int vocab, void *q_slot, void *q_out, hipStream_t st) {
  if (last_tok >= vocab || (last_tok < 0 && !part) || (elem_bytes != 2 && elem_bytes != 4)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((size_t)L * Hq * d + 255) / 256));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_prefill_q<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)tq, last_tok, part, L, Hq,
                       Hkv, d, vocab, (uint16_t *)q_slot, (uint16_t *)q_out);
  else
    hipLaunchKernelGGL(k_prefill_q<float>, grid, dim3(256), 0, st, (const float *)tq, last_tok, part, L, Hq, Hkv, d,
                       vocab, (float *)q_slot, (float *)q_out);
  return hipGetLastError();
}

}  // namespace gr
