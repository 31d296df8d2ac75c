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
//   k_soft_embed    e = u * proj, split in kSoftSplit ranges of the user vector
//   k_soft_proj     e * w_{q,k,v}[l], split in kSoftSplit ranges of the embedding
//                   dimension (partial sums, added in order by the readers)
//   k_prefill_ctx   table rows (or the soft row, rounded to the model dtype) into the
//                   native layout: K rows copied as 16-byte chunks, V transposed through
//                   LDS; padding tokens zero; the key-norm and |v| maxima of each (layer,
//                   kv head) folded in (cleared by k_prefill_q before it, turned into the
//                   bounds by k_pf_bounds_finish after it)
//   k_prefill_q     the last position's query into the request's slot
//
// All of it is HBM-bound gather and GEMV work: no matrix cores.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "gr_internal.h"

namespace gr {
namespace {

// Fixed device array for the soft token's partial sums of the allocation-free prefill
// (gr_ctx_prefill_noalloc): every call on one GPU shares it.  Host code never passes its name
// to a kernel (on the host the name is a stand-in, not the device address): the address of
// each device's copy comes from hipGetSymbolAddress (prefill_scratch).
static __device__ __align__(256) float scratch[kPrefillScratchFloats];

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

// grid (ceil(de / 256), kSoftSplit): partial sums of e over kSoftSplit ranges of the user
// vector, e_part [kSoftSplit][de], added in order by k_soft_proj
__global__ __launch_bounds__(256) void k_soft_embed(const float *__restrict__ u, const float *__restrict__ proj,
                                                    int du, int de, float *__restrict__ e_part) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= de) return;
  const int chunk = (du + kSoftSplit - 1) / kSoftSplit;
  const int i0 = blockIdx.y * chunk, i1 = min(du, i0 + chunk);
  float a = 0.f;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) a = fmaf(u[i], proj[(size_t)i * de + j], a);
  e_part[(size_t)blockIdx.y * de + j] = a;
}

// grid (ceil(ct / 256), L, kSoftSplit): thread = one output column of one layer over one
// range of the embedding dimension; consecutive threads read consecutive weight columns
__global__ __launch_bounds__(256) void k_soft_proj(const float *__restrict__ e, const float *__restrict__ wq,
                                                   const float *__restrict__ wk, const float *__restrict__ wv,
                                                   int de, int L, int cq, int ckv, float *__restrict__ part) {
  __shared__ float se[kMaxEmbed / kSoftSplit];
  const int chunk = (de + kSoftSplit - 1) / kSoftSplit;
  const int i0 = blockIdx.z * chunk, i1 = min(de, i0 + chunk);
  for (int i = i0 + (int)threadIdx.x; i < i1; i += 256) {
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < kSoftSplit; ++s) a += e[(size_t)s * de + i];
    se[i - i0] = a;
  }
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

// element e of a 16-byte chunk as float (bf16 or f32 payload)
template <typename T>
__device__ inline float chunk_f32(const uint4 &x, int e) {
  const uint32_t w = e / (int)(4 / sizeof(T)) == 0 ? x.x : e / (int)(4 / sizeof(T)) == 1 ? x.y
                   : e / (int)(4 / sizeof(T)) == 2 ? x.z : x.w;
  if (sizeof(T) == 2) return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  return __uint_as_float(w);
}

// In place, per (layer, kv head): kn = sqrt(largest squared key norm), vs = 2^e with
// max|v| < 2^e (max|v| = m 2^e, m in [0.5, 1)), kept a normal float.  The decode's fixed
// softmax reference and value scaling read these; they are the same as a load computes.
__global__ void k_pf_bounds_finish(float *kn, float *vs, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    kn[i] = sqrtf(__uint_as_float(((const uint32_t *)kn)[i]));
    int ex = 0;
    (void)frexpf(__uint_as_float(((const uint32_t *)vs)[i]), &ex);
    vs[i] = ldexpf(1.f, min(max(ex, -126), 127));
  }
}

// grid (Np / 64, Hkv, L), 256 threads.  Besides the copy, each workgroup folds its tokens
// into the (layer, kv head) maxima of the squared key norm and of |v| (float bits, atomic
// max: non-negative floats order like their bit patterns).  A row's squared norm is summed
// per 16-byte chunk in element order, then over the row's chunks (consecutive lanes) by an
// xor-shuffle tree.
template <typename T>
__global__ __launch_bounds__(256) void k_prefill_ctx(const T *__restrict__ tk, const T *__restrict__ tv,
                                                     const int32_t *__restrict__ tok, int N, int Np, int soft_pos,
                                                     const float *__restrict__ part, int L, int cq, int Hkv, int d,
                                                     int vocab, T *__restrict__ nk, T *__restrict__ nvt,
                                                     uint32_t *__restrict__ kn_bits, uint32_t *__restrict__ vm_bits) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int PITCH = 128 + EPC;          // LDS row pitch (elements), 16-byte multiple
  __shared__ __align__(16) T sv[kPfTile * PITCH];
  __shared__ float sred[2][4];
  const int tile = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int cpr = d / EPC, ckv = Hkv * d, ct = cq + 2 * ckv;
  const size_t head = (size_t)l * Hkv + h;
  float kmax = 0.f, vmax = 0.f;
  // kPfTile * cpr is a multiple of 256 for every supported (d, dtype): all lanes run every
  // iteration, so the shuffles below see whole rows
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
        // ids from device memory (the allocation-free prefill) are not checked on the host:
        // clamped into the table, so every read stays in bounds
        const int id = min(max(tok[n], 0), vocab - 1);
        const size_t row = (((size_t)l * vocab + (size_t)id) * Hkv + h) * d + (size_t)ch * EPC;
        kc = *reinterpret_cast<const uint4 *>(tk + row);
        vc = *reinterpret_cast<const uint4 *>(tv + row);
      }
    }
    *reinterpret_cast<uint4 *>(nk + (head * Np + n) * d + (size_t)ch * EPC) = kc;
    *reinterpret_cast<uint4 *>(sv + t * PITCH + ch * EPC) = vc;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float x = chunk_f32<T>(kc, e);
      ss = fmaf(x, x, ss);
      vmax = fmaxf(vmax, fabsf(chunk_f32<T>(vc, e)));
    }
    for (int o = cpr / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    kmax = fmaxf(kmax, ss);
  }
  for (int o = 32; o > 0; o >>= 1) {
    kmax = fmaxf(kmax, __shfl_xor(kmax, o));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  }
  if ((threadIdx.x & 63) == 0) {
    sred[0][threadIdx.x >> 6] = kmax;
    sred[1][threadIdx.x >> 6] = vmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicMax(kn_bits + head, __float_as_uint(fmaxf(fmaxf(sred[0][0], sred[0][1]), fmaxf(sred[0][2], sred[0][3]))));
    atomicMax(vm_bits + head, __float_as_uint(fmaxf(fmaxf(sred[1][0], sred[1][1]), fmaxf(sred[1][2], sred[1][3]))));
  }
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

// Also clears the key-norm / |v| maxima that k_prefill_ctx (launched after it) folds into.
// The last token's id is last_tok, or (last_dev set) read from device memory and clamped into
// the table; last_tok < 0 without last_dev: the soft token's query.
template <typename T>
__global__ __launch_bounds__(256) void k_prefill_q(const T *__restrict__ tq, int last_tok,
                                                   const int32_t *__restrict__ last_dev,
                                                   const float *__restrict__ part, int L, int Hq, int Hkv, int d,
                                                   int vocab, T *__restrict__ q_slot, T *__restrict__ q_out,
                                                   uint32_t *__restrict__ kn_bits, uint32_t *__restrict__ vm_bits) {
  const int cq = Hq * d, ct = cq + 2 * Hkv * d;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < L * Hkv) {
    kn_bits[i] = 0u;
    vm_bits[i] = 0u;
  }
  if (i >= L * cq) return;
  const int l = i / cq, c = i - l * cq;
  const int lt = last_dev ? min(max(*last_dev, 0), vocab - 1) : last_tok;
  const T v = lt >= 0 ? tq[((size_t)l * vocab + (size_t)lt) * cq + c]
                      : from_f32<T>(soft_col(part, L, ct, l, c));
  q_slot[i] = v;
  if (q_out) q_out[i] = v;
}

}  // namespace

hipError_t launch_soft_token(const float *u, const float *proj, int du, int de, const float *wq, const float *wk,
                             const float *wv, int L, int cq, int ckv, float *e_buf, float *part, hipStream_t st) {
  if (du < 1 || de < 1 || de > kMaxEmbed || L < 1 || cq < 1 || ckv < 1) return hipErrorInvalidValue;
  if (!u || !proj || !wq || !wk || !wv || !e_buf || !part) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_soft_embed, dim3((unsigned)((de + 255) / 256), kSoftSplit), dim3(256), 0, st, u, proj, du, de,
                     e_buf);
  const int ct = cq + 2 * ckv;
  hipLaunchKernelGGL(k_soft_proj, dim3((unsigned)((ct + 255) / 256), (unsigned)L, kSoftSplit), dim3(256), 0, st,
                     e_buf, wq, wk, wv, de, L, cq, ckv, part);
  return hipGetLastError();
}

hipError_t launch_prefill_ctx(int elem_bytes, const void *tk, const void *tv, const int32_t *tok, int N, int Np,
                              int soft_pos, const float *part, int L, int Hq, int Hkv, int d, int vocab, void *nk,
                              void *nvt, float *knmax, float *vscale, hipStream_t st) {
  if (N < 1 || Np % kPfTile != 0 || N > Np || (d != 64 && d != 128) || (elem_bytes != 2 && elem_bytes != 4) ||
      soft_pos >= N || (soft_pos >= 0 && !part))
    return hipErrorInvalidValue;
  const int n = L * Hkv;
  uint32_t *kb = (uint32_t *)knmax, *vb = (uint32_t *)vscale;
  const dim3 grid((unsigned)(Np / kPfTile), (unsigned)Hkv, (unsigned)L);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_prefill_ctx<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)tk, (const uint16_t *)tv,
                       tok, N, Np, soft_pos, part, L, Hq * d, Hkv, d, vocab, (uint16_t *)nk, (uint16_t *)nvt, kb, vb);
  else
    hipLaunchKernelGGL(k_prefill_ctx<float>, grid, dim3(256), 0, st, (const float *)tk, (const float *)tv, tok, N,
                       Np, soft_pos, part, L, Hq * d, Hkv, d, vocab, (float *)nk, (float *)nvt, kb, vb);
  hipLaunchKernelGGL(k_pf_bounds_finish, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, knmax, vscale, n);
  return hipGetLastError();
}

hipError_t launch_prefill_q(int elem_bytes, const void *tq, int last_tok, const int32_t *last_dev, const float *part,
                            int L, int Hq, int Hkv, int d, int vocab, void *q_slot, void *q_out, float *knmax,
                            float *vscale, hipStream_t st) {
  if (last_tok >= vocab || (last_tok < 0 && !last_dev && !part) || (elem_bytes != 2 && elem_bytes != 4) ||
      Hkv > Hq * d)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(((size_t)L * Hq * d + 255) / 256));
  uint32_t *kb = (uint32_t *)knmax, *vb = (uint32_t *)vscale;
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_prefill_q<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)tq, last_tok, last_dev, part,
                       L, Hq, Hkv, d, vocab, (uint16_t *)q_slot, (uint16_t *)q_out, kb, vb);
  else
    hipLaunchKernelGGL(k_prefill_q<float>, grid, dim3(256), 0, st, (const float *)tq, last_tok, last_dev, part, L, Hq,
                       Hkv, d, vocab, (float *)q_slot, (float *)q_out, kb, vb);
  return hipGetLastError();
}

hipError_t prefill_scratch(float **out) {
  // once per device, with that device current: the address of its copy of the array
  static std::mutex mu;
  static std::vector<float *> ptrs;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= ptrs.size()) ptrs.resize((size_t)dev + 1, nullptr);
  if (!ptrs[(size_t)dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    ptrs[(size_t)dev] = static_cast<float *>(p);
  }
  *out = ptrs[(size_t)dev];
  return hipSuccess;
}

}  // namespace gr
