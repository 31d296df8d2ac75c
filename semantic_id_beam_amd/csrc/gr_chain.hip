// The layer chain of the decode step on gfx950 (MI355X): projections, norms and the SwiGLU MLP
// between the attention layers, so that layer l+1's new-token query, key and value come from
// layer l's output.  The pages run the decode on Qwen3-1.7B (paper-daily.com, "Advancing
// Generative Recommendation Inference", section "Performance"; zhiding.cn recsys-examples
// article, section "语义ID生成式推荐专用推理框架"); the layer is a pre-norm decoder layer of that
// shape with synthetic weights.
//
// Rows.  A step's beams are packed row by row, request after request, each request's block
// starting at a multiple of 32 (row0 of its descriptor) and padded up to the next multiple of
// 32; the packed row count is padded to a multiple of 128.  Padding rows (beams past the live
// count, the tail) start at zero and never reach BeamKV or the hidden vector.
//
//   k_chain_start   x = the new token's input vector (embed[s-1][code], or the request's x_last
//                   at s = 0), float32; xn = bf16(RMSNorm(x) * g_attn[0])
//   k_rmsnorm       xn = bf16(RMSNorm(x) * g)
//   k_gemm<EPI>     C = A W^T with A [rows][K] bf16 and W [N][K] bf16 (a projection's weight,
//                   out x in), fp32 accumulation on v_mfma_f32_32x32x16_bf16, and the epilogue:
//                     EPI_QKV     q -> the step's q rows (bf16), k and v -> BeamKV slot
//                                 [layer][s-1][beam] of the row's request (bf16)
//                     EPI_RESID   x += C (float32 residual stream)
//                     EPI_SWIGLU  act = bf16(silu(gate) * up); the tile's weight rows alternate
//                                 32 gate rows and the 32 matching up rows
//   k_chain_final   h = RMSNorm(x) * g_final (float32) into each request's hidden rows
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gr_internal.h"

namespace gr {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
#define GR_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ T gld(const void *p) {
  return *(const GR_GLOBAL T *)(p);
}
template <typename T>
__device__ __forceinline__ void gst(void *p, const T &v) {
  *(GR_GLOBAL T *)(p) = v;
}

// float -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return bf16_bits(a) | (bf16_bits(b) << 16); }

__device__ __forceinline__ float block_sum(float v, float *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];  // the same order in every thread
  return s;
}

// packed row -> request: reqs[] ordered by row0
__device__ __forceinline__ int find_row_req(const StepReq *reqs, int n, int row) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (reqs[mid].row0 <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ uint8_t *slot_of(const Dev &dev, int slot) { return dev.slots + (size_t)slot * dev.sl.slot_bytes; }

// RMSNorm of one float32 row of D into bf16: xn = bf16(x / sqrt(mean(x^2) + eps) * g).  One
// workgroup of 256 per row, D a multiple of 4 (each thread a 4-element run at a time).
__device__ __forceinline__ void norm_row(const float *x, const float *g, uint16_t *xn, int D, float eps, float *red) {
  float ss = 0.f;
  for (int i = 4 * (int)threadIdx.x; i < D; i += 4 * 256) {
    const f32x4_t v = gld<f32x4_t>(x + i);
    ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)D + eps);
  for (int i = 4 * (int)threadIdx.x; i < D; i += 4 * 256) {
    const f32x4_t v = gld<f32x4_t>(x + i), w = gld<f32x4_t>(g + i);
    gst<u32x2_t>(xn + i, u32x2_t{pack_bf16(v[0] * r * w[0], v[1] * r * w[1]), pack_bf16(v[2] * r * w[2], v[3] * r * w[3])});
  }
}

__global__ __launch_bounds__(256) void k_chain_start(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  __shared__ float red[4];
  const ChainDev &c = dev.ch;
  const int row = blockIdx.x, D = c.D;
  float *x = c.x + (size_t)row * D;
  const StepReq R = reqs[find_row_req(reqs, n_reqs, row)];
  const uint8_t *slot = slot_of(dev, R.slot);
  const int s = R.level, j = row - R.row0;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const bool live = row >= R.row0 && j < n_live && j < R.n_bound;
  const float *src = nullptr;
  const uint16_t *emb = nullptr;
  if (live) {
    if (s == 0) {
      src = (const float *)(slot + dev.sl.q_last);
    } else {
      const int code = ((const int *)(slot + dev.sl.codes[s & 1]))[j * dev.dm.levels + (s - 1)];
      emb = c.embed + ((size_t)(s - 1) * dev.dm.V + code) * D;
    }
  }
  for (int i = 4 * (int)threadIdx.x; i < D; i += 4 * 256) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (src) {
      v = gld<f32x4_t>(src + i);
    } else if (emb) {
      const u32x2_t b = gld<u32x2_t>(emb + i);
      v = f32x4_t{__uint_as_float(b[0] << 16), __uint_as_float(b[0] & 0xFFFF0000u), __uint_as_float(b[1] << 16),
                  __uint_as_float(b[1] & 0xFFFF0000u)};
    }
    gst<f32x4_t>(x + i, v);
  }
  __syncthreads();
  norm_row(x, c.g_attn, c.xn + (size_t)row * D, D, c.eps, red);
}

__global__ __launch_bounds__(256) void k_rmsnorm(const float *__restrict__ x, const float *__restrict__ g,
                                                 uint16_t *__restrict__ xn, int D, float eps) {
  __shared__ float red[4];
  norm_row(x + (size_t)blockIdx.x * D, g, xn + (size_t)blockIdx.x * D, D, eps, red);
}

__global__ __launch_bounds__(256) void k_chain_final(Dev dev, const StepReq *__restrict__ reqs, int n_reqs) {
  __shared__ float red[4];
  const ChainDev &c = dev.ch;
  const int row = blockIdx.x, D = c.D;
  const StepReq R = reqs[find_row_req(reqs, n_reqs, row)];
  uint8_t *slot = slot_of(dev, R.slot);
  const int j = row - R.row0;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[R.level & 1];
  if (row < R.row0 || j >= n_live || j >= R.n_bound) return;  // uniform over the workgroup
  const float *x = c.x + (size_t)row * D;
  float ss = 0.f;
  for (int i = 4 * (int)threadIdx.x; i < D; i += 4 * 256) {
    const f32x4_t v = gld<f32x4_t>(x + i);
    ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
  }
  const float r = rsqrtf(block_sum(ss, red) / (float)D + c.eps);
  float *h = (float *)(slot + dev.sl.h) + (size_t)j * D;
  for (int i = 4 * (int)threadIdx.x; i < D; i += 4 * 256) {
    const f32x4_t v = gld<f32x4_t>(x + i), w = gld<f32x4_t>(c.g_final + i);
    gst<f32x4_t>(h + i, f32x4_t{v[0] * r * w[0], v[1] * r * w[1], v[2] * r * w[2], v[3] * r * w[3]});
  }
}

// ---------------------------------------------------------------------------------------- GEMM
// Workgroup: 2 x NWN waves over a 128 (rows) x NWN*WN (weight rows) tile; wave (wm, wn) owns
// 64 x WN as 2 x (WN/32) MFMA blocks.  The 256-row tiles of the wide projections run eight waves
// of 64 x 64 (two waves per SIMD; the 128 x 128 tiles four of 64 x 64): against four waves of
// 64 x 128, the gate/up and q/k/v projections at 2,048 rows took about 4 % less time.  The K
// loop takes 64 columns per stage: the stage's A tile (16 KB) and W tile (BN/8 KB) go from
// global memory straight into LDS (global_load_lds_dwordx4, 1 KB of consecutive LDS per wave
// instruction), a ring of three stages with two in flight and one barrier per stage (4 k-steps
// of 16 between barriers); each k-step's fragments are read while the previous k-step's MFMAs
// run.  LDS rows are 128 bytes
// (8 chunks of 16): chunk c of row r sits at c ^ (r & 7) ^ ((r >> 3) & 1), so each group of 16
// lanes (16 rows, one chunk each) covers the 64 banks once.  The MFMA computes the transposed
// block D[n][m] = W_blk (32 x 16) x A_blk^T (16 x 32): lane (m, hh) then holds output row m,
// columns 8a + 4hh + {0..3} of the block, so each epilogue write is a run of four columns of one
// row.
enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };
constexpr int GBM = 128, GBK = 64, GNST = 3;
constexpr int kMaxKSplit = 8;  // K ranges of a split-K projection
constexpr int kWideNWN = 4;  // waves along the weight rows of a 256-row tile

__device__ __forceinline__ void dma16(const void *src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct GemmArgs {
  const uint16_t *A;    // [rows][K] bf16
  const uint16_t *W0;   // weight rows: EPI_QKV: q rows [0, n1), k rows [n1, n2), v rows [n2, N);
  const uint16_t *W1;   //   EPI_SWIGLU: W0 gate [I][K], W1 up [I][K] (N = 2I); else W0 [N][K]
  const uint16_t *W2;
  int n1, n2, N, K;
  int layer;            // EPI_QKV: BeamKV layer
  float *x;             // EPI_RESID: residual [rows][N] float32
  uint16_t *out;        // EPI_QKV: q rows [rows][n1]; EPI_SWIGLU: act [rows][N / 2]
  int ksplit;           // > 1: K in ksplit ranges, raw sums of the live rows to part[ks][row][col]
  float *part;          //   (SwiGLU columns in logical order: gate i at i, up i at N/2 + i)
};

// a packed row's request and whether the row is a live beam of it
__device__ __forceinline__ bool row_live(const Dev &dev, const StepReq *reqs, int n_reqs, int row) {
  const StepReq &R = reqs[find_row_req(reqs, n_reqs, row)];
  const int j = row - R.row0;
  const int n_live = ((const int *)(slot_of(dev, R.slot) + dev.sl.n_live))[R.level & 1];
  return row >= R.row0 && j < n_live && j < R.n_bound;
}

// source row of weight-tile row r (tile columns n0 ..); SwiGLU tiles alternate 32 gate rows and
// the matching 32 up rows
template <int EPI>
__device__ __forceinline__ const uint16_t *w_row(const GemmArgs &g, int n0, int r) {
  if constexpr (EPI == EPI_SWIGLU) {
    const int b = r >> 5, i = n0 / 2 + (b >> 1) * 32 + (r & 31);
    return ((b & 1) ? g.W1 : g.W0) + (size_t)i * g.K;
  } else if constexpr (EPI == EPI_QKV) {
    const int n = n0 + r;
    return n < g.n1 ? g.W0 + (size_t)n * g.K : n < g.n2 ? g.W1 + (size_t)(n - g.n1) * g.K : g.W2 + (size_t)(n - g.n2) * g.K;
  } else {
    return g.W0 + (size_t)(n0 + r) * g.K;
  }
}

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0 || N == 4 || N == 6 || N == 8 || N == 12, "unsupported wait");
}

template <int EPI, int WN, int NWN>
__global__ __launch_bounds__(128 * NWN) void k_gemm(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                    GemmArgs g, int m_tiles) {
  constexpr int NW = 2 * NWN;                                     // waves: 2 along rows x NWN
  constexpr int BN = NWN * WN;                                    // weight rows per tile
  constexpr int NB = WN / 32;                                     // MFMA blocks along the weight rows per wave
  constexpr int AI = GBM * 8 / (64 * NW), WI = BN * 8 / (64 * NW);  // DMA instructions per lane and stage
  static_assert(GNST == 3 && (WN == 32 || WN == 64 || WN == 128) && (BN == 128 || BN == 256), "tile shape");
  static_assert(EPI != EPI_SWIGLU || NB % 2 == 0, "a wave holds gate and up blocks in pairs");
  __shared__ bf16x8_t sA[GNST][GBM * 8];
  __shared__ bf16x8_t sW[GNST][BN * 8];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1;
  // workgroups are dealt round-robin over the 8 XCDs (blockIdx % 8): when the weight tiles split
  // evenly, XCD x takes weight tiles x, x+8, ... and runs every row tile of each, so a weight tile
  // is fetched into one XCD's L2 only (the smaller activation rows are what each XCD re-reads)
  const int n_tiles = g.N / BN;
  // split-K: range ks of K, the tile index the rest (ranges outermost)
  const int tile = (int)blockIdx.x % (m_tiles * n_tiles), ks = (int)blockIdx.x / (m_tiles * n_tiles);
  int mt, nt;
  if ((n_tiles & 7) == 0) {
    const int xcd = tile & 7, idx = tile >> 3;
    mt = idx % m_tiles;
    nt = (idx / m_tiles) * 8 + xcd;
  } else {
    mt = tile % m_tiles;
    nt = tile / m_tiles;
  }
  const int m0 = mt * GBM, n0 = nt * BN;
  const int KT = g.K / GBK / g.ksplit, k0 = ks * KT * GBK;

  // DMA: instruction i of wave w fills LDS chunks p = (i * NW + w) * 64 + lane: row p >> 3, stored
  // position p & 7 <- global chunk (p & 7) ^ swz(row); the 8 rows of one instruction lie in one
  // 32-row weight block
  const uint16_t *asrc[AI], *wsrc[WI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int p = (i * NW + w) * 64 + lane, r = p >> 3, c = (p & 7) ^ swz(r);
    asrc[i] = g.A + (size_t)(m0 + r) * g.K + k0 + c * 8;
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int p = (i * NW + w) * 64 + lane, r = p >> 3, c = (p & 7) ^ swz(r);
    wsrc[i] = w_row<EPI>(g, n0, r) + k0 + c * 8;
  }
  const uint32_t adst = lds_addr(&sA[0][0]) + w * 1024, wdst = lds_addr(&sW[0][0]) + w * 1024;
  auto issue = [&](int kt) {
    const int st = kt % GNST;
#pragma unroll
    for (int i = 0; i < AI; ++i) dma16(asrc[i] + kt * GBK, adst + st * (GBM * 128) + i * NW * 1024);
#pragma unroll
    for (int i = 0; i < WI; ++i) dma16(wsrc[i] + kt * GBK, wdst + st * (BN * 128) + i * NW * 1024);
  };

  f32x16_t acc[NB][2];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16_t{};

  issue(0);
  if (KT > 1) issue(1);
  const int rl = lane & 31, sw = swz(rl);
  for (int kt = 0; kt < KT; ++kt) {
    // stage kt has landed once at most the copies of stage kt+1 remain in flight
    if (kt + 1 < KT) vm_wait_barrier<AI + WI>(); else vm_wait_barrier<0>();
    if (kt + 2 < KT) issue(kt + 2);  // into the stage of tile kt-1, which every wave has left
    const int st = kt % GNST;
    const bf16x8_t *a = &sA[st][(wm * 64 + rl) * 8], *b = &sW[st][(wn * WN + rl) * 8];
    bf16x8_t af[2][2], wf[2][NB];
    auto frags = [&](int ks, int buf) {
      const int ch = (2 * ks + hh) ^ sw;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) af[buf][mb] = a[mb * 32 * 8 + ch];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[buf][nb] = b[nb * 32 * 8 + ch];
    };
    frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      // the next k-step's reads are issued ahead of this k-step's MFMAs (kept in that order)
      if (ks + 1 < GBK / 16) frags(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][nb], af[ks & 1][mb], acc[nb][mb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: lane (rl, hh) of block (nb, mb) holds row m0 + wm*64 + mb*32 + rl, columns
  // n0 + wn*WN + nb*32 + 8a + 4hh + c, c = 0..3, in acc[nb][mb][4a + c]
  const int ncol0 = n0 + wn * WN;
  if (g.ksplit > 1) {
    // raw sums of the live rows to this range's partials; k_gemm_reduce adds the ranges
    float *part = g.part + (size_t)ks * m_tiles * GBM * g.N;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int row = m0 + wm * 64 + mb * 32 + rl;
      if (!row_live(dev, reqs, n_reqs, row)) continue;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int col = ncol0 + nb * 32;
        if constexpr (EPI == EPI_SWIGLU) col = (nb & 1 ? g.N / 2 : 0) + ncol0 / 2 + (nb >> 1) * 32;
#pragma unroll
        for (int a = 0; a < 4; ++a)
          gst<f32x4_t>(part + (size_t)row * g.N + col + 8 * a + 4 * hh,
                       f32x4_t{acc[nb][mb][4 * a], acc[nb][mb][4 * a + 1], acc[nb][mb][4 * a + 2], acc[nb][mb][4 * a + 3]});
      }
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = m0 + wm * 64 + mb * 32 + rl;
    if constexpr (EPI == EPI_RESID) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float *p = g.x + (size_t)row * g.N + ncol0 + nb * 32 + 8 * a + 4 * hh;
          const f32x4_t o = gld<f32x4_t>(p);
          gst<f32x4_t>(p, f32x4_t{o[0] + acc[nb][mb][4 * a], o[1] + acc[nb][mb][4 * a + 1],
                                  o[2] + acc[nb][mb][4 * a + 2], o[3] + acc[nb][mb][4 * a + 3]});
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
      // blocks 2p and 2p+1 of the wave hold gate columns and the matching up columns
#pragma unroll
      for (int pr = 0; pr < NB / 2; ++pr) {
        const int i0 = ncol0 / 2 + pr * 32;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float gt = acc[2 * pr][mb][4 * a + c], up = acc[2 * pr + 1][mb][4 * a + c];
            v[c] = gt / (1.f + expf(-gt)) * up;
          }
          gst<u32x2_t>(g.out + (size_t)row * (g.N / 2) + i0 + 8 * a + 4 * hh,
                       u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])});
        }
      }
    } else {
      // q columns -> the step's q rows; k, v columns -> BeamKV of the row's request (live beams
      // at steps s >= 1 only).  The 32 rows of a block belong to one request; the WN columns of
      // a wave to one of q, k, v.
      if (ncol0 < g.n1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            gst<u32x2_t>(g.out + (size_t)row * g.n1 + ncol0 + nb * 32 + 8 * a + 4 * hh,
                         u32x2_t{pack_bf16(acc[nb][mb][4 * a], acc[nb][mb][4 * a + 1]),
                                 pack_bf16(acc[nb][mb][4 * a + 2], acc[nb][mb][4 * a + 3])});
      } else {
        const int blk0 = m0 + wm * 64 + mb * 32;
        const StepReq R = reqs[find_row_req(reqs, n_reqs, blk0)];
        const int s = R.level, j = row - R.row0;
        uint8_t *slot = slot_of(dev, R.slot);
        const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
        if (s > 0 && blk0 >= R.row0 && j < n_live && j < R.n_bound) {
          const Dims &dm = dev.dm;
          const bool is_v = ncol0 >= g.n2;
          uint16_t *kv = (uint16_t *)(slot + (is_v ? dev.sl.beamkv_v : dev.sl.beamkv_k));
          const size_t wstride = (size_t)dm.Hkv * dm.d, lvstride = (size_t)dm.W_max * wstride;
          uint16_t *dst = kv + (size_t)g.layer * dm.tl * lvstride + (size_t)(s - 1) * lvstride +
                          (size_t)j * wstride + (ncol0 - (is_v ? g.n2 : g.n1));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
              gst<u32x2_t>(dst + nb * 32 + 8 * a + 4 * hh,
                           u32x2_t{pack_bf16(acc[nb][mb][4 * a], acc[nb][mb][4 * a + 1]),
                                   pack_bf16(acc[nb][mb][4 * a + 2], acc[nb][mb][4 * a + 3])});
        }
      }
    }
  }
}

// The split-K ranges of a row added in range order, then the projection's epilogue (as in
// k_gemm): one workgroup per (request, block of 1024 columns), the request's live rows in turn,
// four columns per thread; every range's four values are loaded before the first is added.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_reduce(Dev dev, const StepReq *__restrict__ reqs, GemmArgs g, int rows) {
  const StepReq R = reqs[blockIdx.x];
  uint8_t *slot = slot_of(dev, R.slot);
  const int s = R.level;
  const int n_live = ((const int *)(slot + dev.sl.n_live))[s & 1];
  const int nr = min(n_live, R.n_bound);
  const int ncols = EPI == EPI_SWIGLU ? g.N / 2 : g.N;
  const int col = (int)blockIdx.y * 1024 + 4 * (int)threadIdx.x;
  if (col >= ncols) return;
  const size_t rstride = (size_t)rows * g.N;
  for (int j = 0; j < nr; ++j) {
    const int row = R.row0 + j;
    const float *p = g.part + (size_t)row * g.N;
    auto sum4 = [&](int c) {
      f32x4_t v[kMaxKSplit];
#pragma unroll
      for (int k = 0; k < kMaxKSplit; ++k)
        if (k < g.ksplit) v[k] = gld<f32x4_t>(p + k * rstride + c);
      f32x4_t acc = v[0];
#pragma unroll
      for (int k = 1; k < kMaxKSplit; ++k)
        if (k < g.ksplit) acc = f32x4_t{acc[0] + v[k][0], acc[1] + v[k][1], acc[2] + v[k][2], acc[3] + v[k][3]};
      return acc;
    };
    if constexpr (EPI == EPI_RESID) {
      const f32x4_t a = sum4(col);
      float *xp = g.x + (size_t)row * g.N + col;
      const f32x4_t o = gld<f32x4_t>(xp);
      gst<f32x4_t>(xp, f32x4_t{o[0] + a[0], o[1] + a[1], o[2] + a[2], o[3] + a[3]});
    } else if constexpr (EPI == EPI_SWIGLU) {
      const f32x4_t gt = sum4(col), up = sum4(ncols + col);
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = gt[c] / (1.f + expf(-gt[c])) * up[c];
      gst<u32x2_t>(g.out + (size_t)row * ncols + col, u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])});
    } else {
      const Dims &dm = dev.dm;
      const size_t wstride = (size_t)dm.Hkv * dm.d, lvstride = (size_t)dm.W_max * wstride;
      const f32x4_t a = sum4(col);
      const u32x2_t b = u32x2_t{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])};
      if (col < g.n1) {
        gst<u32x2_t>(g.out + (size_t)row * g.n1 + col, b);
      } else if (s > 0) {
        const bool is_v = col >= g.n2;
        uint16_t *kv = (uint16_t *)(slot + (is_v ? dev.sl.beamkv_v : dev.sl.beamkv_k));
        gst<u32x2_t>(kv + (size_t)g.layer * dm.tl * lvstride + (size_t)(s - 1) * lvstride + (size_t)j * wstride +
                         (col - (is_v ? g.n2 : g.n1)),
                     b);
      }
    }
  }
}

// ------------------------------------------------------------------- few-row projections
// Steps whose every request has one live row (the first level: one beam each) and at most
// kGemvRows requests: C = A W^T for those rows only, each weight streamed once.  One wave per
// output unit (a weight row; SwiGLU: gate row i and up row i), the unit's weights KL 16-byte
// loads per lane issued before anything waits (across the grid the whole matrix is in flight at
// once); the requests' A rows staged in LDS ([request][K] bf16, conflict-free 16-byte reads);
// products on v_dot2_f32_bf16, each request's sum reduced over the wave's lanes, then lane r
// applies the projection's epilogue for request r.
constexpr int kGemvRows = 8, kGemvWaves = 8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

template <int EPI, int KL>
__global__ __launch_bounds__(64 * kGemvWaves) void k_gemv(Dev dev, const StepReq *__restrict__ reqs, int n_reqs,
                                                          GemmArgs g, int units) {
  constexpr int K = KL * 512, NU = EPI == EPI_SWIGLU ? 2 : 1;
  __shared__ u32x4_t sA[kGemvRows][K / 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int unit = (int)blockIdx.x * kGemvWaves + __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool active = unit < units;  // uniform over the wave
  u32x4_t wr[NU][KL];
  if (active) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const uint16_t *wp = EPI == EPI_SWIGLU ? (u ? g.W1 : g.W0) + (size_t)unit * K : w_row<EPI>(g, 0, unit);
#pragma unroll
      for (int i = 0; i < KL; ++i) wr[u][i] = gld<u32x4_t>(wp + i * 512 + lane * 8);
    }
  }
  for (int c = tid; c < n_reqs * (K / 8); c += 64 * kGemvWaves) {
    const int r = c / (K / 8), k8 = c % (K / 8);
    sA[r][k8] = gld<u32x4_t>(g.A + (size_t)reqs[r].row0 * K + k8 * 8);
  }
  __syncthreads();
  if (!active) return;
  float acc[NU][kGemvRows];
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc[u][r] = 0.f;
#pragma unroll
  for (int i = 0; i < KL; ++i)
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      if (r >= n_reqs) break;  // uniform
      // (pairs taken from whole 8-element vectors: a bit cast of one element of a 4 x 32-bit
      // vector compiled to element 0 for every index)
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, sA[r][i * 64 + lane]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const bf16x8_t wv = __builtin_bit_cast(bf16x8_t, wr[u][i]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[u][r] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{wv[2 * e], wv[2 * e + 1]},
                                                      bf16x2_t{a[2 * e], a[2 * e + 1]}, acc[u][r], false);
      }
    }
  float mine[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    mine[u] = 0.f;
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
      float v = acc[u][r];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      if (lane == r) mine[u] = v;
    }
  }
  if (lane >= n_reqs) return;
  const StepReq &R = reqs[lane];
  const int row = R.row0;
  if constexpr (EPI == EPI_RESID) {
    float *xp = g.x + (size_t)row * g.N + unit;
    gst<float>(xp, gld<float>(xp) + mine[0]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    const float gt = mine[0], up = mine[NU - 1];
    gst<uint16_t>(g.out + (size_t)row * (g.N / 2) + unit, (uint16_t)bf16_bits(gt / (1.f + expf(-gt)) * up));
  } else {
    const uint16_t b = (uint16_t)bf16_bits(mine[0]);
    if (unit < g.n1) {
      gst<uint16_t>(g.out + (size_t)row * g.n1 + unit, b);
    } else if (R.level > 0) {
      const Dims &dm = dev.dm;
      const int s = R.level;
      const size_t wstride = (size_t)dm.Hkv * dm.d, lvstride = (size_t)dm.W_max * wstride;
      const bool is_v = unit >= g.n2;
      uint16_t *kv = (uint16_t *)(slot_of(dev, R.slot) + (is_v ? dev.sl.beamkv_v : dev.sl.beamkv_k));
      gst<uint16_t>(kv + (size_t)g.layer * dm.tl * lvstride + (size_t)(s - 1) * lvstride + (unit - (is_v ? g.n2 : g.n1)),
                    b);
    }
  }
}

template <typename K, typename... Args>
void launch(K kernel, dim3 grid, dim3 block, hipStream_t st, LaunchEv ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

}  // namespace

hipError_t launch_chain_start(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, hipStream_t st,
                              LaunchEv ev) {
  if (rows <= 0 || rows % 128 != 0 || dev.ch.D % 4 != 0) return hipErrorInvalidValue;
  launch(k_chain_start, dim3(rows), dim3(256), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_chain_norm(const Dev &dev, const float *g, int rows, hipStream_t st, LaunchEv ev) {
  if (rows <= 0 || rows % 128 != 0 || dev.ch.D % 4 != 0) return hipErrorInvalidValue;
  launch(k_rmsnorm, dim3(rows), dim3(256), st, ev, (const float *)dev.ch.x, g, dev.ch.xn, dev.ch.D, dev.ch.eps);
  return hipGetLastError();
}

hipError_t launch_chain_final(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, hipStream_t st,
                              LaunchEv ev) {
  if (rows <= 0 || rows % 128 != 0 || dev.ch.D % 4 != 0) return hipErrorInvalidValue;
  launch(k_chain_final, dim3(rows), dim3(256), st, ev, dev, reqs, n_reqs);
  return hipGetLastError();
}

hipError_t launch_chain_gemm(const Dev &dev, const StepReq *reqs, int n_reqs, int rows, int kind, int layer,
                             int few, hipStream_t st, LaunchEv ev) {
  const ChainDev &c = dev.ch;
  const Dims &dm = dev.dm;
  if (rows <= 0 || rows % GBM != 0 || layer < 0 || layer >= dm.L) return hipErrorInvalidValue;
  const size_t D = c.D, I = c.I, Dq = (size_t)dm.Hq * dm.d, Dkv = (size_t)dm.Hkv * dm.d;
  GemmArgs g{};
  g.layer = layer;
  int epi;
  if (kind == kChainQKV) {
    epi = EPI_QKV;
    g.A = c.xn;
    g.W0 = c.wq + layer * Dq * D;
    g.W1 = c.wk + layer * Dkv * D;
    g.W2 = c.wv + layer * Dkv * D;
    g.n1 = (int)Dq;
    g.n2 = (int)(Dq + Dkv);
    g.N = (int)(Dq + 2 * Dkv);
    g.K = (int)D;
    g.out = c.q;
  } else if (kind == kChainO) {
    epi = EPI_RESID;
    g.A = c.o;
    g.W0 = c.wo + layer * D * Dq;
    g.N = (int)D;
    g.K = (int)Dq;
    g.x = c.x;
  } else if (kind == kChainGateUp) {
    epi = EPI_SWIGLU;
    g.A = c.xn;
    g.W0 = c.wg + layer * I * D;
    g.W1 = c.wu + layer * I * D;
    g.N = (int)(2 * I);
    g.K = (int)D;
    g.out = c.act;
  } else if (kind == kChainDown) {
    epi = EPI_RESID;
    g.A = c.act;
    g.W0 = c.wd + layer * D * I;
    g.N = (int)D;
    g.K = (int)I;
    g.x = c.x;
  } else {
    return hipErrorInvalidValue;
  }
  if (g.K % GBK != 0) return hipErrorInvalidValue;
  // one live row per request, at most kGemvRows requests: the rows alone, each weight streamed
  // once (a first-level step's q/k/v projection computes q only: its k and v are never stored)
  if (few > 0 && n_reqs <= kGemvRows && (g.K == 2048 || g.K == 6144)) {
    const int units = epi == EPI_SWIGLU ? g.N / 2 : (epi == EPI_QKV && few == 2 ? g.n1 : g.N);
    const dim3 grid((unsigned)((units + kGemvWaves - 1) / kGemvWaves)), blk(64 * kGemvWaves);
    auto go = [&](auto kl) {
      constexpr int KL = decltype(kl)::value;
      if (epi == EPI_QKV) launch(k_gemv<EPI_QKV, KL>, grid, blk, st, ev, dev, reqs, n_reqs, g, units);
      else if (epi == EPI_RESID) launch(k_gemv<EPI_RESID, KL>, grid, blk, st, ev, dev, reqs, n_reqs, g, units);
      else launch(k_gemv<EPI_SWIGLU, KL>, grid, blk, st, ev, dev, reqs, n_reqs, g, units);
    };
    if (g.K == 2048) go(std::integral_constant<int, 4>{});
    else go(std::integral_constant<int, 12>{});
    return hipGetLastError();
  }
  // 256 weight rows per tile where the q / k / v (or gate / up) ranges allow it and the tiles
  // still fill the chip, else 128
  const int m_tiles = rows / GBM;
  const bool wide = g.N % 256 == 0 && (epi != EPI_QKV || (g.n1 % 256 == 0 && (g.n2 - g.n1) % 256 == 0)) &&
                    (long)m_tiles * (g.N / 256) >= 256;
  if (!wide && g.N % 128 != 0) return hipErrorInvalidValue;
  const int tiles = m_tiles * (g.N / (wide ? 256 : 128));
  // few rows (the first level: one beam per request): the tiles alone leave most compute units
  // without a weight stream, so K is split into up to 8 ranges (at least 4 stages each) whose
  // partial sums a second launch adds in order (deterministic) before the epilogue
  g.ksplit = 1;
  const int KT = g.K / GBK;
  while (g.ksplit < kMaxKSplit && tiles * g.ksplit < 256 && KT % (2 * g.ksplit) == 0 && KT / (2 * g.ksplit) >= 4 &&
         (size_t)2 * g.ksplit * rows * g.N <= c.part_floats)
    g.ksplit *= 2;
  g.part = c.part;
  const dim3 grid((unsigned)(tiles * g.ksplit));
  const LaunchEv e1{ev.start, g.ksplit > 1 ? nullptr : ev.stop};
  auto go = [&](auto wn, auto nwn) {
    constexpr int WN = decltype(wn)::value, NWN = decltype(nwn)::value;
    const dim3 blk(128 * NWN);
    if (epi == EPI_QKV) launch(k_gemm<EPI_QKV, WN, NWN>, grid, blk, st, e1, dev, reqs, n_reqs, g, m_tiles);
    else if (epi == EPI_RESID) launch(k_gemm<EPI_RESID, WN, NWN>, grid, blk, st, e1, dev, reqs, n_reqs, g, m_tiles);
    else launch(k_gemm<EPI_SWIGLU, WN, NWN>, grid, blk, st, e1, dev, reqs, n_reqs, g, m_tiles);
  };
  if (wide) go(std::integral_constant<int, 256 / kWideNWN>{}, std::integral_constant<int, kWideNWN>{});
  else go(std::integral_constant<int, 64>{}, std::integral_constant<int, 2>{});
  if (g.ksplit > 1) {
    const LaunchEv e2{nullptr, ev.stop};
    const int ncols = epi == EPI_SWIGLU ? g.N / 2 : g.N;
    const dim3 rgrid((unsigned)n_reqs, (unsigned)((ncols + 1023) / 1024));
    if (epi == EPI_QKV) launch(k_gemm_reduce<EPI_QKV>, rgrid, dim3(256), st, e2, dev, reqs, g, rows);
    else if (epi == EPI_RESID) launch(k_gemm_reduce<EPI_RESID>, rgrid, dim3(256), st, e2, dev, reqs, g, rows);
    else launch(k_gemm_reduce<EPI_SWIGLU>, rgrid, dim3(256), st, e2, dev, reqs, g, rows);
  }
  return hipGetLastError();
}

}  // namespace gr
