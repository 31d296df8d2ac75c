// Sustained rates of the gfx950 units the decode kernels lean on, as measured ceilings next to
// the published peaks: dense bf16 and f16 MFMA (v_mfma_f32_32x32x16_*: 32,768 flop each) with no
// memory traffic, the vector ALU's fp32 FMA and exp2 (v_exp_f32) rates, and HBM read bandwidth
// (one pass over a 164 MiB buffer, the size of one headline layer's K and V, and over 1 GiB),
// LDS read bandwidth, and MFMA fed by one LDS read per instruction (the attention loop's
// operand path).
// The ALU loops run `iters` iterations of independent operations on registers and write one
// float per thread; the read pass sums 16-byte loads and writes one word per thread.  Prints
// one JSON object.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

enum { kMfmaBf16 = 0, kMfmaF16 = 1, kFma = 2, kExp = 3 };
constexpr int kAcc = 8;  // independent accumulators per wave

template <int MODE>
__global__ __launch_bounds__(256) void k_rate(float *out, int iters, float seed) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(threadIdx.x + i) * 1e-3f;
  f32x16_t acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x16_t{};
  bf16x8_t a, b;
  f16x8_t ah, bh;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x[i] * 1e-3f);
    b[i] = (__bf16)(x[i + 8] * 1e-3f);
    ah[i] = (_Float16)(x[i] * 1e-3f);
    bh[i] = (_Float16)(x[i + 8] * 1e-3f);
  }
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == kMfmaBf16) {
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    } else if constexpr (MODE == kMfmaF16) {
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[j], 0, 0, 0);
    } else if constexpr (MODE == kFma) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
    } else {
      // exp2 of a bounded argument (the iteration converges to a fixed point near -0.4)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * -0.5f;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// every thread sums its grid-stride share of n 16-byte words, U loads in flight
template <int U>
__global__ __launch_bounds__(256) void k_read(const u32x4_t *p, size_t n, unsigned *out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, nt = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  size_t i = tid;
  for (; i + (U - 1) * nt < n; i += U * nt) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * nt);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += nt) {
    const u32x4_t v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[tid] = acc;
}

// LDS read bandwidth: 8 waves per workgroup, one workgroup per compute unit; each wave reads
// 1 KB per ds_read_b128 (64 lanes x 16 consecutive bytes, no bank conflicts) from a 64 KB
// buffer, 8 reads per iteration (8 consecutive 1 KB rows, immediate offsets), and folds the
// words with three-input adds (two VALU instructions per read).
__global__ __launch_bounds__(512) void k_lds_read(unsigned *out, int iters) {
  __shared__ u32x4_t buf[4096];
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = u32x4_t{(unsigned)i, (unsigned)i + 1, 7u, 9u};
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned a0 = 0, a1 = 0;
  for (int it = 0; it < iters; ++it) {
    const u32x4_t *row = buf + ((it + w) & 7) * 512 + lane;  // 8 rows of 1 KB, immediate offsets
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = row[u * 64];  // all 8 reads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 = a0 + v[u][0] + v[u][1];  // v_add3_u32
      a1 = a1 + v[u][2] + v[u][3];
    }
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = a0 ^ a1;
}

// The context-attention loop's shape: each v_mfma_f32_32x32x16_bf16 takes its A operand from
// one ds_read_b128 (1 KB per wave), B from registers; 8 waves per workgroup (2 per SIMD), one
// workgroup per compute unit, 4 accumulators per wave.
__global__ __launch_bounds__(512) void k_mfma_lds(float *out, int iters) {
  __shared__ u32x4_t buf[4096];
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) buf[i] = u32x4_t{0x3c003c00u, 0x3b003b00u, 0x3c003c00u, 0x3a003a00u};
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bf16x8_t b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)((float)(lane + i) * 1e-4f);
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16_t{};
  // software-pipelined: the next iteration's 8 operand reads are in flight during this one's MFMAs
  u32x4_t cur[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) cur[u] = buf[(w & 7) * 512 + lane + u * 64];
  for (int it = 0; it < iters; ++it) {
    const u32x4_t *row = buf + ((it + 1 + w) & 7) * 512 + lane;
    u32x4_t nxt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) nxt[u] = row[u * 64];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cur[u]), b, acc[u & 3], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

bool ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "rate_probe: %s: %s\n", what, hipGetErrorString(e));
    return false;
  }
  return true;
}

}  // namespace

int main(int argc, char **argv) {
  // 1024 workgroups of 4 waves: 4 waves per SIMD on 256 compute units
  const int grid = 1024, block = 256, iters = argc > 1 ? atoi(argv[1]) : 8192;
  if (iters <= 0) return 2;
  float *out = nullptr;
  hipEvent_t e0, e1;
  if (!ok(hipMalloc(&out, sizeof(float) * grid * block), "hipMalloc") || !ok(hipEventCreate(&e0), "event") ||
      !ok(hipEventCreate(&e1), "event"))
    return 1;
  double rate[4];
  for (int mode = 0; mode < 4; ++mode) {
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      if (!ok(hipEventRecord(e0), "record")) return 1;
      if (mode == kMfmaBf16) k_rate<kMfmaBf16><<<grid, block>>>(out, iters, 1.f);
      if (mode == kMfmaF16) k_rate<kMfmaF16><<<grid, block>>>(out, iters, 1.f);
      if (mode == kFma) k_rate<kFma><<<grid, block>>>(out, iters, 1.f);
      if (mode == kExp) k_rate<kExp><<<grid, block>>>(out, iters, 1.f);
      if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
          !ok(hipEventSynchronize(e1), "sync"))
        return 1;
      float ms = 0.f;
      if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
      if (rep > 0 && ms < best) best = ms;  // the first run warms up
    }
    const double threads = (double)grid * block, sec = best * 1e-3;
    if (mode <= kMfmaF16)
      rate[mode] = threads / 64 * iters * kAcc * 32768.0 / sec / 1e12;  // TFLOP/s
    else
      rate[mode] = threads / 64 * iters * 16 / sec / 1e9;  // wave instructions per ns (x64 lanes)
  }
  // LDS: 256 workgroups of 512 threads (one per compute unit), best of 2 after a warm-up
  double lds_tbs = 0, mfma_lds = 0;
  {
    const int lgrid = 256, lblock = 512, liters = iters / 4;
    for (int mode = 0; mode < 2; ++mode) {
      float best = 1e30f;
      for (int rep = 0; rep < 3; ++rep) {
        if (!ok(hipEventRecord(e0), "record")) return 1;
        if (mode == 0) k_lds_read<<<lgrid, lblock>>>(reinterpret_cast<unsigned *>(out), liters);
        if (mode == 1) k_mfma_lds<<<lgrid, lblock>>>(out, liters);
        if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
            !ok(hipEventSynchronize(e1), "sync"))
          return 1;
        float ms = 0.f;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
        if (rep > 0 && ms < best) best = ms;
      }
      const double waves = (double)lgrid * lblock / 64, sec = best * 1e-3;
      if (mode == 0) lds_tbs = waves * liters * 8 * 1024.0 / sec / 1e12;
      else mfma_lds = waves * liters * 8 * 32768.0 / sec / 1e12;
    }
  }
  // HBM reads: 4096 workgroups of 256 threads, best of 4 passes after a warm-up pass
  const size_t rbytes[2] = {(size_t)164 << 20, (size_t)1 << 30};
  const int rgrid = 4096;
  u32x4_t *buf = nullptr;
  unsigned *rout = nullptr;
  if (!ok(hipMalloc(&buf, rbytes[1]), "hipMalloc") || !ok(hipMemset(buf, 1, rbytes[1]), "hipMemset") ||
      !ok(hipMalloc(&rout, sizeof(unsigned) * rgrid * 256), "hipMalloc"))
    return 1;
  double tbs[2];
  for (int b = 0; b < 2; ++b) {
    float best = 1e30f;
    for (int rep = 0; rep < 5; ++rep) {
      if (!ok(hipEventRecord(e0), "record")) return 1;
      k_read<8><<<rgrid, 256>>>(buf, rbytes[b] / 16, rout);
      if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
          !ok(hipEventSynchronize(e1), "sync"))
        return 1;
      float ms = 0.f;
      if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
      if (rep > 0 && ms < best) best = ms;
    }
    tbs[b] = rbytes[b] / (best * 1e-3) / 1e12;
  }
  printf("{\"mfma_bf16_TFLOPs\": %.1f, \"mfma_f16_TFLOPs\": %.1f, \"fma_f32_wave_instr_per_ns\": %.2f, "
         "\"exp2_f32_wave_instr_per_ns\": %.2f, \"fma_f32_TFLOPs\": %.1f, \"iters\": %d, "
         "\"hbm_read_164MiB_TBs\": %.2f, \"hbm_read_1GiB_TBs\": %.2f, \"lds_read_TBs\": %.1f, "
         "\"mfma_bf16_lds_operand_TFLOPs\": %.1f}\n",
         rate[0], rate[1], rate[2], rate[3], rate[2] * 64 * 2 / 1e3, iters, tbs[0], tbs[1], lds_tbs, mfma_lds);
  hipFree(rout);
  hipFree(buf);
  hipFree(out);
  return 0;
}
