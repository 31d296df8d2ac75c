// Sustained rates of the gfx950 units the decode kernels lean on, as measured ceilings next to
// the published peaks: dense bf16 and f16 MFMA (v_mfma_f32_32x32x16_*: 32,768 flop each) with no
// memory traffic, the vector ALU's fp32 FMA and exp2 (v_exp_f32) rates, and HBM read bandwidth
// (one pass over a 164 MiB buffer, the size of one headline layer's K and V, and over 1 GiB).
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
         "\"hbm_read_164MiB_TBs\": %.2f, \"hbm_read_1GiB_TBs\": %.2f}\n",
         rate[0], rate[1], rate[2], rate[3], rate[2] * 64 * 2 / 1e3, iters, tbs[0], tbs[1]);
  hipFree(rout);
  hipFree(buf);
  hipFree(out);
  return 0;
}
