// Seeded synthetic inputs generated on the device: the same values as the host generators.
//
// A bf16 block is a Philox4x64-10 counter stream (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011, the Philox section) as numpy's Philox bit
// generator produces it: block b (four 64-bit words) is the bijection applied to counter
// b + 1 under the block's 128-bit key; the words are read little-endian as 16-bit indices
// into a table of 65536 bf16 values.  Test-input plumbing only: none of the decode step's
// arithmetic is here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;  // round multipliers
constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;  // key increments

// One thread per block of 16 values.
__global__ __launch_bounds__(256) void k_bf16_normal(uint64_t key0, uint64_t key1, uint64_t n_values,
                                                     const uint16_t *__restrict__ table,
                                                     uint16_t *__restrict__ out) {
  const uint64_t n_blocks = (n_values + 15) / 16;
  for (uint64_t b = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < n_blocks;
       b += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t x0 = b + 1, x1 = 0, x2 = 0, x3 = 0, k0 = key0, k1 = key1;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      if (r) {
        k0 += kW0;
        k1 += kW1;
      }
      const uint64_t hi0 = __umul64hi(kM0, x0), lo0 = kM0 * x0;
      const uint64_t hi1 = __umul64hi(kM1, x2), lo1 = kM1 * x2;
      const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
      x0 = y0;
      x1 = lo1;
      x2 = y2;
      x3 = lo0;
    }
    const uint64_t w[4] = {x0, x1, x2, x3};
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t word = w[i >> 1];
      const uint32_t lo = table[(word >> (32 * (i & 1))) & 0xFFFF];
      const uint32_t hi = table[(word >> (32 * (i & 1) + 16)) & 0xFFFF];
      v[i] = lo | (hi << 16);
    }
    const uint64_t base = 16 * b;
    if (base + 16 <= n_values && (((uintptr_t)(out + base)) & 15) == 0) {
      uint4 *o = (uint4 *)(out + base);
      o[0] = make_uint4(v[0], v[1], v[2], v[3]);
      o[1] = make_uint4(v[4], v[5], v[6], v[7]);
    } else {
      for (int i = 0; i < 16 && base + i < n_values; ++i)
        out[base + i] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
    }
  }
}

}  // namespace

// Writes n_values bf16 bit patterns to device memory `out`: value i = table[16-bit piece i of
// the stream of key (key_lo, key_hi)].  `table` is a device array of 65536 entries.  Enqueued
// on `stream` (a hipStream_t; null = the default stream).  Returns 0, or the HIP error code.
extern "C" int synth_bf16_normal(uint64_t key_lo, uint64_t key_hi, uint64_t n_values, const uint16_t *table,
                                 uint16_t *out, void *stream) {
  if (n_values == 0) return 0;
  if (!table || !out) return (int)hipErrorInvalidValue;
  const uint64_t n_blocks = (n_values + 15) / 16;
  const uint64_t wgs = (n_blocks + 255) / 256;
  const unsigned grid = (unsigned)(wgs < 65536 ? wgs : 65536);
  hipLaunchKernelGGL(k_bf16_normal, dim3(grid), dim3(256), 0, (hipStream_t)stream, key_lo, key_hi, n_values, table,
                     out);
  return (int)hipGetLastError();
}
