// Shared device definitions for the gfx950 quantized attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int kHeadDim = 128;     // the pages' head size (64 is also supported)
constexpr int kQBlock = 32;       // Q/K quantization block (rows)
constexpr int kSeqAlign = 256;    // padding of the quantized layouts
constexpr int kKeyTile = 128;     // BN: keys per online-softmax tile
constexpr int kAttnWaves = 8;     // waves per attention workgroup
constexpr int kQueryTile = 32 * kAttnWaves;     // BM: queries per workgroup
constexpr int kVGroup = 64;       // keys per permuted group of the V^T layout
constexpr int kVChunkRows = 512;  // minimum rows per partial-amax chunk of V

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Slot p (0..63) of a permuted 64-key group holds key kappa(p):
//   p = 32 g + 16 u + r  ->  kappa = 32 u + 8 (r/4) + 4 g + (r%4).
// This is the key order in which the 32x32x32 INT8 MFMA leaves scores in a
// lane (query = lane%32, lane group g = lane/32, accumulator register r of
// sub-tile u), so P can feed the FP8 MFMA straight from registers.
__host__ __device__ __forceinline__ int vslot_of_key(int kappa) {
  int u = kappa >> 5, rem = kappa & 31;
  int r = ((rem >> 3) << 2) | (rem & 3);
  int g = (rem >> 2) & 1;
  return (g << 5) | (u << 4) | r;
}

// 64-lane max of a float (all lanes receive the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Workgroup index remap so that consecutive logical tiles land on the same
// XCD: hardware dispatches workgroup i to XCD i % 8.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int nx = 8;
  int per = n / nx, rem = n % nx;
  int x = i % nx, local = i / nx;
  return x < rem ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

}  // namespace sage
