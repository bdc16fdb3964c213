// Fused attention forward on quantized inputs for gfx950.
//
// Source: diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention
// backend: aiter package or Hub kernel?", problem statement: INT8 QK^T and
// FP8 PV with FP32 accumulation, bf16 [B, S, H, 128], no mask, non-causal.
// The online (flash-style) softmax streams key tiles; P is quantized to FP8
// E4M3FN with the fixed scale 448 (the largest E4M3FN value), folded into the
// exponent of exp2.
//
// Work decomposition: one workgroup = 4 waves = 128 queries of one (b, h);
// each wave owns 32 queries and streams all keys in tiles of 128.
//   QK:  S^T[key][query] = K . Q^T with v_mfma_i32_32x32x32_i8 (A = K rows
//        from LDS, B = the wave's Q rows kept in VGPRs). Lane l then holds
//        query l%32 and keys 8 (r/4) + 4 (l/32) + r%4 of each 32-key
//        sub-tile, so row max / row sum are in-lane plus one swap with lane
//        l^32, and one 32-key sub-tile is exactly one K quantization block
//        (one dequantization factor per sub-tile, uniform over the wave).
//   PV:  O^T[channel][query] += V^T . P^T with v_mfma_f32_32x32x64_f8f6f4
//        (A = V^T rows from LDS, B = P straight from registers). The V^T
//        layout stores keys in the order the score accumulator leaves them,
//        so no shuffles are needed between the two products.
// LDS tiles are rows of 128 bytes whose 16-byte chunks are XOR-swizzled by
// the row index, so the 64 lanes' 16-byte reads hit distinct banks.
#pragma once

#include "sage_common.hpp"

namespace sage {

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// Cooperative copy of one 128-row x 128-byte tile (rows `row_stride` bytes
// apart in global memory) into swizzled LDS. 256 threads, 4 x 16 B each.
__device__ __forceinline__ void stage_tile(uint8_t* __restrict__ lds, const uint8_t* __restrict__ src,
                                           int64_t row_stride, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + 256 * it;
    const int row = idx >> 3, ch = idx & 7;
    const uint4 w = *(const uint4*)(src + row * row_stride + ch * 16);
    *(uint4*)(lds + swz(row, ch)) = w;
  }
}

// The wave's Q fragment: lane l holds bytes [64 g, 64 g + 64) of query row
// l%32 (g = l/32); step s of the 128-deep contraction uses 16 of them. K
// operands use the same byte mapping, so the products pair matching dims.
__device__ __forceinline__ void load_q_frag(const int8_t* __restrict__ qrow, v4i qf[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = *(const v4i*)(qrow + 16 * s);
}

// S^T for the 128 keys of the staged tile against the wave's 32 queries:
// sacc[u] covers keys [32 u, 32 u + 32) of the tile.
__device__ __forceinline__ void qk_tile(const uint8_t* __restrict__ lds_k, const v4i qf[4], int li, int g,
                                        v16i sacc[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v16i acc = {0};
    const int row = 32 * u + li;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i kop = *(const v4i*)(lds_k + swz(row, 4 * g + s));
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qf[s], acc, 0, 0, 0);
    }
    sacc[u] = acc;
  }
}

__device__ __forceinline__ int key_of(int u, int r, int g) { return 32 * u + 8 * (r >> 2) + 4 * g + (r & 3); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const int8_t* __restrict__ q8, const float* __restrict__ qscale,
                     const int8_t* __restrict__ k8, const float* __restrict__ kscale,
                     const uint8_t* __restrict__ v8t, const float* __restrict__ vscale, int S, int H,
                     int S_pad, int nqt, int num_wg, float c, float log2_448,
                     uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kKeyTile * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kHeadDim * kKeyTile];

  const int wg = xcd_remap(blockIdx.x, num_wg);
  const int qt = wg % nqt;
  const int64_t bh = wg / nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q0 = qt * kQueryTile + wave * 32;
  const int nbp = S_pad / kQBlock;

  v4i qf[4];
  load_q_frag(q8 + ((bh * S_pad + q0 + li) * kHeadDim + 64 * g), qf);
  const float qs = qscale[bh * nbp + q0 / kQBlock];

  const uint8_t* kbase = (const uint8_t*)k8 + bh * S_pad * kHeadDim;
  const uint8_t* vbase = v8t + bh * kHeadDim * (int64_t)S_pad;
  const float* ksb = kscale + bh * nbp;

  float m = -INFINITY, m2 = -INFINITY, l = 0.0f;
  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) o[cb] = (v16f){0};

  const int ntiles = (S + kKeyTile - 1) / kKeyTile;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * kKeyTile;
    __syncthreads();
    stage_tile(lds_k, kbase + (int64_t)k0 * kHeadDim, kHeadDim, tid);
    stage_tile(lds_v, vbase + k0, S_pad, tid);
    __syncthreads();

    v16i sacc[4];
    qk_tile(lds_k, qf, li, g, sacc);

    float f[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) f[u] = (qs * ksb[k0 / kQBlock + u]) * c;

    const int nvalid = S - k0;
    const bool tail = nvalid < kKeyTile;
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (tail && 32 * u >= nvalid) continue;
      int mx = INT32_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int a = sacc[u][r];
        if (tail && key_of(u, r, g) >= nvalid) a = INT32_MIN;
        mx = max(mx, a);
      }
      tmax = fmaxf(tmax, (float)mx * f[u]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m, tmax);
    const float m2_new = m_new - log2_448;
    const float alpha = __builtin_amdgcn_exp2f(m2 - m2_new);
    // Scores beyond 2^19 (log2 units) make the fp32 spacing of m coarse
    // enough for P' to pass 464, where the conversion would give NaN.
    const bool big = __ballot(m_new > 524288.0f) != 0;

    float lsum = 0.0f;
    v8i pop[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j + e;
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sacc[u][r], f[u], -m2_new));
          if (tail && key_of(u, r, g) >= nvalid) pe = 0.0f;
          lsum += pe;
          p[e] = big ? fminf(pe, 448.0f) : pe;
        }
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
        pop[u >> 1][4 * (u & 1) + j] = wd;
      }
    }
    l = l * alpha + lsum;
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) o[cb] *= alpha;
    }

#pragma unroll
    for (int w = 0; w < 2; ++w) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int row = 32 * cb + li;
        const v4i lo = *(const v4i*)(lds_v + swz(row, 4 * w + 2 * g));
        const v4i hi = *(const v4i*)(lds_v + swz(row, 4 * w + 2 * g + 1));
        const v8i vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop[w], o[cb], 0, 0, 0, 0, 0, 0);
      }
    }
    m = m_new;
    m2 = m2_new;
  }

  // Epilogue: O = acc * v_scale / l, bf16, layout [B, S, H, D].
  const float lt = l + __shfl_xor(l, 32, 64);
  const float rl = __fdiv_rn(1.0f, lt);
  const int qi = q0 + li;
  if (qi < S) {
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    uint16_t* orow = out + ((b * S + qi) * H + h) * kHeadDim;
    const float* vsb = vscale + bh * kHeadDim;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c0 = 32 * cb + 8 * rg + 4 * g;
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bits[e] = f32_to_bf16_rne((o[cb][4 * rg + e] * vsb[c0 + e]) * rl);
        *(uint2*)(orow + c0) = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
      }
    }
  }
}

// Debug dump of int32 scores through the same staging and MFMA path.
// grid (key tiles, query tiles of 128), 256 threads.
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ q8,
                                                       const int8_t* __restrict__ k8, int S_pad,
                                                       int64_t bh, int rA, int r0, int nr, int cA,
                                                       int c0, int nc, int32_t* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kKeyTile * 128];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int k0 = cA + blockIdx.x * kKeyTile;
  const int qa = rA + blockIdx.y * kQueryTile + wave * 32;
  stage_tile(lds_k, (const uint8_t*)k8 + (bh * S_pad + k0) * kHeadDim, kHeadDim, tid);
  __syncthreads();
  if (qa >= S_pad) return;
  v4i qf[4];
  load_q_frag(q8 + ((bh * S_pad + qa + li) * kHeadDim + 64 * g), qf);
  v16i sacc[4];
  qk_tile(lds_k, qf, li, g, sacc);
  const int row = qa + li;
  if (row < r0 || row >= r0 + nr) return;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + key_of(u, r, g);
      if (key >= c0 && key < c0 + nc) scores[(int64_t)(row - r0) * nc + (key - c0)] = sacc[u][r];
    }
}

}  // namespace sage
