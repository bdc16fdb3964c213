// Fused attention forward on quantized inputs for gfx950.
//
// Source: diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention
// backend: aiter package or Hub kernel?", problem statement: INT8 QK^T and
// FP8 PV with FP32 accumulation, bf16 [B, S, H, 128], no mask, non-causal.
// The online (flash-style) softmax streams key tiles; P is quantized to FP8
// E4M3FN with the fixed scale 448 (the largest E4M3FN value), folded into the
// exponent of exp2.
//
// The INT8 score accumulators start at 0x4B400000, the bit pattern of the
// fp32 value 1.5 * 2^23: since |A| < 2^21, the accumulated integer
// 0x4B400000 + A is the bit pattern of the exact fp32 value 1.5 * 2^23 + A,
// so the scores are read as floats without a conversion instruction, and
// integer order of the biased values is still score order.
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
// (row / 2) % 8: a 16-byte read is served for 16 lanes at a time from 64
// four-byte banks, and the 16 rows a lane group reads then cover all 256
// bytes of the banks exactly once.
#pragma once

#include "sage_common.hpp"

namespace sage {

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_key(row)) << 4); }

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
// sacc[u] covers keys [32 u, 32 u + 32) of the tile; every accumulator
// starts from `init`.
__device__ __forceinline__ void qk_tile(const uint8_t* __restrict__ lds_k, const v4i qf[4], int li, int g,
                                        const v16i& init, v16i sacc[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v16i acc = init;
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

// Asynchronous copy of one 128-row x 128-byte tile into swizzled LDS with
// global_load_lds_dwordx4: each wave instruction writes 1 KB (8 rows)
// contiguously, lane l at +16 l, so the swizzle is applied by choosing each
// lane's source chunk. kWaves waves split the 16 row groups.
template <int kWaves>
__device__ __forceinline__ void stage_tile_async(uint8_t* lds, const uint8_t* __restrict__ src, int64_t row_stride,
                                                 int wave, int lane) {
  const int rr = lane >> 3, cp = lane & 7;
#pragma unroll
  for (int i = 0; i < 16 / kWaves; ++i) {
    const int grp = wave + kWaves * i;
    const int row = 8 * grp + rr;
    const uint8_t* g = src + row * row_stride + ((cp ^ swz_key(row)) << 4);
    __builtin_amdgcn_global_load_lds((const void*)g,
                                     (__attribute__((address_space(3))) void*)(lds + grp * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ int imax3(int a, int b, int c) { return max(max(a, b), c); }

// Largest of the 16 scores a lane holds for one sub-tile.
__device__ __forceinline__ int max16(const v16i& s) {
  int a = imax3(s[0], s[1], s[2]);
  int b = imax3(s[3], s[4], s[5]);
  a = imax3(a, s[6], s[7]);
  b = imax3(b, s[8], s[9]);
  a = imax3(a, s[10], s[11]);
  b = imax3(b, s[12], s[13]);
  a = imax3(a, s[14], s[15]);
  return max(a, b);
}

// max / sum of a value over lanes l and l^32 (the two halves hold the same
// query rows), with one v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int kScoreBias = 0x4B400000;        // bits of 1.5 * 2^23
constexpr float kScoreBiasF = 12582912.0f;     // 1.5 * 2^23

// P' = 2^(A f - m2) for the 64 scores of a lane, their fp32 sum, and the
// E4M3FN codes packed in the FP8 MFMA B-operand order (byte 16 (u%2) + r of
// pop[u/2] holds sub-tile u, register r). With X = 1.5 * 2^23 + A (the biased
// accumulator read as a float) the exponent is fl32(X f - nc[u]) with
// nc[u] = fl32(fl32(1.5 * 2^23 * f) + m2), one fused multiply-add.
// kClamp: saturate before the conversion (the hardware conversion gives NaN
// above 464). kTail: keys at or past `nvalid` get P' = 0.
template <bool kClamp, bool kTail>
__device__ __forceinline__ float softmax_p(const v16i s[4], const float f[4], const float nc[4], int nvalid,
                                           int g, v8i pop[2]) {
  float lsum = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * j + e;
        float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(__int_as_float(s[u][r]), f[u], -nc[u]));
        if (kTail && key_of(u, r, g) >= nvalid) pe = 0.0f;
        lsum += pe;
        p[e] = kClamp ? fminf(pe, 448.0f) : pe;
      }
      // the first conversion's "old" operand only supplies the upper half,
      // which the second conversion overwrites
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
      pop[u >> 1][4 * (u & 1) + j] = wd;
    }
  }
  return lsum;
}

struct RowState {
  float m, m2, l;
};

// One key tile for one wave: QK^T, online softmax, PV.
template <bool kTail>
__device__ __forceinline__ void attn_tile(const uint8_t* lk, const uint8_t* lv, const v4i qf[4], const v16i& bias,
                                          float qs,
                                          const float* __restrict__ ks4, float c, float log2_448, int nvalid,
                                          int li, int g, RowState& st, v16f o[4]) {
  v16i s[4];
  qk_tile(lk, qf, li, g, bias, s);
  float f[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) f[u] = (qs * ks4[u]) * c;

  // t = fl32(A f) is monotone in A for f >= 0, so the tile max is taken on
  // the (biased) integers of each 32-key block and dequantized once.
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (kTail) {
      if (32 * u >= nvalid) continue;
      v16i sm = s[u];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key_of(u, r, g) >= nvalid) sm[r] = INT32_MIN;
      const int mx = max16(sm);
      if (mx != INT32_MIN) tmax = fmaxf(tmax, (float)(mx - kScoreBias) * f[u]);
    } else {
      tmax = fmaxf(tmax, (float)(max16(s[u]) - kScoreBias) * f[u]);
    }
  }
  tmax = pair_max(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float m2_new = m_new - log2_448;
  const float alpha = __builtin_amdgcn_exp2f(st.m2 - m2_new);
  float nc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) nc[u] = kScoreBiasF * f[u] + m2_new;
  v8i pop[2];
  float lsum;
  // P' of the largest score is 448 * 2^e, where e collects the fp32
  // roundings of m, m2, 1.5 * 2^23 * f and nc. While all of those stay below
  // 2^17 in magnitude each rounding is at most 2^-7 and P' <= 448 * 2^(1/32)
  // < 464, the limit of the conversion (above it the hardware gives NaN).
  // Larger values (outlier-scale Q/K blocks) take the saturating variant.
  float mag = fabsf(m_new);
#pragma unroll
  for (int u = 0; u < 4; ++u) mag = fmaxf(mag, fabsf(nc[u]));
  if (__builtin_expect(__ballot(mag >= 131072.0f) != 0, 0))
    lsum = softmax_p<true, kTail>(s, f, nc, nvalid, g, pop);
  else
    lsum = softmax_p<false, kTail>(s, f, nc, nvalid, g, pop);
  st.l = st.l * alpha + lsum;
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) o[cb] *= alpha;
  }
  st.m = m_new;
  st.m2 = m2_new;

#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = 32 * cb + li;
      const v4i lo = *(const v4i*)(lv + swz(row, 4 * w + 2 * g));
      const v4i hi = *(const v4i*)(lv + swz(row, 4 * w + 2 * g + 1));
      const v8i vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop[w], o[cb], 0, 0, 0, 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const int8_t* __restrict__ q8, const float* __restrict__ qscale,
                     const int8_t* __restrict__ k8, const float* __restrict__ kscale,
                     const uint8_t* __restrict__ v8t, const float* __restrict__ vscale, int S, int H,
                     int S_pad, int nqt, int num_wg, float c, float log2_448,
                     uint16_t* __restrict__ out) {
  // two stages of (K tile, V^T tile), 16 KB each
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][kKeyTile * 128];

  const int wg = xcd_remap(blockIdx.x, num_wg);
  const int qt = wg % nqt;
  const int64_t bh = wg / nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int q0 = qt * kQueryTile + wave * 32;
  const int nbp = S_pad / kQBlock;

  const uint8_t* kbase = (const uint8_t*)k8 + bh * S_pad * kHeadDim;
  const uint8_t* vbase = v8t + bh * kHeadDim * (int64_t)S_pad;
  const float* ksb = kscale + bh * nbp;
  const int ntiles = (S + kKeyTile - 1) / kKeyTile;
  const int nfull = S / kKeyTile;   // tiles with no masked key

  stage_tile_async<kAttnWaves>(lds[0][0], kbase, kHeadDim, wave, lane);
  stage_tile_async<kAttnWaves>(lds[0][1], vbase, S_pad, wave, lane);

  v4i qf[4];
  load_q_frag(q8 + ((bh * S_pad + q0 + li) * kHeadDim + 64 * g), qf);
  const float qs = qscale[bh * nbp + q0 / kQBlock];

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kScoreBias;
  RowState st{-INFINITY, -INFINITY, 0.0f};
  v16f o[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) o[cb] = (v16f){0};

  // Full tiles: tile kt+1 streams into the other LDS stage while tile kt is
  // computed; one barrier per tile.
  for (int kt = 0; kt < nfull; ++kt) {
    const int k0 = kt * kKeyTile;
    const int buf = kt & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kt + 1 < ntiles) {
      stage_tile_async<kAttnWaves>(lds[buf ^ 1][0], kbase + (int64_t)(k0 + kKeyTile) * kHeadDim, kHeadDim, wave, lane);
      stage_tile_async<kAttnWaves>(lds[buf ^ 1][1], vbase + k0 + kKeyTile, S_pad, wave, lane);
    }
    attn_tile<false>(lds[buf][0], lds[buf][1], qf, bias, qs, ksb + k0 / kQBlock, c, log2_448, kKeyTile, li, g, st, o);
  }
  // The last tile when S is not a multiple of the tile: keys >= S masked.
  if (nfull < ntiles) {
    const int k0 = nfull * kKeyTile;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    attn_tile<true>(lds[nfull & 1][0], lds[nfull & 1][1], qf, bias, qs, ksb + k0 / kQBlock, c, log2_448, S - k0, li, g,
                    st, o);
  }

  // Epilogue: O = acc * v_scale / l, bf16, layout [B, S, H, D].
  const float lt = pair_sum(st.l);
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
// grid (key tiles, query tiles of kDebugRows = 128), 256 threads.
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ q8,
                                                       const int8_t* __restrict__ k8, int S_pad,
                                                       int64_t bh, int rA, int r0, int nr, int cA,
                                                       int c0, int nc, int32_t* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kKeyTile * 128];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int k0 = cA + blockIdx.x * kKeyTile;
  const int qa = rA + blockIdx.y * kDebugRows + wave * 32;
  stage_tile(lds_k, (const uint8_t*)k8 + (bh * S_pad + k0) * kHeadDim, kHeadDim, tid);
  __syncthreads();
  if (qa >= S_pad) return;
  v4i qf[4];
  load_q_frag(q8 + ((bh * S_pad + qa + li) * kHeadDim + 64 * g), qf);
  v16i sacc[4];
  const v16i zero = {0};
  qk_tile(lds_k, qf, li, g, zero, sacc);
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
