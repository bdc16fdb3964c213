// Fused attention forward on quantized inputs for gfx950.
//
// Source: diffusers issue #15014, "gfx1201 (RDNA4) SageAttention attention
// backend: aiter package or Hub kernel?", problem statement: QK^T on INT8
// codes and PV on FP8 codes, both summed in fp32, over bf16 [B, S, H, 128]
// without a mask or causality.
// Also instantiated for head dim 64, and for query and key sequences of
// different lengths, with an optional per-row log-sum-exp.
// The online (flash-style) softmax streams key tiles; P is quantized to FP8
// E4M3FN with the fixed scale 448 (the largest E4M3FN value), folded into the
// exponent of exp2.
//
// The INT8 score accumulators start at 0x4B400000, the bit pattern of the
// fp32 value 1.5 * 2^23: since |A| < 2^21, the accumulated integer
// 0x4B400000 + A is the bit pattern of the exact fp32 value 1.5 * 2^23 + A,
// and integer order of the biased values is still score order. One exact
// fp32 subtraction recovers A as a float (a full-rate instruction, where the
// integer-to-float conversion is half rate); the exponent A * f - m2 is then
// formed with a single rounding (one fused multiply-add).
// The row sum l that normalizes the output is the sum of the decoded FP8 codes
// of P (the weights PV applies), formed by the matrix cores: two more FP8
// MFMAs per key tile with an all-ones A operand.
//
// Work decomposition: one workgroup = 8 waves = 256 queries of one (b, h);
// each wave owns 32 queries and streams all keys in tiles of 128.
//   QK:  S^T[key][query] = K . Q^T with v_mfma_i32_32x32x32_i8 (A = K rows
//        from LDS, B = the wave's Q rows kept in VGPRs). Lane l then holds
//        query l%32 and keys 8 (r/4) + 4 (l/32) + r%4 of each 32-key
//        sub-tile, so the row max is in-lane plus one swap with lane l^32,
//        and one 32-key sub-tile is exactly one K quantization block
//        (one dequantization factor per sub-tile, uniform over the wave).
//   PV:  O^T[channel][query] += V^T . P^T with v_mfma_f32_32x32x64_f8f6f4
//        (A = V^T rows from LDS, B = P straight from registers). The V^T
//        layout stores keys in the order the score accumulator leaves them,
//        so no shuffles are needed between the two products.
//   l:   L^T[row][query] += ONES . P^T with the same MFMA and B operand: every
//        row of L^T is the sum of the query's codes, and lane l holds query
//        l%32 in every register.
// LDS tiles are rows of 128 bytes (64 for K at head dim 64) whose 16-byte
// chunks are XOR-swizzled (swz_key): a 16-byte read is served for 16 lanes
// at a time from 64 four-byte banks, and the 16 rows a lane group reads then
// cover all 256 bytes of the banks exactly once.
#pragma once

#include <type_traits>

#include "sage_common.hpp"

namespace sage {

// Swizzle of LDS tiles with rows of kRB bytes (128 or 64): chunk c of row r
// sits at chunk c ^ key(r). A 16-byte read is served for 16 lanes at a time
// from 64 four-byte banks; 16 consecutive rows read at one logical chunk
// then cover all 256 bytes of the banks exactly once.
template <int kRB>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(kRB == 128 || kRB == 64, "row sizes of the two head dims");
  return kRB == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}
template <int kRB>
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRB + ((chunk ^ swz_key<kRB>(row)) << 4); }

// The wave's Q fragment for head dim kD: lane l holds bytes
// [kD/2 g, kD/2 g + kD/2) of query row l%32 (g = l/32, qrow points there);
// step s of the kD-deep contraction uses 16 of them. K operands use the same
// byte mapping, so the products pair matching dims.
template <int kD>
__device__ __forceinline__ void load_q_frag(const int8_t* __restrict__ qrow, v4i qf[kD / 32]) {
#pragma unroll
  for (int s = 0; s < kD / 32; ++s) qf[s] = *(const v4i*)(qrow + 16 * s);
}

// The same fragment computed from bf16 Q inside the attention kernel: the
// wave's 32 query rows [q0, q0 + 32) are exactly one quantization block, so
// the block's amax is a wave maximum. Arithmetic as quant_qk_kernel (scale =
// fl32(amax/127), codes = clamp(rint(fl32(x * fl32(127/amax))), +-127), rows
// >= Sq count as zeros), hence the same codes and scale bit for bit.
template <int kD>
__device__ __forceinline__ void quant_q_frag(const uint16_t* __restrict__ qraw, int64_t b, int h, int H, int Sq,
                                             int row, int g, v4i qf[kD / 32], float& qs) {
  constexpr int kVals = kD / 2;       // values of the row this lane holds
  float x[kVals];
  if (row < Sq) {
    const uint16_t* src = qraw + ((b * Sq + row) * H + h) * kD + kVals * g;
#pragma unroll
    for (int i = 0; i < kVals / 8; ++i) {
      const uint4 w = *(const uint4*)(src + 8 * i);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = bf16_to_f32(ws[j] & 0xFFFFu);
        x[8 * i + 2 * j + 1] = bf16_to_f32(ws[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kVals; ++i) x[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kVals; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max(amax);
  float scale = 0.0f, inv = 0.0f;
  if (amax > 0.0f) {
    inv = __fdiv_rn(127.0f, amax);
    scale = __fdiv_rn(amax, 127.0f);
    if (!isfinite(inv)) { inv = 0.0f; scale = 0.0f; }
  }
#pragma unroll
  for (int sidx = 0; sidx < kD / 32; ++sidx) {
    int wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = __builtin_rintf(x[16 * sidx + 4 * k + e] * inv);
        y = fminf(fmaxf(y, -127.0f), 127.0f);
        word |= ((uint32_t)((int)y) & 0xFFu) << (8 * e);
      }
      wd[k] = (int)word;
    }
    qf[sidx] = (v4i){wd[0], wd[1], wd[2], wd[3]};
  }
  qs = scale;
}

// S^T for the 128 keys of the staged tile against the wave's 32 queries:
// sacc[u] covers keys [32 u, 32 u + 32) of the tile; every accumulator
// starts from `init` (the score bias).
template <int kD>
__device__ __forceinline__ void qk_tile(const uint8_t* __restrict__ lds_k, const v4i qf[kD / 32], int li, int g,
                                        const v16i& init, v16i sacc[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v16i acc = init;
    const int row = 32 * u + li;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) {
      const v4i kop = *(const v4i*)(lds_k + swz<kD>(row, (kD / 32) * g + s));
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, qf[s], acc, 0, 0, 0);
    }
    sacc[u] = acc;
  }
}

__device__ __forceinline__ int key_of(int u, int r, int g) { return 32 * u + 8 * (r >> 2) + 4 * g + (r & 3); }

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

// max of a value over lanes l and l^32 (the two halves hold the same query
// rows), with one v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kScoreBias = 0x4B400000;        // bits of 1.5 * 2^23
constexpr float kScoreBiasF = 12582912.0f;     // 1.5 * 2^23

// P' = 2^fl32(A f - m2) for the 64 scores of a lane and their E4M3FN codes
// packed in the FP8 MFMA B-operand order (byte 16 (u%2) + r of pop[u/2]
// holds sub-tile u, register r). A is read from the biased accumulator
// X = 1.5 * 2^23 + A as the exact difference X - 1.5 * 2^23; the exponent is
// then one fused multiply-add, i.e. the exact A f - m2 rounded once.
// kClamp: saturate before the conversion (the hardware conversion gives NaN
// above 464). kTail: keys at or past `nvalid` get P' = 0. kDump: also store
// the codes to prow[key] (key within the tile; debug builds of the kernel).
template <bool kClamp, bool kTail, bool kDump = false>
__device__ __forceinline__ void softmax_p(const v16i s[4], const float f[4], float m2, int nvalid, int g,
                                          v8i pop[2], uint8_t* prow = nullptr) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * j + e;
        const float a = __int_as_float(s[u][r]) - kScoreBiasF;   // exact
        float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(a, f[u], -m2));
        if (kTail && key_of(u, r, g) >= nvalid) pe = 0.0f;
        p[e] = kClamp ? fminf(pe, 448.0f) : pe;
      }
      // the first conversion's "old" operand only supplies the upper half,
      // which the second conversion overwrites
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
      pop[u >> 1][4 * (u & 1) + j] = wd;
      // the four codes are keys 32 u + 8 j + 4 g + (0..3): one 4-byte store
      if (kDump && prow != nullptr) *(uint32_t*)(prow + 32 * u + 8 * j + 4 * g) = (uint32_t)wd;
    }
  }
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from a buffer into LDS: lane l writes LDS bytes
// [m0 + 16 l, m0 + 16 l + 16). Written as assembly so that the compiler does
// not treat the copy as a store that every later LDS read may alias (it
// would wait for the copy to land before the first read); completion is
// awaited explicitly with vmcnt before the barrier that publishes the tile.
// (M0 is reserved by the compiler, which never keeps a value in it across
// this code; the clobber only documents the write.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const v4i& rsrc, uint32_t m0, uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until every tile copy this wave issued has landed in LDS. The
// assembly form emits the wait; the builtin tells the compiler's own counter
// tracking that all vector-memory loads before this point are complete.
__device__ __forceinline__ void wait_tiles() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unchanged
}

// Staging of K and V^T tiles into LDS rings with buffer_load ... lds, for a
// workgroup of kAttnWaves = 8 waves: lane l of a wave instruction writes LDS
// bytes [16 l, 16 l + 16) of a 1 KB group of rows (K: 1024/kD rows of kD
// bytes; V^T: 8 rows of 128 bytes), i.e. row grp * rows_per_group +
// l / chunks_per_row and swizzled chunk l % chunks_per_row, so it reads the
// source chunk XORed with the row's swizzle key. A tile is kD/8 groups, kD/64
// per wave. The lane offsets are loop-invariant; the tile offset is a scalar.
// Buffer descriptors cover one head's K rows and V^T rows (base, stride 0,
// size in bytes < 2^31, default data format). `lds_k` and `lds_v` are slot 0
// of rings whose slots are kKeyTile * kD bytes apart.
template <int kD>
struct KvStage {
  static constexpr int kGroupsPerWave = kD / 64;
  v4i rk, rv;
  uint32_t koff[kGroupsPerWave], voff[kGroupsPerWave];
  uint32_t kl0, vl0;

  __device__ __forceinline__ KvStage(const uint8_t* kbase, const uint8_t* vbase, int Skv_pad, const uint8_t* lds_k,
                                     const uint8_t* lds_v, int wave, int wave_s, int lane) {
    const uint64_t kaddr = (uint64_t)(uintptr_t)kbase, vaddr = (uint64_t)(uintptr_t)vbase;
    const uint32_t nbytes = (uint32_t)Skv_pad * kD;
    rk = (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)kaddr),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(kaddr >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane((int)nbytes), 0x00020000};
    rv = (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)vaddr),
               __builtin_amdgcn_readfirstlane((int)(uint32_t)(vaddr >> 32) & 0xFFFF),
               __builtin_amdgcn_readfirstlane((int)nbytes), 0x00020000};
    constexpr int kKChunks = kD / 16;   // 16-byte chunks per K row
#pragma unroll
    for (int i = 0; i < kGroupsPerWave; ++i) {
      const int grp = wave + 8 * i;
      const int krow = (1024 / kD) * grp + lane / kKChunks;
      koff[i] = (uint32_t)(krow * kD + (((lane % kKChunks) ^ swz_key<kD>(krow)) << 4));
      const int vrow = 8 * grp + (lane >> 3);
      voff[i] = (uint32_t)(vrow * Skv_pad + (((lane & 7) ^ swz_key<128>(vrow)) << 4));
    }
    // LDS byte address of the first 1 KB row group this wave writes per slot
    kl0 = lds_addr(lds_k) + wave_s * 1024;
    vl0 = lds_addr(lds_v) + wave_s * 1024;
  }
  // K tile t (keys [kKeyTile t, +kKeyTile)) into ring slot `slot`
  __device__ __forceinline__ void load_k(int t, int slot) const {
#pragma unroll
    for (int i = 0; i < kGroupsPerWave; ++i)
      dma16(rk, kl0 + slot * (kKeyTile * kD) + i * 8192, koff[i], (uint32_t)t * (kKeyTile * kD));
  }
  // V^T tile t (columns [kKeyTile t, +kKeyTile) of the kD rows) into slot
  __device__ __forceinline__ void load_v(int t, int slot) const {
#pragma unroll
    for (int i = 0; i < kGroupsPerWave; ++i)
      dma16(rv, vl0 + slot * (kD * kKeyTile) + i * 8192, voff[i], (uint32_t)t * kKeyTile);
  }
};

struct RowState {
  float m, m2;
};

// Vector phase of one key tile for one wave: running max, rescale of the
// output and row-sum accumulators, P' and its FP8 codes. ks4 holds the
// scales of the tile's four 32-key K blocks.
template <int kD, bool kTail, bool kDump = false>
__device__ __forceinline__ void vector_phase(const v16i s[4], float qs, const float4 ks4, float c,
                                             float log2_448, int nvalid, int g, RowState& st, v16f o[kD / 32],
                                             v16f& lacc, v8i pop[2], uint8_t* prow = nullptr) {
  float f[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) f[u] = (qs * (u == 0 ? ks4.x : u == 1 ? ks4.y : u == 2 ? ks4.z : ks4.w)) * c;

  // t = fl32(A f) is monotone in A for f >= 0, so the tile max is taken on
  // the (biased) integers of each 32-key block and dequantized once: the
  // biased maximum read as a float is 1.5 * 2^23 + A, and subtracting
  // 1.5 * 2^23 is exact (both lie in [2^23, 2^24)).
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
      if (mx != INT32_MIN) tmax = fmaxf(tmax, (__int_as_float(mx) - kScoreBiasF) * f[u]);
    } else {
      tmax = fmaxf(tmax, (__int_as_float(max16(s[u])) - kScoreBiasF) * f[u]);
    }
  }
  tmax = pair_max(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float m2_new = m_new - log2_448;
  const float alpha = __builtin_amdgcn_exp2f(st.m2 - m2_new);
  // P' of the largest score is 448 * 2^e, where e collects the fp32
  // roundings of m, m2 and the exponent: at most half an ulp of m and of m2
  // plus 2^-21. While |m| < 2^17 that is below 2^-5 and P' < 448 * 2^(1/32)
  // < 464, the limit of the conversion (above it the hardware gives NaN).
  // Larger maxima (outlier-scale Q/K blocks) take the saturating variant.
  if (__builtin_expect(__ballot(fabsf(m_new) >= 131072.0f) != 0, 0))
    softmax_p<true, kTail, kDump>(s, f, m2_new, nvalid, g, pop, prow);
  else
    softmax_p<false, kTail, kDump>(s, f, m2_new, nvalid, g, pop, prow);
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int cb = 0; cb < kD / 32; ++cb) o[cb] *= alpha;
    // every element of a lane's L^T column is its query's l, and only
    // element 0 is read: the MFMA adds each tile's sum to each element
    // independently, so rescaling element 0 alone keeps it exact
    lacc[0] *= alpha;
  }
  st.m = m_new;
  st.m2 = m2_new;
}

// Row sums of 64 FP8 codes per query column: L^T += ONES . P^T with one FP8
// MFMA (`ones` holds the E4M3FN code of 1.0 in every byte, `p` a lane's 32
// codes of its query). The FP8 MFMA does not add its products exactly:
// within each group of 8 consecutive codes of a lane it cuts every product
// toward zero to a multiple of 2^(E-13), where E is the largest e_a + e_b
// over the group's non-zero products (e the exponent of an operand's
// encoding, -6 for subnormals), and adds the group sums and the accumulator
// in fp32 (debug_fp8_dot_kernel runs the instruction on given codes). With
// the all-ones operand E is the exponent of the group's largest code, so a
// group loses less than 7 * 2^-13 of its sum.
__device__ __forceinline__ void rowsum_mfma(v16f& lacc, const v8i& ones, const v8i& p) {
  lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, p, lacc, 0, 0, 0, 0, 0, 0);
}

// O^T += V^T . P^T for one 128-key tile (8 FP8 MFMAs at head dim 128, with
// the same inexact addition of the exact products as rowsum_mfma), and the
// row sums (2 FP8 MFMAs, rowsum_mfma).
template <int kD>
__device__ __forceinline__ void pv_tile(const uint8_t* lv, const v8i pop[2], int li, int g, v16f o[kD / 32],
                                        v16f& lacc, const v8i& ones) {
#pragma unroll
  for (int w = 0; w < 2; ++w) rowsum_mfma(lacc, ones, pop[w]);
#pragma unroll
  for (int w = 0; w < 2; ++w) {
#pragma unroll
    for (int cb = 0; cb < kD / 32; ++cb) {
      const int row = 32 * cb + li;
      const v4i lo = *(const v4i*)(lv + swz<128>(row, 4 * w + 2 * g));
      const v4i hi = *(const v4i*)(lv + swz<128>(row, 4 * w + 2 * g + 1));
      const v8i vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop[w], o[cb], 0, 0, 0, 0, 0, 0);
    }
  }
}

// One workgroup = 8 waves = 256 queries of one (b, h); each wave owns 32
// queries and streams every key tile. Waves w and w + 4 run on the same SIMD.
// Per tile a wave has a matrix phase (QK^T of the tile, PV of the previous
// one) and a vector phase (online softmax). Between two barriers, waves 0-3
// run vector then matrix phase and waves 4-7 matrix then vector phase, so
// that on each SIMD one wave's exp/FMA work meets the other wave's MFMAs:
//   interval i, waves 0-3: softmax(i), QK(i+1), PV(i)
//   interval i, waves 4-7: QK(i), PV(i-1), softmax(i)
// (waves 4-7 issue QK first because their vector phase needs its scores;
// the PV MFMAs issued after them are still in the pipe when it starts)
// (waves 0-3 compute QK(0) before interval 0; waves 4-7 compute PV(T-1)
// after the last one). The matrix phase runs at raised wave priority
// (s_setprio 2): its few MFMA and LDS issues then go first, and the other
// wave's vector work fills the cycles between them. Interval i reads K
// tiles i, i+1 and V tiles i-1, i, and loads K tile i+2 and V tile i+1 into
// the third slot of each three-stage LDS ring.
// kDump (debug instantiation): the P codes of every tile are also stored to
// pdump [B, H, Sq, Skv_pad] (key order; padded keys 0).
template <int kD, bool kQuantQ, bool kDump = false>
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const int8_t* __restrict__ q8, const float* __restrict__ qscale,
                     const uint16_t* __restrict__ qraw,
                     const int8_t* __restrict__ k8, const float* __restrict__ kscale,
                     const uint8_t* __restrict__ v8t, const float* __restrict__ vscale, int Sq, int Skv,
                     int H, int Sq_pad, int Skv_pad, int nqt, int num_wg, float c, float log2_448,
                     uint16_t* __restrict__ out, float* __restrict__ lse, uint8_t* __restrict__ pdump) {
  static_assert(kAttnWaves == 8, "the phase skew pairs waves w and w + 4");
  static_assert(kD == 128 || kD == 64, "head dims 64 and 128");
  // K tile: kKeyTile rows of kD bytes; V^T tile: kD rows of kKeyTile bytes
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[3][kKeyTile * kD];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v[3][kD * kKeyTile];

  const int wg = xcd_remap(blockIdx.x, num_wg);
  const int qt = wg % nqt;
  const int64_t bh = wg / nqt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool lead = wave_s < 4;
  const int q0 = qt * kQueryTile + wave * 32;
  uint8_t* prow = (kDump && q0 + li < Sq) ? pdump + ((bh * Sq + q0 + li) * (int64_t)Skv_pad) : nullptr;
  auto prow_at = [&](int i) { return prow != nullptr ? prow + i * kKeyTile : nullptr; };

  const uint8_t* kbase = (const uint8_t*)k8 + bh * Skv_pad * kD;
  const uint8_t* vbase = v8t + bh * kD * (int64_t)Skv_pad;
  const float* ksb = kscale + bh * (Skv_pad / kQBlock);
  const int T = (Skv + kKeyTile - 1) / kKeyTile;

  const KvStage<kD> stage(kbase, vbase, Skv_pad, lds_k[0], lds_v[0], wave, wave_s, lane);
  auto load_k = [&](int t, int slot) { stage.load_k(t, slot); };
  auto load_v = [&](int t, int slot) { stage.load_v(t, slot); };

  load_k(0, 0);
  load_v(0, 0);
  if (T > 1) load_k(1, 1);

  // The wave's Q fragment and block scale: from the quantized tensors, or
  // (kQuantQ) quantized here from bf16 Q.
  v4i qf[kD / 32];
  float qs;
  if (kQuantQ) {
    quant_q_frag<kD>(qraw, bh / H, (int)(bh % H), H, Sq, q0 + li, g, qf, qs);
  } else {
    load_q_frag<kD>(q8 + ((bh * Sq_pad + q0 + li) * kD + (kD / 2) * g), qf);
    qs = qscale[bh * (Sq_pad / kQBlock) + q0 / kQBlock];
  }

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kScoreBias;
  // Opaque to the optimizer: the bias then stays in VGPRs for the whole loop
  // instead of being copied from SGPRs before every tile.
  asm volatile("" : "+v"(bias));
  RowState st{-INFINITY, -INFINITY};
  v16f lacc = (v16f){0};         // row sums of the codes (every register of a lane: its query)
  v8i ones;
#pragma unroll
  for (int k = 0; k < 8; ++k) ones[k] = 0x38383838;   // E4M3FN 1.0 in every byte
  v16f o[kD / 32];
#pragma unroll
  for (int cb = 0; cb < kD / 32; ++cb) o[cb] = (v16f){0};
  v16i s[4];
  v8i pop[2];

  wait_tiles();
  __syncthreads();

  // The two wave groups run separate loops with the same barrier count:
  // interval i (0 <= i < T-1) ends with a barrier; tile i lives in slot
  // i % 3 of both rings. The last interval (i = T-1), whose tile may be
  // ragged (keys >= Skv masked), has no barrier after it.
  if (lead) {
    qk_tile<kD>(lds_k[0], qf, li, g, bias, s);
    // The K block scales of tile i + 1 are loaded during tile i, which hides
    // the scalar-load latency. The slot of tile i is i % 3; the loop body is
    // instantiated per slot, so ring offsets are immediates of the LDS reads
    // rather than per-tile VALU address arithmetic.
    float4 ksc = *(const float4*)ksb;
    auto step = [&](int i, auto slot) {
      constexpr int sl = decltype(slot)::value;
      if (i + 2 < T) load_k(i + 2, (sl + 2) % 3);
      load_v(i + 1, (sl + 1) % 3);
      const float4 ksn = *(const float4*)(ksb + (i + 1) * (kKeyTile / kQBlock));
      vector_phase<kD, false, kDump>(s, qs, ksc, c, log2_448, kKeyTile, g, st, o, lacc, pop, prow_at(i));
      ksc = ksn;
      __builtin_amdgcn_s_setprio(2);
      qk_tile<kD>(lds_k[(sl + 1) % 3], qf, li, g, bias, s);
      pv_tile<kD>(lds_v[sl], pop, li, g, o, lacc, ones);
      __builtin_amdgcn_s_setprio(0);
      wait_tiles();
      __syncthreads();
    };
    int i0 = 0;
    for (; i0 + 3 <= T - 1; i0 += 3) {
      step(i0, std::integral_constant<int, 0>{});
      step(i0 + 1, std::integral_constant<int, 1>{});
      step(i0 + 2, std::integral_constant<int, 2>{});
    }
    if (i0 < T - 1) step(i0++, std::integral_constant<int, 0>{});
    if (i0 < T - 1) step(i0++, std::integral_constant<int, 1>{});
    const int i = T - 1;
    vector_phase<kD, true, kDump>(s, qs, ksc, c, log2_448, Skv - i * kKeyTile, g, st, o, lacc, pop, prow_at(i));
    pv_tile<kD>(lds_v[i % 3], pop, li, g, o, lacc, ones);
  } else {
    // (slot-instantiated body as above; the scales of tile i load at the
    // start of the matrix phase, well ahead of the vector phase)
    auto step = [&](int i, auto slot) {
      constexpr int sl = decltype(slot)::value;
      if (i + 2 < T) load_k(i + 2, (sl + 2) % 3);
      load_v(i + 1, (sl + 1) % 3);
      const float4 ksc = *(const float4*)(ksb + i * (kKeyTile / kQBlock));
      __builtin_amdgcn_s_setprio(2);
      qk_tile<kD>(lds_k[sl], qf, li, g, bias, s);
      if (i > 0) pv_tile<kD>(lds_v[(sl + 2) % 3], pop, li, g, o, lacc, ones);
      __builtin_amdgcn_s_setprio(0);
      vector_phase<kD, false, kDump>(s, qs, ksc, c, log2_448, kKeyTile, g, st, o, lacc, pop, prow_at(i));
      wait_tiles();
      __syncthreads();
    };
    int i0 = 0;
    for (; i0 + 3 <= T - 1; i0 += 3) {
      step(i0, std::integral_constant<int, 0>{});
      step(i0 + 1, std::integral_constant<int, 1>{});
      step(i0 + 2, std::integral_constant<int, 2>{});
    }
    if (i0 < T - 1) step(i0++, std::integral_constant<int, 0>{});
    if (i0 < T - 1) step(i0++, std::integral_constant<int, 1>{});
    const int i = T - 1;
    const int sl = i % 3;
    if (i > 0) pv_tile<kD>(lds_v[(sl + 2) % 3], pop, li, g, o, lacc, ones);
    qk_tile<kD>(lds_k[sl], qf, li, g, bias, s);
    const float4 ksc = *(const float4*)(ksb + i * (kKeyTile / kQBlock));
    vector_phase<kD, true, kDump>(s, qs, ksc, c, log2_448, Skv - i * kKeyTile, g, st, o, lacc, pop, prow_at(i));
    pv_tile<kD>(lds_v[sl], pop, li, g, o, lacc, ones);
  }

  // Epilogue: O = acc * v_scale / l, bf16, layout [B, Sq, H, D]; optional
  // log-sum-exp [B, H, Sq].
  const float lt = lacc[0];
  const float rl = __fdiv_rn(1.0f, lt);
  const int qi = q0 + li;
  if (lse != nullptr && g == 0 && qi < Sq) {
    // log-sum-exp of the row's scaled scores: l = sum 2^(t - m2) (up to the
    // FP8 rounding of each term), so ln sum e^(scale * score) = ln 2 * (m2 + log2 l)
    lse[bh * Sq + qi] = (st.m2 + __builtin_amdgcn_logf(lt)) * 0.6931471805599453f;
  }
  if (qi < Sq) {
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    uint16_t* orow = out + ((b * Sq + qi) * H + h) * kD;
    const float* vsb = vscale + bh * kD;
#pragma unroll
    for (int cb = 0; cb < kD / 32; ++cb) {
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

// Debug dump of the int32 scores of one (b, h) through the attention
// kernel's own path: K tiles staged into LDS by KvStage (buffer-to-LDS
// copies into the swizzled slot), the wave's Q fragment in VGPRs, the INT8
// MFMA sequence of qk_tile with accumulators starting from the bias
// 0x4B400000; the bias is subtracted when a score is stored.
// grid (key tiles of the window, query tiles of kQueryTile rows), 8 waves.
template <int kD>
__global__ __launch_bounds__(64 * kAttnWaves) void debug_qk_kernel(const int8_t* __restrict__ q8,
                                                                  const int8_t* __restrict__ k8, int S_pad,
                                                                  int64_t bh, int rA, int r0, int nr, int cA,
                                                                  int c0, int nc, int32_t* __restrict__ scores) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds_k[kKeyTile * kD];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int t = cA / kKeyTile + blockIdx.x;
  const uint8_t* kbase = (const uint8_t*)k8 + bh * S_pad * kD;
  const KvStage<kD> stage(kbase, kbase, S_pad, lds_k, lds_k, wave, wave_s, lane);
  stage.load_k(t, 0);
  wait_tiles();
  __syncthreads();
  const int qa = rA + blockIdx.y * kQueryTile + wave * 32;
  v4i qf[kD / 32];
  load_q_frag<kD>(q8 + ((bh * S_pad + qa + li) * kD + (kD / 2) * g), qf);
  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kScoreBias;
  v16i sacc[4];
  qk_tile<kD>(lds_k, qf, li, g, bias, sacc);
  const int row = qa + li;
  if (row < r0 || row >= r0 + nr) return;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t * kKeyTile + key_of(u, r, g);
      if (key >= c0 && key < c0 + nc)
        scores[(int64_t)(row - r0) * nc + (key - c0)] = sacc[u][r] - kScoreBias;
    }
}

// Debug run of the PV step's FP8 MFMA on n given pairs of 64-code vectors:
// out[c] = init[c] + a[c] . b[c]. Workgroup x (one wave) takes pairs
// [32x, 32x + 32): row i of the A operand is a[32x + i] and column j of the B
// operand b[32x + j], each lane holding bytes [32h, 32h + 32) of its vector
// (h = lane / 32), as pv_tile feeds V^T rows and P columns. The dot products
// are the diagonal of the 32 x 32 result: element (c, c) sits in lane
// c + 32 * ((c >> 2) & 1), accumulator register 4 * (c >> 3) + (c & 3).
__global__ __launch_bounds__(64) void debug_fp8_dot_kernel(const uint8_t* __restrict__ a,
                                                           const uint8_t* __restrict__ b, int64_t n,
                                                           const float* __restrict__ init, float* __restrict__ out) {
  const int lane = threadIdx.x, h = lane >> 5, i = lane & 31;
  const int64_t c = (int64_t)blockIdx.x * 32 + i;
  v8i av = (v8i){0}, bv = (v8i){0};
  float c0 = 0.0f;
  if (c < n) {
    const v4i alo = *(const v4i*)(a + 64 * c + 32 * h), ahi = *(const v4i*)(a + 64 * c + 32 * h + 16);
    const v4i blo = *(const v4i*)(b + 64 * c + 32 * h), bhi = *(const v4i*)(b + 64 * c + 32 * h + 16);
    av = (v8i){alo[0], alo[1], alo[2], alo[3], ahi[0], ahi[1], ahi[2], ahi[3]};
    bv = (v8i){blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
    c0 = init[c];
  }
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = c0;   // column c of the accumulator starts at init[c]
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
  const int rsel = 4 * (i >> 3) + (i & 3);
  float d = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (r == rsel) d = acc[r];
  if (c < n && h == ((i >> 2) & 1)) out[c] = d;
}

}  // namespace sage
