/*
 * sage.h - C ABI of the MI355X (gfx950) SageAttention-style quantized
 * attention forward.
 *
 * What it computes (diffusers issue #15014, "gfx1201 (RDNA4) SageAttention
 * attention backend: aiter package or Hub kernel?", problem statement): the
 * forward of softmax(Q K^T * softmax_scale) V where QK^T multiplies INT8
 * codes and PV FP8 codes, both summing in fp32, with one scale per 32-row
 * block of Q and of K and one per channel of V, on bf16 [B, S, H, 128]
 * inputs of one shape, unmasked and non-causal. The
 * call there is gfx1201_sage_attention(q, k, v, softmax_scale). Inference
 * only, and no log-sum-exp is returned (diffusers PR #15060, "Add
 * aiter_sage_hub attention backend for AMD RDNA4 (gfx1201)", section "What
 * does this PR do?"). Unsupported inputs are rejected with an error code
 * rather than served differently (the issue's section "Describe the
 * solution you'd like" asks for an explicit failure there); a caller may
 * fall back on its own.
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a device pointer owned by the caller. The
 *     library never allocates, frees or synchronizes device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns before it completes;
 *     results are valid after the caller synchronizes that stream.
 *   - All argument checks run on the host before any launch; a failing check
 *     returns its code and touches no memory. Launch failures return
 *     SAGE_ERR_HIP. sage_last_error() gives a thread-local detail string.
 *   - No global mutable state besides that string: calls are thread-safe;
 *     calls that share output or workspace buffers must be ordered by the
 *     caller.
 *   - Sizes: B, S, H >= 1, S <= 2^24, B, H <= 2^20 and B*H*S_pad*D < 2^62;
 *     each launch's grid (about B*H*S_pad/128 workgroups for the largest)
 *     must also stay below 2^31. Larger sizes return SAGE_ERR_SHAPE.
 *   - Head dim: D == 128 is the pages' operation. D == 64 is also accepted
 *     by every entry point (the pages' callers
 *     fall back for it: the VAE's head dim 64, diffusers PR #15060, section
 *     "What does this PR do?"); every "128" channel count below then reads
 *     D. Other head dims return SAGE_ERR_UNSUPPORTED.
 *   - softmax_scale must be finite and >= 0 (SAGE_ERR_SHAPE otherwise): the
 *     kernels take each key block's maximum on the integer scores, which
 *     orders the scaled scores only for a non-negative factor.
 *   - Inputs containing NaN/Inf, or whose scaled scores overflow fp32, are
 *     outside the contract (no guarantee on the output).
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_NULL = 1,        /* a required pointer is NULL                     */
  SAGE_ERR_SHAPE = 2,       /* B, S or H < 1, or sizes overflow               */
  SAGE_ERR_UNSUPPORTED = 3, /* head dim other than 128 or 64; unknown flags    */
  SAGE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
  SAGE_ERR_WORKSPACE = 5,   /* workspace/scratch smaller than required        */
  SAGE_ERR_HIP = 6,         /* a HIP launch failed                            */
  SAGE_ERR_RANGE = 7        /* debug-dump window outside the tensor           */
} sage_status;

/* ABI version of this header (incremented on any incompatible change). */
int sage_abi_version(void);

/* Static name of a status code. */
const char* sage_status_str(int status);

/* Thread-local text describing the last failing call on this thread. */
const char* sage_last_error(void);

/* Key-tile width BN of sage_attn_fwd. The online softmax rescales once per
 * tile, and P is quantized relative to the running row max after each tile,
 * so the result depends on BN; a reference implementation needs it. */
int sage_kv_tile(void);

/* Padded sequence length of the quantized layouts: S rounded up to a
 * multiple of 256. Padded rows/keys hold zeros and are masked. */
int64_t sage_seq_pad(int64_t S);

/* Bytes of scratch sage_quant_v needs (per-chunk partial maxima). */
size_t sage_quant_v_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D);

/* Bytes of workspace sage_attention needs: the quantized K and V, their
 * scales and sage_quant_v's scratch, each 256-byte aligned (Q needs none: the
 * attention kernel quantizes it), about 2 bytes per element of K or V, i.e.
 * 0.67 bytes per element of the three inputs. 0 on bad sizes. */
size_t sage_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D);

/*
 * sage_quant_qk - INT8 quantization of Q or K per 32-row block (issue #15014,
 * problem statement: one scale per 32-row block of Q and of K).
 *   x       bf16 [B, S, H, D], contiguous (row (b, s, h) holds D values).
 *   x_i8    int8 [B, H, S_pad, D] out, S_pad = sage_seq_pad(S); rows >= S
 *           are written as zeros.
 *   x_scale fp32 [B, H, S_pad/32] out; block t covers rows [32t, 32t+32) of
 *           one (b, h); blocks past S get 0.
 * Per block: amax = max |x| over its valid rows (a short last block uses
 * only its valid rows); scale = fl32(amax/127); q = clamp(rint_even(
 * fl32(x * fl32(127/amax))), -127, 127); amax = 0 (or a non-finite
 * reciprocal) gives scale 0 and q = 0. Pointers 16-byte aligned.
 */
sage_status sage_quant_qk(const void* x, int64_t B, int64_t S, int64_t H, int64_t D,
                          int8_t* x_i8, float* x_scale, void* stream);

/*
 * sage_quant_v - FP8 E4M3FN quantization of V per channel (issue #15014,
 * problem statement: one scale per channel of V).
 *   v        bf16 [B, S, H, D], contiguous.
 *   v_fp8_t  uint8 [B, H, D, S_pad] out: OCP E4M3FN codes, transposed (one
 *            row of S_pad keys per channel). Within each group of 64 keys
 *            starting at a multiple of 64, slot p holds key
 *              kappa(p) = 32*u + 8*(r/4) + 4*g + (r%4),
 *            where p = 32*g + 16*u + r, g in {0,1}, u in {0,1}, r in [0,16)
 *            (the key order the fused kernel's PV operands use). Keys >= S
 *            hold code 0.
 *   v_scale  fp32 [B, H, D] out.
 *   scratch  device memory of sage_quant_v_scratch_bytes(...) bytes.
 * Per channel c of (b, h): amax = max over s < S of |v|; v_scale =
 * fl32(amax/448); code = E4M3FN_rne(fl32(v * fl32(448/amax))); amax = 0
 * gives scale 0 and code 0. 448 is the largest E4M3FN value.
 */
sage_status sage_quant_v(const void* v, int64_t B, int64_t S, int64_t H, int64_t D,
                         uint8_t* v_fp8_t, float* v_scale, void* scratch, size_t scratch_bytes,
                         void* stream);

/*
 * sage_quant_kv - sage_quant_qk(K) and sage_quant_v(V) together, as the
 * attention needs them (issue #15014, problem statement: K per 32-row block,
 * V per channel). Same arguments, layouts, results and errors as those two
 * calls; the first of its two launches quantizes K and takes V's per-chunk
 * maxima in one pass over both tensors. scratch as for sage_quant_v.
 */
sage_status sage_quant_kv(const void* k, const void* v, int64_t B, int64_t S, int64_t H, int64_t D,
                          int8_t* k_i8, float* k_scale, uint8_t* v_fp8_t, float* v_scale, void* scratch,
                          size_t scratch_bytes, void* stream);

/* Size of the static device buffer sage_quant_v_noalloc uses (8 MiB per GPU). */
#define SAGE_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * sage_quant_v_noalloc - sage_quant_v without a scratch argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments,
 * layouts, results and errors as sage_quant_v, except:
 *   - the per-chunk partial maxima live in a static device buffer of
 *     SAGE_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from the
 *     first call on that GPU until the process ends; shapes whose scratch
 *     (sage_quant_v_scratch_bytes) exceeds it return SAGE_ERR_WORKSPACE;
 *   - the call allocates and frees nothing; its first call on a device
 *     looks up the buffer's device address (hipGetSymbolAddress), on the
 *     current device, which must be the device of `stream`;
 *   - every call on one GPU shares that buffer: calls that may overlap on
 *     one GPU (different streams, no ordering between them) race and must
 *     be serialized by the caller. Each call overwrites all of the scratch
 *     it reads, so no state carries from one call to the next.
 */
sage_status sage_quant_v_noalloc(const void* v, int64_t B, int64_t S, int64_t H, int64_t D,
                                 uint8_t* v_fp8_t, float* v_scale, void* stream);

/*
 * sage_attn_fwd - fused attention on quantized inputs (issue #15014,
 * problem statement: QK^T on INT8 codes, PV on FP8 codes, fp32 sums).
 * Inputs are the outputs of sage_quant_qk (Q and K) and sage_quant_v.
 * out: bf16 [B, S, H, D] (the input layout), rows >= S are not written.
 * Per query row i, over key tiles of sage_kv_tile() keys in key order:
 *   A = q8 . k8^T (exact int32);  c = fl32(fl32(softmax_scale)*fl32(log2 e));
 *   f = fl32(fl32(q_scale*k_scale)*c) per (query block, key block);
 *   t = fl32(A*f); m = running max of t (keys >= S masked);
 *   m2 = fl32(m - fl32(log2 448)); P' = 2^fl32(A*f - m2), the exponent
 *   being the exact real value A*f - m2 rounded once (a fused multiply-add;
 *   hardware exp2), so P' = 448 * 2^(t - m) up to rounding;
 *   p8 = E4M3FN(min(P', 448)); acc[c] = sum p8 * v8[c] and l = sum p8
 *   (FP8 MFMAs, fp32 accumulation, rescaled by 2^(m2_old - m2) when the max
 *   moves): the normalizer sums the same FP8 weights that multiply V;
 *   out = bf16_rne(acc * v_scale[c] / l).
 * The FP8 MFMA adds its exact products after cutting each to a grid set by
 * the largest exponents in its group of 8 (sage_debug_fp8_dot), so l can be
 * below the exact sum of the codes by less than 7 * 2^-13 of it, and each
 * element of acc off by less than 7 * 2^-13 * max|v8[c]| * (l + S / 512).
 */
sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                          const float* k_scale, const uint8_t* v_fp8_t, const float* v_scale,
                          int64_t B, int64_t S, int64_t H, int64_t D, float softmax_scale, void* out,
                          void* stream);

/*
 * sage_attention - one call: sage_quant_kv(K, V) and the attention with Q quantized inside the kernel (sage_attn_fwd_qbf16; the
 * result equals sage_quant_qk(Q) followed by sage_attn_fwd), with every
 * intermediate inside the caller's workspace (>= sage_workspace_bytes(B, S, H, D) bytes, 256-byte
 * aligned). This is the gfx1201_sage_attention(q, k, v, softmax_scale)
 * operation of the issue's problem statement. q, k, v, out: bf16
 * [B, S, H, D].
 */
sage_status sage_attention(const void* q, const void* k, const void* v, int64_t B, int64_t S,
                           int64_t H, int64_t D, float softmax_scale, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * sage_debug_qk_scores - debug dump of the exact int32 scores A = q8 . k8^T
 * of one (b, h), rows [r0, r0+nr) x keys [c0, c0+nc), computed through the
 * attention kernel's own path: K tiles staged into LDS by the same
 * buffer-to-LDS copies into the same swizzled layout, the same Q fragments,
 * the same INT8 MFMA sequence with the accumulators starting from the same
 * bias (0x4B400000, subtracted when a score is stored).
 *   scores  int32 [nr, nc] out, row-major.
 * Windows must satisfy 0 <= r0, 0 < nr, r0+nr <= S_pad (same for keys).
 * D is 128 or 64.
 */
sage_status sage_debug_qk_scores(const int8_t* q_i8, const int8_t* k_i8, int64_t B, int64_t S,
                                 int64_t H, int64_t D, int64_t b, int64_t h, int64_t r0,
                                 int64_t nr, int64_t c0, int64_t nc, int32_t* scores,
                                 void* stream);

/*
 * sage_debug_p_codes - debug run of sage_attn_fwd that also stores the FP8
 * E4M3FN codes of P' = 448 * 2^(t - m) as the attention kernel forms them:
 * per key tile of sage_kv_tile() keys, against the running row maximum m
 * after that tile (the online softmax of diffusers issue #15014, "gfx1201
 * (RDNA4) SageAttention attention backend: aiter package or Hub kernel?",
 * problem statement: FP32 softmax, FP8 PV with the fixed scale 448).
 *   q_i8 .. v_scale, B, S, H, D, softmax_scale, out  as sage_attn_fwd (out
 *            receives the same output bit for bit).
 *   codes    uint8 [B, H, S, S_pad] out, caller-owned: codes[b,h,i,j] is the
 *            code of query i and key j (natural key order); keys >= S are 0.
 * S <= 131072 (SAGE_ERR_RANGE otherwise): the codes take S * S_pad bytes
 * per (b, h), up to 17 GB. Test and diagnostic use only.
 */
sage_status sage_debug_p_codes(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                               const float* k_scale, const uint8_t* v_fp8_t, const float* v_scale,
                               int64_t B, int64_t S, int64_t H, int64_t D, float softmax_scale,
                               uint8_t* codes, void* out, void* stream);

/*
 * sage_debug_fp8_dot - debug run of the FP8 MFMA of the PV step (FP8 PV with
 * fp32 accumulation, diffusers issue #15014 problem statement) on n given
 * pairs of E4M3FN vectors of 64 codes: out[c] = init[c] + a[c] . b[c], where
 * a takes the place of a V^T row and b that of a column of P.
 *   a, b  uint8 [n, 64] in, 16-byte aligned, device; consumed in groups of 8
 *         consecutive codes.
 *   init  fp32 [n] in, device: the accumulator before the MFMA.
 *   out   fp32 [n] out, device.
 * The products are exact but their sum is not: in each group of 8 the MFMA
 * cuts every product toward zero to a multiple of 2^(E-13), where E is the
 * largest e_a + e_b over the group's non-zero products and e is the exponent
 * of an operand's encoding (-6 for subnormals), then adds the group sums and
 * init in fp32.
 * 1 <= n <= 2^24 (SAGE_ERR_RANGE otherwise). Test and diagnostic use only.
 */
sage_status sage_debug_fp8_dot(const uint8_t* a, const uint8_t* b, int64_t n, const float* init, float* out,
                               void* stream);

/* ---------------------------------------------------------------------------
 * Extensions beyond the gfx1201 operation: log-sum-exp output, query and
 * key/value sequences of different lengths, and optional K smoothing.
 * ------------------------------------------------------------------------- */

/* Flags of sage_attention_ex. */
#define SAGE_SMOOTH_K 1u  /* quantize K - mean_s(K) instead of K (sage_quant_k_smooth) */

/* Bytes of scratch sage_quant_k_smooth needs (fp64 channel sums per 256-row chunk). */
size_t sage_k_smooth_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D);

/*
 * sage_quant_k_smooth - K smoothing followed by sage_quant_qk's INT8
 * quantization. The pages name K smoothing as SageAttention's default option
 * and measure it on and off (InvokeAI PR #9657, "feat(attention): add opt-in
 * SageAttention backend for diffusion models", sections "How it works" and
 * "QA Instructions"); it subtracts the mean of K over the sequence per
 * (b, h, channel), to which exact softmax is invariant because every score
 * of a query row moves by the same amount.
 *   k        bf16 [B, S, H, D], contiguous.
 *   k_i8     int8 [B, H, S_pad, D] out; k_scale fp32 [B, H, S_pad/32] out
 *            (as sage_quant_qk, applied to the smoothed values).
 *   k_mean   fp32 [B, H, D] out.
 *   scratch  device memory of sage_k_smooth_scratch_bytes(...) bytes.
 * Per channel c of (b, h): k_mean = the exact mean of k[s] over s < S,
 * rounded once to fp32 (nearest, ties to even). The sums are formed in fp64,
 * which is exact while the values of a channel span fewer than about
 * 45 - log2(S) binades (outside that range the mean may differ from the
 * exact rounding by one ulp). The values quantized are fl32(k - k_mean) on
 * rows s < S (padded rows stay 0).
 */
sage_status sage_quant_k_smooth(const void* k, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* k_i8,
                                float* k_scale, float* k_mean, void* scratch, size_t scratch_bytes,
                                void* stream);

/*
 * sage_attn_fwd_ex - sage_attn_fwd with a query sequence of Sq rows and a
 * key/value sequence of Skv rows (cross-attention), and an optional
 * log-sum-exp output. The pages' operation falls back for unequal Q/K/V
 * shapes and returns no LSE, which keeps ring attention from using it
 * (diffusers PR #15060, "Add aiter_sage_hub attention backend for AMD RDNA4
 * (gfx1201)", section "What does this PR do?").
 *   q_i8, q_scale   from sage_quant_qk on Q [B, Sq, H, D] (S_pad = sage_seq_pad(Sq)).
 *   k_i8, k_scale   from sage_quant_qk or sage_quant_k_smooth on K [B, Skv, H, D].
 *   v_fp8_t, v_scale from sage_quant_v on V [B, Skv, H, D].
 *   out  bf16 [B, Sq, H, D].
 *   lse  fp32 [B, H, Sq] or NULL (4-byte aligned): per query row,
 *        ln(sum_j exp(softmax_scale * q.k_j)) of the dequantized scores,
 *        formed from the kernel's state as ln2 * (m2 + log2 l) (m2 and l as
 *        in sage_attn_fwd after the last key tile; l sums the FP8 codes of
 *        P, so this is the exact value up to their rounding, at most
 *        ln(1 + 2^-4) per row and unbiased on average, and up to the FP8
 *        MFMA's cuts, which lower it by less than 8.6e-4).
 * sage_attn_fwd(..., S, ...) equals sage_attn_fwd_ex(..., S, S, ..., NULL).
 */
sage_status sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                             const uint8_t* v_fp8_t, const float* v_scale, int64_t B, int64_t Sq, int64_t Skv,
                             int64_t H, int64_t D, float softmax_scale, void* out, float* lse, void* stream);

/* Bytes of workspace sage_attention_ex needs (any flags). 0 on bad sizes. */
size_t sage_workspace_bytes_ex(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D);

/*
 * sage_attention_ex - one call for q bf16 [B, Sq, H, D] and k, v bf16
 * [B, Skv, H, D]: sage_quant_qk(Q), sage_quant_qk(K) (or, with
 * SAGE_SMOOTH_K, sage_quant_k_smooth(K)), sage_quant_v(V) and
 * sage_attn_fwd_ex, intermediates in the caller's workspace
 * (>= sage_workspace_bytes_ex bytes, 256-byte aligned). lse may be NULL.
 * Unknown flag bits return SAGE_ERR_UNSUPPORTED.
 */
sage_status sage_attention_ex(const void* q, const void* k, const void* v, int64_t B, int64_t Sq, int64_t Skv,
                              int64_t H, int64_t D, float softmax_scale, unsigned flags, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd_qbf16 - sage_attn_fwd_ex with Q given as bf16 [B, Sq, H, D]
 * and quantized inside the attention kernel, as the pages' kernel quantizes
 * its inputs "inside the kernel" (diffusers issue #15014, problem
 * statement). Each wave's 32 query rows are exactly one quantization block,
 * so the codes and scales equal sage_quant_qk's bit for bit and the output
 * equals sage_attn_fwd_ex on sage_quant_qk(Q). K and V come quantized
 * (reusable across calls that share them). sage_attention and
 * sage_attention_ex use this path.
 */
sage_status sage_attn_fwd_qbf16(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8_t,
                                const float* v_scale, int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                                float softmax_scale, void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
