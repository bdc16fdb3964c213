// C ABI of the quantized attention forward (declared in include/sage.h):
// host-side validation, workspace layout and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "sage.h"
#include "sage_attn.hpp"
#include "sage_common.hpp"
#include "sage_quant.hpp"

// Scratch of sage_quant_v_noalloc (the per-chunk partial maxima of V), in
// device memory that exists from module load until the process ends, one
// copy per GPU. Host code never passes this name to a kernel: it stands for
// a host-side shadow, not a device address. The device address comes from
// hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[SAGE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kAbiVersion = 1;
constexpr int64_t kDebugPMaxSeq = 131072;  // sage_debug_p_codes: S x S_pad bytes per head
constexpr int64_t kDebugDotMax = int64_t(1) << 24;  // sage_debug_fp8_dot pairs
thread_local char g_last_error[512] = "";

sage_status fail(sage_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sage_status fail(sage_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

// Test hook: SAGE_TEST_FAIL_LAUNCH=1 makes every launching entry point
// report SAGE_ERR_HIP after validation, without launching, so callers' error
// paths can be exercised on any host.
bool forced_launch_failure() {
  const char* e = getenv("SAGE_TEST_FAIL_LAUNCH");
  return e && e[0] == '1';
}

int64_t seq_pad(int64_t S) { return (S + sage::kSeqAlign - 1) / sage::kSeqAlign * sage::kSeqAlign; }

sage_status check_shape(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (D != 128 && D != 64) return fail(SAGE_ERR_UNSUPPORTED, "head dim %lld unsupported (64 or 128)", (long long)D);
  if (B < 1 || S < 1 || H < 1) return fail(SAGE_ERR_SHAPE, "B, S, H must be >= 1 (got %lld, %lld, %lld)",
                                           (long long)B, (long long)S, (long long)H);
  // S_pad * B * H * D must stay well inside int64, and one head's quantized
  // K or V^T (S_pad * 128 bytes) inside the 2^31-byte reach of a buffer
  // descriptor offset
  if (S > (int64_t)1 << 24 || B > (int64_t)1 << 20 || H > (int64_t)1 << 20)
    return fail(SAGE_ERR_SHAPE, "sizes too large (S <= 2^24, B, H <= 2^20)");
  const double n = (double)B * (double)H * (double)seq_pad(S) * (double)D;
  if (n >= 4.0e18) return fail(SAGE_ERR_SHAPE, "sizes overflow");
  return SAGE_OK;
}

sage_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(SAGE_ERR_NULL, "%s is NULL", name);
  if (((uintptr_t)p) & 15) return fail(SAGE_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return SAGE_OK;
}

#define SAGE_TRY(expr)                  \
  do {                                  \
    sage_status _s = (expr);            \
    if (_s != SAGE_OK) return _s;       \
  } while (0)

sage_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SAGE_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return SAGE_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sage_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SAGE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SAGE_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SAGE_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAGE_OK;
}

// V amax chunks: rows of at least kVChunkRows per chunk, at most 32 chunks
// per (b, h) (the quantize kernel reduces them per workgroup).
int64_t v_nchunk(int64_t S) {
  const int64_t n = (S + sage::kVChunkRows - 1) / sage::kVChunkRows;
  return n < 32 ? n : 32;
}
int64_t v_chunk_rows(int64_t S) { return (S + v_nchunk(S) - 1) / v_nchunk(S); }

size_t v_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  // partial maxima [B*H, nchunk, D]
  return align256((size_t)(B * H * v_nchunk(S) * D) * 4);
}

// Intermediates of sage_attention, each 256-byte aligned: K codes, V codes
// (transposed), K and V scales, and sage_quant_v's scratch. Q needs no
// region: the attention kernel quantizes it.
struct Workspace {
  size_t k8, v8, ks, vs, scratch_off, total, scratch_bytes;
};

Workspace layout(int64_t B, int64_t S, int64_t H, int64_t D) {
  Workspace w{};
  const int64_t Sp = seq_pad(S);
  const size_t codes = align256((size_t)(B * H * Sp * D));
  w.k8 = 0;
  w.v8 = w.k8 + codes;
  w.ks = w.v8 + codes;
  w.vs = w.ks + align256((size_t)(B * H * (Sp / 32)) * 4);
  w.scratch_off = w.vs + align256((size_t)(B * H * D) * 4);
  w.scratch_bytes = v_scratch_bytes(B, S, H, D);
  w.total = w.scratch_off + w.scratch_bytes;
  return w;
}

template <int kD, bool kSmooth>
void launch_quant_qk(const void* x, int64_t S, int64_t H, int64_t Sp, int nbp, int64_t total, int64_t grid,
                     const float* xmean, int8_t* xq, float* xs, hipStream_t st) {
  hipLaunchKernelGGL((sage::quant_qk_kernel<kD, kSmooth>), dim3((unsigned)grid), dim3(256), 0, st,
                     (const uint16_t*)x, (int)S, (int)H, (int)Sp, nbp, total, xmean, xq, xs);
}

sage_status quant_qk_impl(const void* x, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* xq, float* xs,
                          hipStream_t st, const float* xmean = nullptr) {
  const int64_t Sp = seq_pad(S);
  const int nbp = (int)(Sp / sage::kQBlock);
  const int64_t total = B * H * nbp;
  const int64_t grid = (total + 3) / 4;
  if (grid > INT32_MAX) return fail(SAGE_ERR_SHAPE, "grid too large");
  if (D == 64) {
    if (xmean) launch_quant_qk<64, true>(x, S, H, Sp, nbp, total, grid, xmean, xq, xs, st);
    else launch_quant_qk<64, false>(x, S, H, Sp, nbp, total, grid, nullptr, xq, xs, st);
  } else {
    if (xmean) launch_quant_qk<128, true>(x, S, H, Sp, nbp, total, grid, xmean, xq, xs, st);
    else launch_quant_qk<128, false>(x, S, H, Sp, nbp, total, grid, nullptr, xq, xs, st);
  }
  return launched("sage_quant_qk");
}

int64_t k_sum_chunks(int64_t S) { return (S + sage::kKSumRows - 1) / sage::kKSumRows; }

size_t k_smooth_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  // fp64 chunk sums [B*H, ceil(S/256), D]
  return align256((size_t)(B * H * k_sum_chunks(S) * D) * 8);
}

// K smoothing: per-channel mean over S, then INT8 quantization of K - mean.
template <int kD>
void launch_k_mean(const void* k, int64_t S, int64_t H, int nck, int64_t total, int64_t BH, void* scratch_buf,
                   float* kmean, hipStream_t st) {
  // 4 waves of 64/(kD/8) chunks each per workgroup
  const int64_t per_wg = 4 * (64 / (kD / 8));
  hipLaunchKernelGGL(sage::k_block_sum_kernel<kD>, dim3((unsigned)((total + per_wg - 1) / per_wg)), dim3(256), 0,
                     st, (const uint16_t*)k, (int)S, (int)H, nck, total, (double*)scratch_buf);
  hipLaunchKernelGGL(sage::k_mean_kernel<kD>, dim3((unsigned)BH), dim3(kD), 0, st, (const double*)scratch_buf, nck,
                     (int)S, kmean);
}

sage_status quant_k_smooth_impl(const void* k, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* kq,
                                float* ks, float* kmean, void* scratch_buf, hipStream_t st) {
  const int nck = (int)k_sum_chunks(S);
  const int64_t total = B * H * nck;
  const int64_t BH = B * H;
  if ((total + 15) / 16 > INT32_MAX || BH > INT32_MAX) return fail(SAGE_ERR_SHAPE, "grid too large");
  if (D == 64) launch_k_mean<64>(k, S, H, nck, total, BH, scratch_buf, kmean, st);
  else launch_k_mean<128>(k, S, H, nck, total, BH, scratch_buf, kmean, st);
  SAGE_TRY(launched("sage_quant_k_smooth (mean)"));
  return quant_qk_impl(k, B, S, H, D, kq, ks, st, kmean);
}

int64_t v_tiles_per_head(int64_t S) {
  return (seq_pad(S) / 128 + sage::kVTilesPerWg - 1) / sage::kVTilesPerWg;
}

// grid sizes of the V passes (and of the fused K/V pre-pass) fit int32
sage_status check_v_grids(int64_t B, int64_t S, int64_t H) {
  const int64_t BH = B * H;
  const int64_t nkwg = (B * H * (seq_pad(S) / sage::kQBlock) + 3) / 4;
  if (BH * v_nchunk(S) + nkwg > INT32_MAX || BH * v_tiles_per_head(S) > INT32_MAX)
    return fail(SAGE_ERR_SHAPE, "grid too large");
  return SAGE_OK;
}

template <int kD>
void launch_v_quant(const void* v, int64_t S, int64_t H, int64_t BH, const float* partial, float* vs, uint8_t* vt,
                    hipStream_t st) {
  const int64_t nvt = v_tiles_per_head(S);
  hipLaunchKernelGGL(sage::v_quant_kernel<kD>, dim3((unsigned)(BH * nvt)), dim3(2 * kD), 0, st, (const uint16_t*)v,
                     (int)S, (int)H, (int)seq_pad(S), (int)nvt, partial, (int)v_nchunk(S), vs, vt);
}

template <int kD>
void launch_quant_v(const void* v, int64_t S, int64_t H, int nchunk, int64_t BH, float* partial, float* vs,
                    uint8_t* vt, hipStream_t st) {
  hipLaunchKernelGGL(sage::v_amax_partial_kernel<kD>, dim3((unsigned)(BH * nchunk)), dim3(256), 0, st,
                     (const uint16_t*)v, (int)S, (int)H, nchunk, (int)v_chunk_rows(S), partial);
  launch_v_quant<kD>(v, S, H, BH, partial, vs, vt, st);
}

sage_status quant_v_impl(const void* v, int64_t B, int64_t S, int64_t H, int64_t D, uint8_t* vt, float* vs,
                         void* scratch_buf, hipStream_t st) {
  SAGE_TRY(check_v_grids(B, S, H));
  const int nchunk = (int)v_nchunk(S);
  const int64_t BH = B * H;
  float* partial = (float*)scratch_buf;
  if (D == 64) launch_quant_v<64>(v, S, H, nchunk, BH, partial, vs, vt, st);
  else launch_quant_v<128>(v, S, H, nchunk, BH, partial, vs, vt, st);
  return launched("sage_quant_v");
}

// K quantization and V quantization with one fused first pass: one launch
// quantizes K and takes V's per-chunk maxima, a second quantizes V.
template <int kD>
void launch_quant_kv(const void* k, const void* v, int64_t B, int64_t S, int64_t H, int8_t* kq, float* ks,
                     float* partial, float* vs, uint8_t* vt, hipStream_t st) {
  const int64_t BH = B * H;
  const int nbp = (int)(seq_pad(S) / sage::kQBlock);
  const int64_t total = BH * nbp;
  const int64_t nkwg = (total + 3) / 4;
  const int nchunk = (int)v_nchunk(S);
  hipLaunchKernelGGL(sage::kv_prepass_kernel<kD>, dim3((unsigned)(nkwg + BH * nchunk)), dim3(256), 0, st,
                     (const uint16_t*)k, (const uint16_t*)v, (int)S, (int)H, (int)seq_pad(S), nbp, total, (int)nkwg,
                     kq, ks, nchunk, (int)v_chunk_rows(S), partial);
  launch_v_quant<kD>(v, S, H, BH, partial, vs, vt, st);
}

sage_status quant_kv_impl(const void* k, const void* v, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* kq,
                          float* ks, uint8_t* vt, float* vs, void* scratch_buf, hipStream_t st) {
  SAGE_TRY(check_v_grids(B, S, H));
  float* partial = (float*)scratch_buf;
  if (D == 64) launch_quant_kv<64>(k, v, B, S, H, kq, ks, partial, vs, vt, st);
  else launch_quant_kv<128>(k, v, B, S, H, kq, ks, partial, vs, vt, st);
  return launched("sage_quant_kv");
}

template <int kD, bool kQuantQ, bool kDump = false>
void launch_attn(const int8_t* q8, const float* qs, const void* qraw, const int8_t* k8, const float* ks,
                 const uint8_t* vt, const float* vs, int64_t Sq, int64_t Skv, int64_t H, int nqt, int64_t nwg,
                 float c, float log2_448, void* out, float* lse, hipStream_t st, uint8_t* pdump = nullptr) {
  hipLaunchKernelGGL((sage::attn_fwd_kernel<kD, kQuantQ, kDump>), dim3((unsigned)nwg), dim3(64 * sage::kAttnWaves), 0,
                     st, q8, qs, (const uint16_t*)qraw, k8, ks, vt, vs, (int)Sq, (int)Skv, (int)H, (int)seq_pad(Sq),
                     (int)seq_pad(Skv), nqt, (int)nwg, c, log2_448, (uint16_t*)out, lse, pdump);
}

// Fused attention. Q comes either quantized (q8, qs) or, when qraw is not
// NULL, as bf16 [B, Sq, H, D] that the kernel quantizes itself.
sage_status attn_impl(const int8_t* q8, const float* qs, const void* qraw, const int8_t* k8, const float* ks,
                      const uint8_t* vt, const float* vs, int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                      float softmax_scale, void* out, float* lse, hipStream_t st) {
  const int nqt = (int)((Sq + sage::kQueryTile - 1) / sage::kQueryTile);
  const int64_t nwg = B * H * nqt;
  if (nwg > INT32_MAX) return fail(SAGE_ERR_SHAPE, "grid too large");
  const float c = (float)softmax_scale * (float)1.4426950408889634;  // fl32(fl32(scale) * fl32(log2 e))
  const float log2_448 = (float)std::log2(448.0);
  if (D == 64) {
    if (qraw) launch_attn<64, true>(q8, qs, qraw, k8, ks, vt, vs, Sq, Skv, H, nqt, nwg, c, log2_448, out, lse, st);
    else launch_attn<64, false>(q8, qs, qraw, k8, ks, vt, vs, Sq, Skv, H, nqt, nwg, c, log2_448, out, lse, st);
  } else {
    if (qraw) launch_attn<128, true>(q8, qs, qraw, k8, ks, vt, vs, Sq, Skv, H, nqt, nwg, c, log2_448, out, lse, st);
    else launch_attn<128, false>(q8, qs, qraw, k8, ks, vt, vs, Sq, Skv, H, nqt, nwg, c, log2_448, out, lse, st);
  }
  return launched("sage_attn_fwd");
}

struct WorkspaceEx {
  size_t k8, v8, ks, vs, kmean, scratch_off, scratch_bytes, total;
};

// Intermediates of sage_attention_ex, each 256-byte aligned (no Q region:
// the attention kernel quantizes Q); the scratch region serves sage_quant_v
// and, before it, the K-smoothing block sums.
WorkspaceEx layout_ex(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D) {
  (void)Sq;
  WorkspaceEx w{};
  const int64_t Skp = seq_pad(Skv);
  w.k8 = 0;
  w.v8 = w.k8 + align256((size_t)(B * H * Skp * D));
  w.ks = w.v8 + align256((size_t)(B * H * Skp * D));
  w.vs = w.ks + align256((size_t)(B * H * (Skp / 32)) * 4);
  w.kmean = w.vs + align256((size_t)(B * H * D) * 4);
  w.scratch_off = w.kmean + align256((size_t)(B * H * D) * 4);
  const size_t a = v_scratch_bytes(B, Skv, H, D), b = k_smooth_scratch_bytes(B, Skv, H, D);
  w.scratch_bytes = a > b ? a : b;
  w.total = w.scratch_off + w.scratch_bytes;
  return w;
}

}  // namespace

extern "C" {

int sage_abi_version(void) { return kAbiVersion; }

const char* sage_status_str(int s) {
  switch (s) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_NULL: return "SAGE_ERR_NULL";
    case SAGE_ERR_SHAPE: return "SAGE_ERR_SHAPE";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED";
    case SAGE_ERR_ALIGN: return "SAGE_ERR_ALIGN";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP";
    case SAGE_ERR_RANGE: return "SAGE_ERR_RANGE";
    default: return "SAGE_ERR_UNKNOWN";
  }
}

const char* sage_last_error(void) { return g_last_error; }

int sage_kv_tile(void) { return sage::kKeyTile; }

int64_t sage_seq_pad(int64_t S) { return S < 1 ? 0 : seq_pad(S); }

size_t sage_quant_v_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (check_shape(B, S, H, D) != SAGE_OK) return 0;
  return v_scratch_bytes(B, S, H, D);
}

size_t sage_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (check_shape(B, S, H, D) != SAGE_OK) return 0;
  return layout(B, S, H, D).total;
}

sage_status sage_quant_qk(const void* x, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* x_i8,
                          float* x_scale, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(x, "x"));
  SAGE_TRY(check_ptr(x_i8, "x_i8"));
  SAGE_TRY(check_ptr(x_scale, "x_scale"));
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return quant_qk_impl(x, B, S, H, D, x_i8, x_scale, (hipStream_t)stream);
}

sage_status sage_quant_v(const void* v, int64_t B, int64_t S, int64_t H, int64_t D, uint8_t* v_fp8_t,
                         float* v_scale, void* scratch_buf, size_t scratch_bytes, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(v, "v"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(scratch_buf, "scratch"));
  if (scratch_bytes < v_scratch_bytes(B, S, H, D))
    return fail(SAGE_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes, v_scratch_bytes(B, S, H, D));
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return quant_v_impl(v, B, S, H, D, v_fp8_t, v_scale, scratch_buf, (hipStream_t)stream);
}

sage_status sage_quant_kv(const void* k, const void* v, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* k_i8,
                          float* k_scale, uint8_t* v_fp8_t, float* v_scale, void* scratch_buf, size_t scratch_bytes,
                          void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(k, "k"));
  SAGE_TRY(check_ptr(v, "v"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(scratch_buf, "scratch"));
  if (scratch_bytes < v_scratch_bytes(B, S, H, D))
    return fail(SAGE_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes, v_scratch_bytes(B, S, H, D));
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return quant_kv_impl(k, v, B, S, H, D, k_i8, k_scale, v_fp8_t, v_scale, scratch_buf, (hipStream_t)stream);
}

sage_status sage_quant_v_noalloc(const void* v, int64_t B, int64_t S, int64_t H, int64_t D, uint8_t* v_fp8_t,
                                 float* v_scale, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(v, "v"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  const size_t need = v_scratch_bytes(B, S, H, D);
  if (need > (size_t)SAGE_NOALLOC_SCRATCH_BYTES)
    return fail(SAGE_ERR_WORKSPACE, "needs %zu bytes of scratch, above the %zu-byte static buffer (use sage_quant_v)",
                need, (size_t)SAGE_NOALLOC_SCRATCH_BYTES);
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  void* buf = nullptr;
  SAGE_TRY(noalloc_scratch(&buf));
  return quant_v_impl(v, B, S, H, D, v_fp8_t, v_scale, buf, (hipStream_t)stream);
}

sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                          const uint8_t* v_fp8_t, const float* v_scale, int64_t B, int64_t S, int64_t H,
                          int64_t D, float softmax_scale, void* out, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(q_i8, "q_i8"));
  SAGE_TRY(check_ptr(q_scale, "q_scale"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(out, "out"));
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return attn_impl(q_i8, q_scale, nullptr, k_i8, k_scale, v_fp8_t, v_scale, B, S, S, H, D, softmax_scale, out,
                   nullptr, (hipStream_t)stream);
}

sage_status sage_debug_p_codes(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                               const uint8_t* v_fp8_t, const float* v_scale, int64_t B, int64_t S, int64_t H,
                               int64_t D, float softmax_scale, uint8_t* codes, void* out, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(q_i8, "q_i8"));
  SAGE_TRY(check_ptr(q_scale, "q_scale"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(out, "out"));
  if (!codes) return fail(SAGE_ERR_NULL, "codes is NULL");
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (S > kDebugPMaxSeq) return fail(SAGE_ERR_RANGE, "S above %lld (the code dump is S x S_pad bytes per head)",
                                     (long long)kDebugPMaxSeq);
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  const int nqt = (int)((S + sage::kQueryTile - 1) / sage::kQueryTile);
  const int64_t nwg = B * H * nqt;
  if (nwg > INT32_MAX) return fail(SAGE_ERR_SHAPE, "grid too large");
  const float c = softmax_scale * (float)1.4426950408889634;
  const float log2_448 = (float)std::log2(448.0);
  hipStream_t st = (hipStream_t)stream;
  if (D == 64)
    launch_attn<64, false, true>(q_i8, q_scale, nullptr, k_i8, k_scale, v_fp8_t, v_scale, S, S, H, nqt, nwg, c,
                                 log2_448, out, nullptr, st, codes);
  else
    launch_attn<128, false, true>(q_i8, q_scale, nullptr, k_i8, k_scale, v_fp8_t, v_scale, S, S, H, nqt, nwg, c,
                                  log2_448, out, nullptr, st, codes);
  return launched("sage_debug_p_codes");
}

sage_status sage_attention(const void* q, const void* k, const void* v, int64_t B, int64_t S, int64_t H,
                           int64_t D, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(q, "q"));
  SAGE_TRY(check_ptr(k, "k"));
  SAGE_TRY(check_ptr(v, "v"));
  SAGE_TRY(check_ptr(out, "out"));
  if (!workspace) return fail(SAGE_ERR_NULL, "workspace is NULL");
  if (((uintptr_t)workspace) & 255) return fail(SAGE_ERR_ALIGN, "workspace is not 256-byte aligned");
  const Workspace w = layout(B, S, H, D);
  if (workspace_bytes < w.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  int8_t* k8 = (int8_t*)(ws + w.k8);
  uint8_t* v8 = (uint8_t*)(ws + w.v8);
  float* ks = (float*)(ws + w.ks);
  float* vs = (float*)(ws + w.vs);
  // K and V by the fused pre-pass; Q is quantized inside the attention
  // kernel (each wave's 32 queries are one block).
  SAGE_TRY(quant_kv_impl(k, v, B, S, H, D, k8, ks, v8, vs, ws + w.scratch_off, st));
  return attn_impl(nullptr, nullptr, q, k8, ks, v8, vs, B, S, S, H, D, softmax_scale, out, nullptr, st);
}

sage_status sage_debug_qk_scores(const int8_t* q_i8, const int8_t* k_i8, int64_t B, int64_t S, int64_t H,
                                 int64_t D, int64_t b, int64_t h, int64_t r0, int64_t nr, int64_t c0,
                                 int64_t nc, int32_t* scores, void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(q_i8, "q_i8"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  if (!scores) return fail(SAGE_ERR_NULL, "scores is NULL");
  const int64_t Sp = seq_pad(S);
  if (b < 0 || b >= B || h < 0 || h >= H) return fail(SAGE_ERR_RANGE, "(b, h) outside the tensor");
  if (r0 < 0 || nr < 1 || r0 + nr > Sp || c0 < 0 || nc < 1 || c0 + nc > Sp)
    return fail(SAGE_ERR_RANGE, "window outside [0, S_pad)");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  // query tiles of kQueryTile rows and key tiles of kKeyTile keys covering
  // the window; S_pad is a multiple of both, so every staged row exists
  const int64_t rA = r0 / sage::kQueryTile * sage::kQueryTile, cA = c0 / sage::kKeyTile * sage::kKeyTile;
  const int64_t gy = (r0 + nr - rA + sage::kQueryTile - 1) / sage::kQueryTile;
  const int64_t gx = (c0 + nc - cA + sage::kKeyTile - 1) / sage::kKeyTile;
  if (gx > INT32_MAX || gy > 65535) return fail(SAGE_ERR_RANGE, "window too large");
  hipStream_t st = (hipStream_t)stream;
  if (D == 64)
    hipLaunchKernelGGL(sage::debug_qk_kernel<64>, dim3((unsigned)gx, (unsigned)gy), dim3(64 * sage::kAttnWaves), 0,
                       st, q_i8, k_i8, (int)Sp, b * H + h, (int)rA, (int)r0, (int)nr, (int)cA, (int)c0, (int)nc,
                       scores);
  else
    hipLaunchKernelGGL(sage::debug_qk_kernel<128>, dim3((unsigned)gx, (unsigned)gy), dim3(64 * sage::kAttnWaves), 0,
                       st, q_i8, k_i8, (int)Sp, b * H + h, (int)rA, (int)r0, (int)nr, (int)cA, (int)c0, (int)nc,
                       scores);
  return launched("sage_debug_qk_scores");
}

sage_status sage_debug_fp8_dot(const uint8_t* a, const uint8_t* b, int64_t n, const float* init, float* out,
                               void* stream) {
  SAGE_TRY(check_ptr(a, "a"));
  SAGE_TRY(check_ptr(b, "b"));
  if (!init) return fail(SAGE_ERR_NULL, "init is NULL");
  if (!out) return fail(SAGE_ERR_NULL, "out is NULL");
  if ((((uintptr_t)init) | ((uintptr_t)out)) & 3) return fail(SAGE_ERR_ALIGN, "init or out is not 4-byte aligned");
  if (n < 1 || n > kDebugDotMax) return fail(SAGE_ERR_RANGE, "n must be in [1, %lld]", (long long)kDebugDotMax);
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  hipLaunchKernelGGL(sage::debug_fp8_dot_kernel, dim3((unsigned)((n + 31) / 32)), dim3(64), 0, (hipStream_t)stream,
                     a, b, n, init, out);
  return launched("sage_debug_fp8_dot");
}

size_t sage_k_smooth_scratch_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (check_shape(B, S, H, D) != SAGE_OK) return 0;
  return k_smooth_scratch_bytes(B, S, H, D);
}

sage_status sage_quant_k_smooth(const void* k, int64_t B, int64_t S, int64_t H, int64_t D, int8_t* k_i8,
                                float* k_scale, float* k_mean, void* scratch_buf, size_t scratch_bytes,
                                void* stream) {
  SAGE_TRY(check_shape(B, S, H, D));
  SAGE_TRY(check_ptr(k, "k"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(k_mean, "k_mean"));
  SAGE_TRY(check_ptr(scratch_buf, "scratch"));
  if (scratch_bytes < k_smooth_scratch_bytes(B, S, H, D))
    return fail(SAGE_ERR_WORKSPACE, "scratch has %zu bytes, needs %zu", scratch_bytes,
                k_smooth_scratch_bytes(B, S, H, D));
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return quant_k_smooth_impl(k, B, S, H, D, k_i8, k_scale, k_mean, scratch_buf, (hipStream_t)stream);
}

sage_status sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                             const uint8_t* v_fp8_t, const float* v_scale, int64_t B, int64_t Sq, int64_t Skv,
                             int64_t H, int64_t D, float softmax_scale, void* out, float* lse, void* stream) {
  SAGE_TRY(check_shape(B, Sq, H, D));
  SAGE_TRY(check_shape(B, Skv, H, D));
  SAGE_TRY(check_ptr(q_i8, "q_i8"));
  SAGE_TRY(check_ptr(q_scale, "q_scale"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(out, "out"));
  if (lse && (((uintptr_t)lse) & 3)) return fail(SAGE_ERR_ALIGN, "lse is not 4-byte aligned");
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return attn_impl(q_i8, q_scale, nullptr, k_i8, k_scale, v_fp8_t, v_scale, B, Sq, Skv, H, D, softmax_scale, out,
                   lse, (hipStream_t)stream);
}

size_t sage_workspace_bytes_ex(int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D) {
  if (check_shape(B, Sq, H, D) != SAGE_OK || check_shape(B, Skv, H, D) != SAGE_OK) return 0;
  return layout_ex(B, Sq, Skv, H, D).total;
}

sage_status sage_attention_ex(const void* q, const void* k, const void* v, int64_t B, int64_t Sq, int64_t Skv,
                              int64_t H, int64_t D, float softmax_scale, unsigned flags, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  SAGE_TRY(check_shape(B, Sq, H, D));
  SAGE_TRY(check_shape(B, Skv, H, D));
  SAGE_TRY(check_ptr(q, "q"));
  SAGE_TRY(check_ptr(k, "k"));
  SAGE_TRY(check_ptr(v, "v"));
  SAGE_TRY(check_ptr(out, "out"));
  if (flags & ~(unsigned)SAGE_SMOOTH_K) return fail(SAGE_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if (lse && (((uintptr_t)lse) & 3)) return fail(SAGE_ERR_ALIGN, "lse is not 4-byte aligned");
  if (!workspace) return fail(SAGE_ERR_NULL, "workspace is NULL");
  if (((uintptr_t)workspace) & 255) return fail(SAGE_ERR_ALIGN, "workspace is not 256-byte aligned");
  const WorkspaceEx w = layout_ex(B, Sq, Skv, H, D);
  if (workspace_bytes < w.total)
    return fail(SAGE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, w.total);
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  char* ws = (char*)workspace;
  hipStream_t st = (hipStream_t)stream;
  int8_t* k8 = (int8_t*)(ws + w.k8);
  uint8_t* v8 = (uint8_t*)(ws + w.v8);
  float* ks = (float*)(ws + w.ks);
  float* vs = (float*)(ws + w.vs);
  if (flags & SAGE_SMOOTH_K) {
    SAGE_TRY(quant_k_smooth_impl(k, B, Skv, H, D, k8, ks, (float*)(ws + w.kmean), ws + w.scratch_off, st));
    SAGE_TRY(quant_v_impl(v, B, Skv, H, D, v8, vs, ws + w.scratch_off, st));
  } else {
    SAGE_TRY(quant_kv_impl(k, v, B, Skv, H, D, k8, ks, v8, vs, ws + w.scratch_off, st));
  }
  return attn_impl(nullptr, nullptr, q, k8, ks, v8, vs, B, Sq, Skv, H, D, softmax_scale, out, lse, st);
}

sage_status sage_attn_fwd_qbf16(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8_t,
                                const float* v_scale, int64_t B, int64_t Sq, int64_t Skv, int64_t H, int64_t D,
                                float softmax_scale, void* out, float* lse, void* stream) {
  SAGE_TRY(check_shape(B, Sq, H, D));
  SAGE_TRY(check_shape(B, Skv, H, D));
  SAGE_TRY(check_ptr(q, "q"));
  SAGE_TRY(check_ptr(k_i8, "k_i8"));
  SAGE_TRY(check_ptr(k_scale, "k_scale"));
  SAGE_TRY(check_ptr(v_fp8_t, "v_fp8_t"));
  SAGE_TRY(check_ptr(v_scale, "v_scale"));
  SAGE_TRY(check_ptr(out, "out"));
  if (lse && (((uintptr_t)lse) & 3)) return fail(SAGE_ERR_ALIGN, "lse is not 4-byte aligned");
  if (!(std::isfinite(softmax_scale) && softmax_scale >= 0.0f))
    return fail(SAGE_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  if (forced_launch_failure()) return fail(SAGE_ERR_HIP, "forced launch failure (SAGE_TEST_FAIL_LAUNCH)");
  return attn_impl(nullptr, nullptr, q, k_i8, k_scale, v_fp8_t, v_scale, B, Sq, Skv, H, D, softmax_scale, out, lse,
                   (hipStream_t)stream);
}

}  // extern "C"
