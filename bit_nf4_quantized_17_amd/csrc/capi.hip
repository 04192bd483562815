// capi.hip -- the C ABI of libqlora_nf4 (declared in include/qlora_nf4.h):
// host-side validation, workspace layout and kernel launches.  Nothing here
// allocates, frees or synchronises; every launch goes on the caller's stream.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>
#include <string>

#include "../../include/qlora_nf4.h"
#include "common.h"

using namespace qln;

namespace {

thread_local std::string g_err;

struct TimingHook {
  hipEvent_t fwd_begin = nullptr, fwd_end = nullptr, dx_begin = nullptr, dx_end = nullptr;
};
thread_local TimingHook g_hook;

void record(hipEvent_t ev, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev, st);
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return QL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

constexpr int64_t kMaxGridY = 65535;

int check_weight(const qlora_nf4_weight* w) {
  if (!w) return fail(QL_ERR_NULL, "weight descriptor is NULL");
  if (w->block != 64 || (w->dq_block != 256 && w->dq_block != 0))
    return fail(QL_ERR_UNSUPPORTED, "block=%d dq_block=%d (block 64; dq_block 256, or 0 for fp32 scales)",
                w->block, w->dq_block);
  if (w->codebook != QL_CODEBOOK_NF4 && w->codebook != QL_CODEBOOK_INT4)
    return fail(QL_ERR_UNSUPPORTED, "codebook=%d", w->codebook);
  if (w->dq_format != QL_DQ_E4M3 && w->dq_format != QL_DQ_UINT8)
    return fail(QL_ERR_UNSUPPORTED, "dq_format=%d (QL_DQ_E4M3 or QL_DQ_UINT8)", w->dq_format);
  if (!w->codes || (w->dq_block && !w->qscale) || !w->dscale)
    return fail(QL_ERR_NULL, "weight buffer is NULL");
  if (w->rows <= 0 || w->cols <= 0 || w->cols % 64)
    return fail(QL_ERR_SHAPE, "weight shape %lld x %lld (need positive, cols %% 64 == 0)",
                (long long)w->rows, (long long)w->cols);
  if (!aligned16(w->codes) || (w->dq_block && !aligned16(w->qscale)) || !aligned16(w->dscale))
    return fail(QL_ERR_ALIGN, "weight buffers must be 16-byte aligned");
  return QL_OK;
}

NF4View view(const qlora_nf4_weight* w) {
  NF4View v;
  v.codes = w->codes;
  v.qscale = w->dq_block ? w->qscale : nullptr;
  v.fp32_scale = w->dq_block == 0;
  v.u8_scale = w->dq_block != 0 && w->dq_format == QL_DQ_UINT8;
  const uint32_t* bits = codebook_bits(w->codebook);
  for (int i = 0; i < 16; ++i) std::memcpy(&v.lv[i], &bits[i], 4);
  v.dscale = w->dscale;
  v.N = w->rows;
  v.K = w->cols;
  return v;
}

int check_layer(const qlora_nf4_weight* w, int64_t M, int r, int compute_dtype) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (M <= 0) return fail(QL_ERR_SHAPE, "M=%lld must be positive", (long long)M);
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QL_ERR_UNSUPPORTED, "r=%d outside [1, %d]", r, QLORA_MAX_RANK);
  if (compute_dtype != QL_DTYPE_BF16)
    return fail(QL_ERR_UNSUPPORTED, "compute_dtype=%d (only QL_DTYPE_BF16)", compute_dtype);
  if ((w->rows + 127) / 128 > kMaxGridY || (w->cols + 127) / 128 > kMaxGridY)
    return fail(QL_ERR_SHAPE, "weight dimension too large");
  if ((M + 127) / 128 > 0x7fffffffLL) return fail(QL_ERR_SHAPE, "M too large");
  return QL_OK;
}

// forward workspace: the split-K partials of T (of the tiled path, or of the
// decode path at M <= 16)
size_t fwd_ws(int64_t M, int64_t N, int64_t K, int r) {
  (void)N;
  size_t b = (size_t)skinny_partial_elems(M, K, r) * sizeof(float);
  if (M <= 16) b = std::max(b, decode_ws_bytes(K, r));
  return align256(b);
}

// backward workspace: U fp32 [M][r] | T fp32 [M][r] (when recomputed) | fp32 split partials
struct BwdLayout {
  size_t u_off, t_off, part_off, total;
};

BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K, int r) {
  BwdLayout L;
  const size_t mr = align256((size_t)M * (size_t)r * sizeof(float));
  int64_t parts = std::max({skinny_partial_elems(M, N, r), skinny_partial_elems(N, M, r),
                            skinny_partial_elems(K, M, r), skinny_partial_elems(M, K, r)});
  L.u_off = 0;
  L.t_off = mr;
  L.part_off = 2 * mr;
  L.total = L.part_off + align256((size_t)parts * sizeof(float));
  return L;
}

// checks shared by both backward entry points (all but the workspace)
int check_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
              const uint16_t* A, const uint16_t* B, int r, int compute_dtype, const float* T_saved,
              const uint16_t* dX, const uint16_t* dA, const uint16_t* dB) {
  int rc = check_layer(w, M, r, compute_dtype);
  if (rc) return rc;
  if (!X || !dY || !A || !B || !dA || !dB) return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(X) || !aligned16(dY) || !aligned16(A) || !aligned16(B) || !aligned16(dA) ||
      !aligned16(dB) || (T_saved && !aligned16(T_saved)) || (dX && !aligned16(dX)))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return QL_OK;
}

// the backward's launches over a workspace of bwd_layout(M, N, K, r).total bytes
int run_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
            const uint16_t* A, const uint16_t* B, int r, float alpha, const float* T_saved,
            uint16_t* dX, uint16_t* dA, uint16_t* dB, char* ws, hipStream_t st) {
  const int64_t N = w->rows, K = w->cols;
  const BwdLayout L = bwd_layout(M, N, K, r);
  float* U = (float*)(ws + L.u_off);
  float* part = (float*)(ws + L.part_off);
  const float s = alpha / (float)r;
  const float* T = T_saved;
  hipError_t e;
  if (!T) {
    float* Tw = (float*)(ws + L.t_off);
    e = launch_lora_down(X, A, M, K, r, part, Tw, st);
    if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd: T recompute launch");
    T = Tw;
  }
  e = launch_lora_u(dY, B, M, N, r, part, U, st);
  if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd: U launch");
  e = launch_lora_db(dY, T, M, N, r, s, part, dB, st);
  if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd: dB launch");
  if (dX) {
    record(g_hook.dx_begin, st);
    e = launch_dx_main(view(w), dY, M, U, A, r, s, dX, st);
    record(g_hook.dx_end, st);
    if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd: dX launch");
  }
  e = launch_lora_da(U, X, M, K, r, s, part, dA, st);
  return hip_status(e, "qlora_linear_bwd: dA launch");
}

// Scratch of the allocation-free backward: a fixed array in the library's
// device data, one copy per GPU (made when the code object is loaded on it
// and held until the process ends).  Its host-side name is a stand-in, not a
// device address; the address comes from hipGetSymbolAddress, resolved on
// the first call on each device with that device current and kept per
// device.  No part of it needs to start at zero: within one call every
// kernel writes each scratch element before any kernel of the call reads it.
static __device__ __align__(256) unsigned char scratch[QLORA_BWD_NOALLOC_MAX_BYTES];

int scratch_of_current_device(char** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QL_ERR_UNSUPPORTED, "device %d (the scratch table covers devices 0..%d)", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "qlora_linear_bwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(QL_ERR_HIP, "qlora_linear_bwd_noalloc: hipGetSymbolAddress(scratch) gave NULL");
    addr[dev] = (char*)p;
  }
  *out = addr[dev];
  return QL_OK;
}

}  // namespace

extern "C" {

int qlora_abi_version(void) { return QLORA_ABI_VERSION; }

int qlora_set_timing_events(void* fwd_begin, void* fwd_end, void* dx_begin, void* dx_end) {
  g_hook.fwd_begin = (hipEvent_t)fwd_begin;
  g_hook.fwd_end = (hipEvent_t)fwd_end;
  g_hook.dx_begin = (hipEvent_t)dx_begin;
  g_hook.dx_end = (hipEvent_t)dx_end;
  return ok();
}

const char* qlora_last_error(void) { return g_err.c_str(); }

void nf4_levels(float out[16]) {
  if (!out) return;
  for (int i = 0; i < 16; ++i) std::memcpy(&out[i], &kNF4LevelBits[i], 4);
}

int qlora_codebook_levels(int codebook, float out[16]) {
  if (codebook != QL_CODEBOOK_NF4 && codebook != QL_CODEBOOK_INT4)
    return fail(QL_ERR_UNSUPPORTED, "codebook=%d", codebook);
  if (!out) return fail(QL_ERR_NULL, "output is NULL");
  const uint32_t* bits = codebook_bits(codebook);
  for (int i = 0; i < 16; ++i) std::memcpy(&out[i], &bits[i], 4);
  return ok();
}

int nf4_storage_bytes(int64_t rows, int64_t cols, int block, int dq_block, size_t* codes_bytes,
                      size_t* qscale_bytes, size_t* dscale_bytes) {
  if (block != 64 || (dq_block != 256 && dq_block != 0))
    return fail(QL_ERR_UNSUPPORTED, "block=%d dq_block=%d (block 64; dq_block 256, or 0 for fp32 scales)",
                block, dq_block);
  if (rows <= 0 || cols <= 0 || cols % 64)
    return fail(QL_ERR_SHAPE, "shape %lld x %lld (need positive, cols %% 64 == 0)",
                (long long)rows, (long long)cols);
  const int64_t nb = rows * cols / 64;
  if (codes_bytes) *codes_bytes = (size_t)(rows * cols / 2);
  if (qscale_bytes) *qscale_bytes = dq_block ? (size_t)nb : 0;
  if (dscale_bytes) *dscale_bytes = (size_t)(dq_block ? (nb + 255) / 256 : nb) * sizeof(float);
  return ok();
}

int qlora_quantize(const float* W, int64_t rows, int64_t cols, int codebook, int dq_block,
                   int dq_format, uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax_out,
                   void* stream) {
  if (dq_block != 256 && dq_block != 0)
    return fail(QL_ERR_UNSUPPORTED, "dq_block=%d (256, or 0 for fp32 scales)", dq_block);
  if (dq_format != QL_DQ_E4M3 && dq_format != QL_DQ_UINT8)
    return fail(QL_ERR_UNSUPPORTED, "dq_format=%d (QL_DQ_E4M3 or QL_DQ_UINT8)", dq_format);
  if (codebook != QL_CODEBOOK_NF4 && codebook != QL_CODEBOOK_INT4)
    return fail(QL_ERR_UNSUPPORTED, "codebook=%d", codebook);
  if (!W || !codes || (dq_block && !qscale) || !dscale) return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (rows <= 0 || cols <= 0 || cols % 64)
    return fail(QL_ERR_SHAPE, "shape %lld x %lld (need positive, cols %% 64 == 0)",
                (long long)rows, (long long)cols);
  if ((rows * cols / 64 + 255) / 256 > 0x7fffffffLL) return fail(QL_ERR_SHAPE, "weight too large");
  if (!aligned16(W) || !aligned16(codes) || (dq_block && !aligned16(qscale)) || !aligned16(dscale) ||
      (absmax_out && !aligned16(absmax_out)))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const int fmt = dq_block == 0 ? SCALE_FP32 : dq_format == QL_DQ_UINT8 ? SCALE_U8 : SCALE_E4M3;
  return hip_status(launch_quantize(W, rows, cols, codebook, fmt, codes, qscale, dscale,
                                    absmax_out, (hipStream_t)stream),
                    "qlora_quantize launch");
}

int nf4_quantize(const float* W, int64_t rows, int64_t cols, int block, int dq_block,
                 uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax_out, void* stream) {
  if (block != 64 || (dq_block != 256 && dq_block != 0))
    return fail(QL_ERR_UNSUPPORTED, "block=%d dq_block=%d (block 64; dq_block 256, or 0 for fp32 scales)",
                block, dq_block);
  return qlora_quantize(W, rows, cols, QL_CODEBOOK_NF4, dq_block, QL_DQ_E4M3, codes, qscale, dscale, absmax_out,
                        stream);
}

int nf4_dequantize(const qlora_nf4_weight* w, uint16_t* W_bf16, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (!W_bf16) return fail(QL_ERR_NULL, "output is NULL");
  if ((w->rows * w->cols / 64 + 255) / 256 > 0x7fffffffLL) return fail(QL_ERR_SHAPE, "weight too large");
  if (!aligned16(W_bf16)) return fail(QL_ERR_ALIGN, "output must be 16-byte aligned");
  return hip_status(launch_dequantize(view(w), W_bf16, (hipStream_t)stream), "nf4_dequantize launch");
}

int qlora_merge(const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B, int r, float alpha,
                uint16_t* W_out, void* stream) {
  int rc = check_weight(w);
  if (rc) return rc;
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QL_ERR_UNSUPPORTED, "r=%d outside [1, %d]", r, QLORA_MAX_RANK);
  if (!A || !B || !W_out) return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_out))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (!merge_fits(w->rows, w->cols, r)) return fail(QL_ERR_SHAPE, "weight or adapter too large (32-bit offsets)");
  return hip_status(launch_merge(view(w), A, B, r, alpha / (float)r, W_out, (hipStream_t)stream),
                    "qlora_merge launch");
}

int qlora_unmerge(const uint16_t* W_merged, int64_t rows, int64_t cols, const uint16_t* A,
                  const uint16_t* B, int r, float alpha, uint16_t* W_out, void* stream) {
  if (rows <= 0 || cols <= 0 || cols % 8)
    return fail(QL_ERR_SHAPE, "weight shape %lld x %lld (need positive, cols %% 8 == 0)", (long long)rows,
                (long long)cols);
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QL_ERR_UNSUPPORTED, "r=%d outside [1, %d]", r, QLORA_MAX_RANK);
  if (!W_merged || !A || !B || !W_out) return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(W_merged) || !aligned16(A) || !aligned16(B) || !aligned16(W_out))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (!merge_fits(rows, cols, r)) return fail(QL_ERR_SHAPE, "weight or adapter too large (32-bit offsets)");
  return hip_status(launch_unmerge(W_merged, rows, cols, A, B, r, alpha / (float)r, W_out, (hipStream_t)stream),
                    "qlora_unmerge launch");
}

size_t qlora_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 1 || r > QLORA_MAX_RANK) return 0;
  return fwd_ws(M, N, K, r);
}

int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t M, const uint16_t* A,
                     const uint16_t* B, int r, float alpha, int compute_dtype, uint16_t* Y,
                     float* T_save, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layer(w, M, r, compute_dtype);
  if (rc) return rc;
  if (!X || !A || !B || !Y || !T_save) return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(X) || !aligned16(A) || !aligned16(B) || !aligned16(Y) || !aligned16(T_save))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t need = fwd_ws(M, w->rows, w->cols, r);
  if (need && (!workspace || workspace_bytes < need))
    return fail(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (workspace && !aligned16(workspace)) return fail(QL_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const float s = alpha / (float)r;
  if (decode_fits(M, view(w), r)) {   // decode sizes: T partials, then one weight-streaming launch
    record(g_hook.fwd_begin, st);
    hipError_t e = launch_decode(view(w), X, M, A, B, r, s, Y, T_save, (float*)workspace, st);
    record(g_hook.fwd_end, st);
    return hip_status(e, "qlora_linear_fwd: decode launch");
  }
  hipError_t e = launch_lora_down(X, A, M, w->cols, r, (float*)workspace, T_save, st);
  if (e != hipSuccess) return hip_status(e, "qlora_linear_fwd: lora_down launch");
  record(g_hook.fwd_begin, st);
  e = launch_fwd_main(view(w), X, M, T_save, B, r, s, Y, st);
  record(g_hook.fwd_end, st);
  return hip_status(e, "qlora_linear_fwd: main launch");
}

int qlora_dual_fwd(const qlora_nf4_weight* w_gate, const qlora_nf4_weight* w_up, const uint16_t* X,
                   int64_t M, const uint16_t* A_gate, const uint16_t* B_gate, const uint16_t* A_up,
                   const uint16_t* B_up, int r, float alpha, int compute_dtype, int epilogue,
                   uint16_t* Y_gate, uint16_t* Y_up, uint16_t* H, float* T_gate_save,
                   float* T_up_save, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layer(w_gate, M, r, compute_dtype);
  if (rc) return rc;
  rc = check_weight(w_up);
  if (rc) return rc;
  if (w_up->rows != w_gate->rows || w_up->cols != w_gate->cols)
    return fail(QL_ERR_SHAPE, "gate %lld x %lld and up %lld x %lld weights differ in shape",
                (long long)w_gate->rows, (long long)w_gate->cols, (long long)w_up->rows,
                (long long)w_up->cols);
  if (epilogue != QL_DUAL_SEPARATE && epilogue != QL_DUAL_SWIGLU)
    return fail(QL_ERR_UNSUPPORTED, "epilogue=%d (QL_DUAL_SEPARATE or QL_DUAL_SWIGLU)", epilogue);
  uint16_t* out1 = epilogue == QL_DUAL_SEPARATE ? Y_gate : H;
  uint16_t* out2 = epilogue == QL_DUAL_SEPARATE ? Y_up : nullptr;
  if (!X || !A_gate || !B_gate || !A_up || !B_up || !T_gate_save || !T_up_save || !out1 ||
      (epilogue == QL_DUAL_SEPARATE && !out2))
    return fail(QL_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(X) || !aligned16(A_gate) || !aligned16(B_gate) || !aligned16(A_up) ||
      !aligned16(B_up) || !aligned16(T_gate_save) || !aligned16(T_up_save) || !aligned16(out1) ||
      (out2 && !aligned16(out2)))
    return fail(QL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const int64_t N = w_gate->rows, K = w_gate->cols;
  if ((N + 256) * K / 2 >= ((int64_t)1 << 31) || K * 2 * 512 >= ((int64_t)1 << 31))
    return fail(QL_ERR_SHAPE, "weight too large for the dual kernel (32-bit offsets)");
  const size_t need = align256((size_t)skinny_partial_elems(M, K, r) * sizeof(float));
  if (need && (!workspace || workspace_bytes < need))
    return fail(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if (workspace && !aligned16(workspace)) return fail(QL_ERR_ALIGN, "workspace must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_lora_down(X, A_gate, M, K, r, (float*)workspace, T_gate_save, st);
  if (e == hipSuccess) e = launch_lora_down(X, A_up, M, K, r, (float*)workspace, T_up_save, st);
  if (e != hipSuccess) return hip_status(e, "qlora_dual_fwd: lora_down launch");
  record(g_hook.fwd_begin, st);
  e = launch_fwd_dual(view(w_gate), view(w_up), X, M, T_gate_save, T_up_save, B_gate, B_up, r,
                      alpha / (float)r, epilogue == QL_DUAL_SEPARATE ? 1 : 2, out1, out2, st);
  record(g_hook.fwd_end, st);
  return hip_status(e, "qlora_dual_fwd: main launch");
}

int qlora_adamw_step(const qlora_adamw_tensor* tensors, int count, float lr, float beta1,
                     float beta2, float eps, float weight_decay, int step, void* stream) {
  if (count < 0) return fail(QL_ERR_SHAPE, "count=%d", count);
  if (count > 0 && !tensors) return fail(QL_ERR_NULL, "tensor list is NULL");
  if (step < 1) return fail(QL_ERR_UNSUPPORTED, "step=%d (counts from 1)", step);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps >= 0.0f) ||
      !std::isfinite(lr) || !std::isfinite(weight_decay))
    return fail(QL_ERR_UNSUPPORTED, "hyperparameters out of range (0 <= beta < 1, eps >= 0, finite lr, wd)");
  std::vector<AdamwTensor> ts((size_t)count);
  for (int i = 0; i < count; ++i) {
    const qlora_adamw_tensor& t = tensors[i];
    if (t.numel < 0 || t.numel >= ((int64_t)1 << 40)) return fail(QL_ERR_SHAPE, "tensor %d: numel=%lld", i, (long long)t.numel);
    if (t.numel > 0 && (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq))
      return fail(QL_ERR_NULL, "tensor %d: a required pointer is NULL", i);
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg) || !aligned16(t.exp_avg_sq) ||
        (t.master && !aligned16(t.master)))
      return fail(QL_ERR_ALIGN, "tensor %d: device pointers must be 16-byte aligned", i);
    ts[i] = AdamwTensor{t.param, t.grad, t.exp_avg, t.exp_avg_sq, t.master, t.numel};
  }
  return hip_status(launch_adamw(ts.data(), count, lr, beta1, beta2, eps, weight_decay, step,
                                 (hipStream_t)stream),
                    "qlora_adamw_step launch");
}

size_t qlora_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  if (M <= 0 || N <= 0 || K <= 0 || r < 1 || r > QLORA_MAX_RANK) return 0;
  return bwd_layout(M, N, K, r).total;
}

int qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY, int64_t M,
                     const uint16_t* A, const uint16_t* B, int r, float alpha, int compute_dtype,
                     const float* T_saved, uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_bwd(w, X, dY, M, A, B, r, compute_dtype, T_saved, dX, dA, dB);
  if (rc) return rc;
  if (!workspace) return fail(QL_ERR_NULL, "workspace is NULL");
  if (!aligned16(workspace)) return fail(QL_ERR_ALIGN, "workspace must be 16-byte aligned");
  const size_t need = bwd_layout(M, w->rows, w->cols, r).total;
  if (workspace_bytes < need)
    return fail(QL_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  return run_bwd(w, X, dY, M, A, B, r, alpha, T_saved, dX, dA, dB, (char*)workspace,
                 (hipStream_t)stream);
}

int qlora_linear_bwd_noalloc(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                             int compute_dtype, const float* T_saved, uint16_t* dX, uint16_t* dA,
                             uint16_t* dB, void* stream) {
  int rc = check_bwd(w, X, dY, M, A, B, r, compute_dtype, T_saved, dX, dA, dB);
  if (rc) return rc;
  const size_t need = bwd_layout(M, w->rows, w->cols, r).total;
  if (need > (size_t)QLORA_BWD_NOALLOC_MAX_BYTES)
    return fail(QL_ERR_WORKSPACE, "the backward needs %zu bytes of scratch; the allocation-free "
                "entry point holds %zu (use qlora_linear_bwd with a workspace)",
                need, (size_t)QLORA_BWD_NOALLOC_MAX_BYTES);
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc) return rc;
  return run_bwd(w, X, dY, M, A, B, r, alpha, T_saved, dX, dA, dB, ws, (hipStream_t)stream);
}

}  // extern "C"
