/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA NF4 linear layer.
 *
 * One frozen weight W [rows = N = out_features][cols = K = in_features] is
 * stored as 4-bit NormalFloat codes with one absmax scale per block of 64
 * consecutive weights of a row, and those block scales are themselves stored
 * as 8-bit floats with one fp32 constant per group of 256 blocks.  The layer
 * computes, for activations X [M][K] and LoRA adapters A [r][K], B [N][r]:
 *
 *   forward   Y  = X W'^T + s (X A^T) B^T,          s = alpha / r
 *   backward  dX = dY W' + s (dY B) A
 *             dA = s (dY B)^T X,   dB = s dY^T (X A^T)     (no gradient for W)
 *
 * where W' is the bfloat16 dequantized weight.  Sources (cited by page title
 * and section):
 *  - Ultralytics glossary "QLoRA", section "How QLoRA works": NF4 codes at
 *    normal quantiles with one absmax scale per 64 weights; double
 *    quantization of the scales to 8 bits in blocks of 256; the forward pass
 *    dequantizes NF4 to bfloat16 right before the matrix product and adds the
 *    LoRA path; the backward pass computes gradients through the dequantized
 *    weights and updates only the two low-rank matrices.  Its closing note:
 *    bnb_4bit_compute_dtype = bfloat16.
 *  - vnread "Grokking QLoRA", section "Double Quantization": the second-level
 *    format is FP8 (read here as OCP E4M3, largest scale of a group -> 448).
 *  - Hugging Face Transformers docs "Bitsandbytes", section "QLoRA" (compute
 *    data type, NF4, nested quantization) and the section on dequantizing a
 *    model back to its original precision.
 *  - IBM "What is LoRA?", PEFT parameters r and lora_alpha ("the scaling
 *    factor"); ezsol "Mastering model fine-tuning", LoRA section: Delta W = B A.
 *
 * Conventions for every call:
 *  - All tensors are dense row-major.  bf16 tensors are passed as uint16_t bit
 *    patterns.  Pointers are DEVICE pointers unless stated otherwise; the
 *    caller owns every buffer (the library never allocates, frees or
 *    synchronises).  Work is enqueued on `stream` (a hipStream_t; NULL means
 *    the null stream) and the call returns at once.
 *  - Validation happens on the host before anything is enqueued: a failing
 *    call enqueues nothing, returns a negative qlora_status and leaves a
 *    message for qlora_last_error().  A launch failure reported by the HIP
 *    runtime returns QL_ERR_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation.
 *  - Preconditions that are documented, not checked: inputs are finite;
 *    outputs do not overlap inputs or each other.
 *  - Device pointers must be 16-byte aligned (QL_ERR_ALIGN otherwise).
 *  - Library state: the compute calls keep no state between calls, so
 *    concurrent calls on different streams are safe as long as they do not
 *    share a workspace or an output buffer (a workspace is scratch for one
 *    call at a time).  Two pieces of state exist: the benchmark timing hook
 *    of qlora_set_timing_events (thread-local HIP event handles that later
 *    calls on the same thread record; empty unless a caller sets it), and
 *    the per-GPU scratch array of qlora_linear_bwd_noalloc, which all calls
 *    of that entry point on one GPU share.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_ABI_VERSION 3

typedef enum {
  QL_OK = 0,
  QL_ERR_NULL = -1,         /* a required pointer is NULL                          */
  QL_ERR_SHAPE = -2,        /* a size is non-positive, or cols % 64 != 0           */
  QL_ERR_UNSUPPORTED = -3,  /* block, dq_block, codebook, dtype or r out of range  */
  QL_ERR_ALIGN = -4,        /* a device pointer is not 16-byte aligned             */
  QL_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required          */
  QL_ERR_HIP = -6           /* the HIP runtime reported an error at launch         */
} qlora_status;

enum { QL_DTYPE_BF16 = 1 };  /* the only compute dtype: bfloat16 operands, fp32 sums */

#define QLORA_MAX_RANK 128

/* Codebooks: the 16 levels a 4-bit code indexes (qlora_codebook_levels()).
 * NF4 is the QLoRA data type; INT4 is the evenly spaced comparison codebook
 * of the Ultralytics "QLoRA" encoding snippet. */
enum { QL_CODEBOOK_NF4 = 0, QL_CODEBOOK_INT4 = 1 };

/* Second-level (double-quantization) formats of the 8-bit block scales.
 * The Ultralytics "QLoRA" double-quantization bullet says "8 bits, blocks of
 * 256"; vnread "Grokking QLoRA", "Double Quantization", names FP8:
 *  QL_DQ_E4M3  (0): OCP FP8 E4M3; per group d = max / 448, q = E4M3(a / d),
 *                   restored fl32(E4M3(q) * d).
 *  QL_DQ_UINT8 (1): the plain integer reading; per group d = fl32(max / 255),
 *                   q = min(255, round-half-even(fl32(a / d))) (0 if d = 0),
 *                   restored fl32(q * d). */
enum { QL_DQ_E4M3 = 0, QL_DQ_UINT8 = 1 };

/* A quantized frozen weight W [rows = N][cols = K] (device pointers).
 *  codes  : N*K/2 bytes; byte e/2 holds flattened element e, even e in the low
 *           nibble; the code indexes the 16 levels of `codebook`.
 *  block  : must be 64 (block b covers flattened elements [64b, 64b+64),
 *           always inside one row because K % 64 == 0); nb = N*K/64.
 *  dq_block = 256 (double quantization, the QLoRA default):
 *    qscale : nb bytes, the 8-bit code of each block's scale in dq_format:
 *             an OCP FP8 E4M3 code at most 0x7E (448, what nf4_quantize
 *             writes; the sign bit and the E4M3 NaN code 0x7F are not valid
 *             scales), or (QL_DQ_UINT8) an integer 0..255;
 *    dscale : ng = ceil(nb/256) fp32; group g covers blocks [256g, 256g+256)
 *             (the last may be shorter); restored block scale is
 *             fl32(v(qscale[b]) * dscale[b/256]), v the code's value.
 *  dq_block = 0 (no double quantization; Transformers "Bitsandbytes", 4-bit
 *    section, nested quantization off):
 *    qscale : unused, may be NULL;
 *    dscale : nb fp32, the block scales (each block's exact absmax).
 *  codebook: QL_CODEBOOK_NF4 (0, the default of a zero-initialised
 *    descriptor) or QL_CODEBOOK_INT4.
 *  dq_format: QL_DQ_E4M3 (0, the default) or QL_DQ_UINT8; read only when
 *    dq_block = 256. */
typedef struct {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* dscale;
  int64_t rows, cols;
  int32_t block, dq_block;
  int32_t codebook;
  int32_t dq_format;
} qlora_nf4_weight;

/* ABI version (QLORA_ABI_VERSION of the built library). */
int qlora_abi_version(void);

/* Message describing the last non-OK status returned on this thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* qlora_last_error(void);

/* The 16 NF4 levels in code order (host memory, 16 floats).  Ultralytics
 * "QLoRA", "How QLoRA works" (the level-building snippet): quantiles of the
 * standard normal at probabilities evenly spaced from 0.9677083 towards 0.5 --
 * 8 positive, 7 negative -- plus an exact zero, sorted and divided by the
 * largest, each rounded once to fp32.  Code 0 is -1, code 7 is +0, code 15 is +1. */
void nf4_levels(float out[16]);

/* The 16 levels of a codebook in code order (host memory, 16 floats): NF4 as
 * nf4_levels(); INT4 is L[i] = -1 + 2 i / 15 rounded once to fp32 (no zero
 * level).  Returns QL_OK, QL_ERR_UNSUPPORTED or QL_ERR_NULL. */
int qlora_codebook_levels(int codebook, float out[16]);

/* Storage of a quantized [rows][cols] weight (host outputs, any may be NULL):
 * codes rows*cols/2 bytes; with dq_block 256, qscale rows*cols/64 bytes and
 * dscale 4*ceil(nb/256) bytes; with dq_block 0, qscale 0 and dscale 4*nb
 * bytes.  Returns QL_OK or QL_ERR_SHAPE / QL_ERR_UNSUPPORTED. */
int nf4_storage_bytes(int64_t rows, int64_t cols, int block, int dq_block,
                      size_t* codes_bytes, size_t* qscale_bytes, size_t* dscale_bytes);

/* Quantize an fp32 weight W [rows][cols] (device) to NF4 with double-quantized
 * scales.  Ultralytics "QLoRA", "How QLoRA works" (NF4 and double
 * quantization bullets, the encoding snippet):
 *   a_b   = max |x| over block b (64 consecutive elements of a row)
 *   code  = argmin_i fl32(|fl32(x / a_b) - L[i]|), lower code on a tie;
 *           an all-zero block gets code 7 (the exact zero level)
 *   d_g   = fl32(max_{b in g} a_b / 448)                       -> dscale[g]
 *   q_b   = E4M3_RNE(fl32(a_b / d_g)), 0 when d_g == 0           -> qscale[b]
 * Outputs: codes [rows*cols/2], qscale [nb], dscale [ng] (device);
 * absmax_out [nb] fp32 (device, may be NULL) receives the exact a_b.
 * dq_block 0 skips the double quantization: dscale [nb] receives a_b and
 * qscale may be NULL (as qlora_quantize with QL_CODEBOOK_NF4). */
int nf4_quantize(const float* W, int64_t rows, int64_t cols, int block, int dq_block,
                 uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax_out,
                 void* stream);

/* Quantize with a codebook (QL_CODEBOOK_NF4 or QL_CODEBOOK_INT4) and a scale
 * format: dq_block 256 with dq_format QL_DQ_E4M3 (as nf4_quantize) or
 * QL_DQ_UINT8 (d_g = fl32(max_{b in g} a_b / 255), q_b = min(255,
 * round-half-even(fl32(a_b / d_g))), 0 when d_g == 0); dq_block 0: fp32 block
 * scales in dscale [nb], qscale unused (dq_format ignored).  Same encode rule
 * as nf4_quantize with the codebook's levels; an all-zero block gets the code
 * of v = 0 (the nearest level, the lower on a tie: 7 for both codebooks).
 * QL_ERR_UNSUPPORTED for an unknown codebook, dq_block or dq_format. */
int qlora_quantize(const float* W, int64_t rows, int64_t cols, int codebook, int dq_block,
                   int dq_format, uint8_t* codes, uint8_t* qscale, float* dscale,
                   float* absmax_out, void* stream);

/* Dequantize to bfloat16: W_bf16[e] = bf16_RNE(fl32(L[code_e] * s_b)) with the
 * restored block scale s_b = fl32(v(q_b) * d_g), v the E4M3 value or (for
 * QL_DQ_UINT8) the integer of the scale byte (or the fp32 dscale[b] when
 * dq_block is 0) and L the weight's codebook.  Transformers docs
 * "Bitsandbytes", section on dequantizing a model to its original precision;
 * Ultralytics "QLoRA" (restore = level times block scale).
 * W_bf16: device, rows*cols uint16 (bf16 bits). */
int nf4_dequantize(const qlora_nf4_weight* w, uint16_t* W_bf16, void* stream);

/* Workspace the forward needs (bytes, 256-byte granular; may be 0). */
size_t qlora_fwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);

/* Forward of the QLoRA linear layer (Ultralytics "QLoRA", "How QLoRA works":
 * dequantize to bf16 right before the matmul, then add the LoRA path).
 *   T_save[m][j] = sum_k X[m][k] A[j][k]                     fp32 [M][r]
 *   Y[m][n]      = bf16(sum_k X[m][k] W'[n][k] + s sum_j T[m][j] B[n][j])  [M][N]
 * with s = fl32(alpha / r); products of bf16 operands summed in fp32 (MFMA),
 * W' the bf16 weight nf4_dequantize writes, and T entering the LoRA product
 * as bf16(s T).  For M <= 16 with K a multiple of 256 and at most 65536 and
 * double-quantized scales (the HBM-bound decode path) the weight is streamed
 * once and dequantized in registers; the path sums T over up to 16 slices
 * of K into the workspace in one small launch, then streams the weight in a
 * second, whose workgroups add the slices in slice order, so T_save and Y do
 * not depend on timing.  Other shapes take the tiled path of M > 16.
 * X [M][K], A [r][K],
 * B [N][r] bf16 (device).  1 <= r <= QLORA_MAX_RANK.  compute_dtype must be
 * QL_DTYPE_BF16.  T_save (fp32, required) is the saved activation the
 * backward reuses; it is kept in fp32 because dB sums M products of it and
 * a bf16 T would cost dB about 2^-9 * sqrt(M) of absolute accuracy.
 * workspace: device, at least qlora_fwd_workspace_bytes(M, N, K, r) bytes
 * (may be NULL when that is 0); its contents on return are unspecified. */
int qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* X, int64_t M,
                     const uint16_t* A, const uint16_t* B, int r, float alpha,
                     int compute_dtype, uint16_t* Y, float* T_save,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Epilogues of qlora_dual_fwd. */
enum { QL_DUAL_SEPARATE = 1, QL_DUAL_SWIGLU = 2 };

/* Gate and up projections of one input in one kernel.  The Transformers
 * "Bitsandbytes" page and the Ultralytics "QLoRA" page fine-tune Llama-2
 * models, whose MLP feeds the same X to a gate and an up projection and
 * multiplies silu(gate) by up; with LoRA on every linear both projections
 * are QLoRA layers.  Each output is the forward of qlora_linear_fwd on its
 * own weight and adapter (same T, same bf16 LoRA operand, same fp32 sums):
 *   G[m][n] = sum_k X W_gate'^T + s T_gate B_gate^T,   U likewise with _up,
 * with the X tile read once for both weights.  epilogue QL_DUAL_SEPARATE
 * writes Y_gate = bf16(G), Y_up = bf16(U) (H unused, may be NULL);
 * QL_DUAL_SWIGLU writes H = bf16(silu(G) * U), silu(x) = x / (1 + e^-x)
 * in fp32 from the fp32 sums (Y_gate, Y_up unused, may be NULL).
 * T_gate_save, T_up_save: fp32 [M][r] (required; the inputs of each
 * projection's qlora_linear_bwd).  w_gate and w_up must have the same shape
 * [N][K]; other arguments as in qlora_linear_fwd (there is no decode-size
 * special case: every M runs the tiled kernel).  workspace: device, at least
 * qlora_fwd_workspace_bytes(M, N, K, r) bytes. */
int qlora_dual_fwd(const qlora_nf4_weight* w_gate, const qlora_nf4_weight* w_up,
                   const uint16_t* X, int64_t M, const uint16_t* A_gate, const uint16_t* B_gate,
                   const uint16_t* A_up, const uint16_t* B_up, int r, float alpha,
                   int compute_dtype, int epilogue, uint16_t* Y_gate, uint16_t* Y_up,
                   uint16_t* H, float* T_gate_save, float* T_up_save,
                   void* workspace, size_t workspace_bytes, void* stream);

/* One tensor of an optimizer step: the bf16 parameter and its gradient, the
 * fp32 first and second moments (same element count), and an optional fp32
 * master copy of the parameter (NULL: the bf16 parameter is the value). */
typedef struct {
  uint16_t* param;
  const uint16_t* grad;
  float* exp_avg;
  float* exp_avg_sq;
  float* master;
  int64_t numel;
} qlora_adamw_tensor;

/* One AdamW step of the adapters over `count` tensors, in as few launches as
 * the tensor list allows (24 tensors each).  Ultralytics "QLoRA", "How QLoRA
 * works" (paged-optimizer bullet) and vnread "Grokking QLoRA", "Paged
 * Optimizers": only the adapters train, and Adam keeps a momentum and a
 * variance per parameter.  The update (Adam with bias correction and
 * decoupled weight decay), in fp32 per element:
 *   theta <- theta (1 - lr weight_decay)
 *   m <- beta1 m + (1 - beta1) g,   v <- beta2 v + (1 - beta2) g^2
 *   theta <- theta - (lr / (1 - beta1^step)) m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 * theta comes from master when given (which receives the new value) and from
 * the bf16 param otherwise; param always receives bf16_RNE(theta).  The
 * moments and master are read and written in place; grad is only read.
 * The pointers may be any device-accessible memory, managed (unified)
 * memory included, which the runtime may page to the host under pressure;
 * the kernel makes no assumption about where the pages live.  step >= 1; 0 <= beta < 1; eps >= 0.  A tensor with
 * numel 0 is skipped. */
int qlora_adamw_step(const qlora_adamw_tensor* tensors, int count, float lr, float beta1,
                     float beta2, float eps, float weight_decay, int step, void* stream);

/* Workspace the backward needs (bytes, 256-byte granular). */
size_t qlora_bwd_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);

/* Backward of the QLoRA linear layer (Ultralytics "QLoRA", "How QLoRA works":
 * gradients pass through the dequantized weights; only A and B receive
 * gradients -- W stays frozen and gets none).  With U = dY B (fp32, kept in
 * the workspace):
 *   dX[m][k] = bf16(sum_n dY[m][n] W'[n][k] + s sum_j U[m][j] A[j][k])  [M][K]
 *   dA[j][k] = bf16(s sum_m U[m][j] X[m][k])                           [r][K]
 *   dB[n][j] = bf16(s sum_m dY[m][n] T[m][j])                          [N][r]
 * U enters the dX product as its bf16 rounding; in dA and dB the fp32 U and
 * T enter as a pair of bf16 terms (hi + lo), so those sums see them to about
 * 2^-17 relative precision.
 * T_saved: the forward's fp32 T_save, or NULL to recompute it in the workspace.
 * dX may be NULL (skipped, e.g. for a first layer); dA and dB are required.
 * Outputs are overwritten, never accumulated into.  W's buffers are only
 * read.  workspace: device, >= qlora_bwd_workspace_bytes(M, N, K, r). */
int qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                     int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                     int compute_dtype, const float* T_saved,
                     uint16_t* dX, uint16_t* dA, uint16_t* dB,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and checks as qlora_linear_bwd, whose
 * kernels it runs, minus the workspace: the scratch (U, the recomputed T,
 * the split partials) lives in a fixed array of QLORA_BWD_NOALLOC_MAX_BYTES
 * in the library's device data, one copy per GPU, held until the process
 * ends.  A call whose qlora_bwd_workspace_bytes(M, N, K, r) exceeds that
 * returns QL_ERR_WORKSPACE and enqueues nothing (32 MiB covers, e.g., M = 8192
 * tokens of a 28672 x 8192 layer at r = 64).  The call allocates nothing; the
 * first call on each device (with that device current) looks up the array's
 * address there, so a caller that captures graphs makes one call before
 * capturing.  `stream` must belong to the current device.  Every call on a
 * GPU shares that GPU's array: calls that can overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.  The
 * array's contents are not meaningful between calls. */
#define QLORA_BWD_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int qlora_linear_bwd_noalloc(const qlora_nf4_weight* w, const uint16_t* X, const uint16_t* dY,
                             int64_t M, const uint16_t* A, const uint16_t* B, int r, float alpha,
                             int compute_dtype, const float* T_saved,
                             uint16_t* dX, uint16_t* dA, uint16_t* dB, void* stream);

/* Merge the adapter into the weight (IBM "What is LoRA?": after training the
 * low-rank update B A is merged into the pretrained weight, which then runs
 * with no extra inference latency; Ultralytics "QLoRA", "Trade-offs": the
 * merge needs the base dequantized to 16 bit first):
 *   W_out[n][k] = bf16_RNE( fl32(W'[n][k]) + s * sum_j B[n][j] A[j][k] ),
 * s = fl32(alpha / r), W' the bf16 dequantized weight (nf4_dequantize), the
 * rank-r sum in fp32 from bf16 products, base and product combined with one
 * fused multiply-add.  A [r][K], B [N][r] bf16 (device); W_out bf16 [N][K]
 * (device, must not overlap W's buffers).  1 <= r <= QLORA_MAX_RANK;
 * rows*cols*2, r*cols*2 and rows*r*2 below 2^31 (QL_ERR_SHAPE otherwise). */
int qlora_merge(const qlora_nf4_weight* w, const uint16_t* A, const uint16_t* B, int r, float alpha,
                uint16_t* W_out, void* stream);

/* Take the adapter back out of a merged weight (swapping adapters on a
 * merged model, IBM "What is LoRA?"):
 *   W_out[n][k] = bf16_RNE( fl32(W_merged[n][k]) - s * sum_j B[n][j] A[j][k] ).
 * After qlora_merge each element comes back to W' within one bf16 unit in the
 * last place (two roundings).  W_merged, W_out bf16 [rows][cols] (device);
 * W_out may equal W_merged (in place).  cols % 8 == 0. */
int qlora_unmerge(const uint16_t* W_merged, int64_t rows, int64_t cols, const uint16_t* A,
                  const uint16_t* B, int r, float alpha, uint16_t* W_out, void* stream);

/* Benchmark timing hook.  When set, later calls ON THIS THREAD record
 * fwd_begin / fwd_end (hipEvent_t handles the caller created) on the call's
 * stream immediately before and after the launch of the forward's main GEMM
 * kernel, and dx_begin / dx_end around the backward's dX GEMM kernel, so the
 * caller can read those kernels' durations with hipEventElapsedTime.  NULL
 * entries record nothing; qlora_set_timing_events(NULL, NULL, NULL, NULL)
 * clears the hook.  Returns QL_OK. */
int qlora_set_timing_events(void* fwd_begin, void* fwd_end, void* dx_begin, void* dx_end);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
