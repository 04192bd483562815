// common.h -- internal declarations shared by the HIP sources of libqlora_nf4.
//
// Layout of a quantized weight W [N][K] (see include/qlora_nf4.h): codes are
// row-major, two per byte (even element in the low nibble); block b covers
// flattened elements [64b, 64b+64); group g covers blocks [256g, 256g+256).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

namespace qln {

typedef uint16_t u16;

constexpr int QLN_MAX_RANK = 128;   // largest LoRA rank the kernels take

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device) pair; safe to call from several host threads.  Kernels
// that take more than the default dynamic LDS call this before each launch.
inline hipError_t set_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

// The 16 NF4 levels as fp32 bit patterns, code order.  Ultralytics glossary
// "QLoRA", "How QLoRA works" (the level-building snippet): normal quantiles at
// probabilities evenly spaced from 0.9677083 towards 0.5 (8 positive, 7
// negative), an exact zero, sorted and divided by the largest; each value is
// the exact formula rounded once to fp32.
constexpr uint32_t kNF4LevelBits[16] = {
    0xbf800000u, 0xbf3239b3u, 0xbf066b30u, 0xbeca32a0u,
    0xbe91a24cu, 0xbe3d353fu, 0xbdba786bu, 0x00000000u,
    0x3da2fb03u, 0x3e24cae1u, 0x3e7c04dcu, 0x3ead0338u,
    0x3ee1a4b7u, 0x3f1007aau, 0x3f3913b1u, 0x3f800000u};

// The comparison codebook of the same snippet: 16 evenly spaced levels on
// [-1, 1], L[i] = -1 + 2 i / 15 rounded once to fp32 (no zero level).
constexpr uint32_t kINT4LevelBits[16] = {
    0xbf800000u, 0xbf5ddddeu, 0xbf3bbbbcu, 0xbf19999au,
    0xbeeeeeefu, 0xbeaaaaabu, 0xbe4ccccdu, 0xbd888889u,
    0x3d888889u, 0x3e4ccccdu, 0x3eaaaaabu, 0x3eeeeeefu,
    0x3f19999au, 0x3f3bbbbcu, 0x3f5ddddeu, 0x3f800000u};

enum Codebook { CODEBOOK_NF4 = 0, CODEBOOK_INT4 = 1 };
inline const uint32_t* codebook_bits(int codebook) {
  return codebook == CODEBOOK_INT4 ? kINT4LevelBits : kNF4LevelBits;
}

// A quantized weight as the kernels see it.  With fp32_scale the block
// scales are the exact fp32 absmax values in dscale[b] (no double
// quantization, qscale unused); otherwise s_b = fl32(v(qscale[b]) *
// dscale[b / 256]) with v the E4M3 value of the byte, or (u8_scale) the
// byte as an integer.  lv holds the codebook's 16 levels.
struct NF4View {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* dscale;
  int64_t N, K;
  bool fp32_scale;
  bool u8_scale;
  float lv[16];
};

// Second-level formats of the block scales (kernels' compile-time modes).
enum ScaleFmt { SCALE_E4M3 = 0, SCALE_FP32 = 1, SCALE_U8 = 2 };
inline int scale_fmt(const NF4View& w) {
  return w.fp32_scale ? SCALE_FP32 : w.u8_scale ? SCALE_U8 : SCALE_E4M3;
}

// The kernels restore a block scale as fl32(E4M3(q) * d) everywhere.  For
// fp32 scales they read q from an empty buffer (0) and OR in the E4M3 code of
// 1.0, and d from dscale[blk >> 0] instead of dscale[blk >> 8]; the product is
// then the stored fp32 scale exactly.
constexpr uint32_t kE4M3One = 0x38u;
inline uint32_t scale_q_or(const NF4View& w) { return w.fp32_scale ? kE4M3One : 0u; }
inline uint32_t scale_d_shift(const NF4View& w) { return w.fp32_scale ? 0u : 8u; }
inline int64_t scale_d_count(const NF4View& w) {
  const int64_t nb = w.N * w.K / 64;
  return w.fp32_scale ? nb : (nb + 255) / 256;
}

// Decision points of the nearest-level rule: cut[j] is the smallest fp32 v
// with fl32(L[j+1] - v) < fl32(v - L[j]), so the code of v in [-1, 1] is the
// number of cut[j] <= v (ties go to the lower code, as argmin does).
struct EncodeCuts {
  float cut[15];
  int zero_code;   // the code of v = 0, given to an all-zero block
};
const EncodeCuts& encode_cuts(int codebook);

// fmt (ScaleFmt): SCALE_FP32 -- dscale receives the nb fp32 block scales
// (qscale unused); SCALE_E4M3 / SCALE_U8 -- 8-bit scales in qscale and one
// group constant per 256 blocks in dscale
hipError_t launch_quantize(const float* W, int64_t N, int64_t K, int codebook, int fmt,
                           uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax,
                           hipStream_t s);
hipError_t launch_dequantize(const NF4View& w, u16* out, hipStream_t s);

// ---- GEMM family (gemm.hip) ----
// Rank-side tile width for r (32, 64 or 128).
int rank_tile(int r);

struct SkinnyPlan {
  int splits;          // contraction splits
  int64_t c_per_split; // contraction length per split (multiple of 64)
};
// Split plan for an I x r output with contraction C.
SkinnyPlan skinny_plan(int64_t I, int64_t C);

// T = X A^T (fp32 partials in ws, summed into fp32 T) ; X [M][K], A [r][K]
hipError_t launch_lora_down(const u16* X, const u16* A, int64_t M, int64_t K, int r,
                            float* ws_partials, float* T, hipStream_t s);
// U = dY B ; dY [M][N], B [N][r] -> U [M][r] fp32
hipError_t launch_lora_u(const u16* dY, const u16* B, int64_t M, int64_t N, int r,
                         float* ws_partials, float* U, hipStream_t s);
// dB = s dY^T T ; -> dB [N][r] (T enters as hi + lo bf16)
hipError_t launch_lora_db(const u16* dY, const float* T, int64_t M, int64_t N, int r, float s,
                          float* ws_partials, u16* dB, hipStream_t st);
// dA = s U^T X ; -> dA [r][K] (U enters as hi + lo bf16)
hipError_t launch_lora_da(const float* U, const u16* X, int64_t M, int64_t K, int r, float s,
                          float* ws_partials, u16* dA, hipStream_t st);
// Y = X W'^T + s T B^T
hipError_t launch_fwd_main(const NF4View& w, const u16* X, int64_t M, const float* T,
                           const u16* B, int r, float s, u16* Y, hipStream_t st);
// one AdamW tensor: bf16 parameter and gradient, fp32 moments, optional fp32 master
struct AdamwTensor {
  u16* param; const u16* grad; float* exp_avg; float* exp_avg_sq; float* master; int64_t n;
};
hipError_t launch_adamw(const AdamwTensor* ts, int count, float lr, float b1, float b2, float eps,
                        float wd, int step, hipStream_t st);

// gate and up projections of one X: Yg = X Wg'^T + s Tg Bg^T, Yu likewise;
// epilogue 1 writes both, 2 writes bf16(silu(g) * u) into Yg (Yu unused)
hipError_t launch_fwd_dual(const NF4View& wg, const NF4View& wu, const u16* X, int64_t M,
                           const float* Tg, const float* Tu, const u16* Bg, const u16* Bu, int r,
                           float s, int epilogue, u16* Yg, u16* Yu, hipStream_t st);
// dX = dY W' + s U A
hipError_t launch_dx_main(const NF4View& w, const u16* dY, int64_t M, const float* U,
                          const u16* A, int r, float s, u16* dX, hipStream_t st);

// Tile-128 variants with guarded loads (any alignment / size).
hipError_t launch_fwd_generic(const NF4View& w, const u16* X, int64_t M, const float* T,
                              const u16* B, int r, float s, u16* Y, hipStream_t st);
hipError_t launch_dx_generic(const NF4View& w, const u16* dY, int64_t M, const float* U,
                             const u16* A, int r, float s, u16* dX, hipStream_t st);

// Forward at M <= 16 (writes Y and T_save): a small launch for the partial
// sums of T = X A^T (into the workspace), then one weight-streaming launch;
// decode_fits says whether a shape can take it, decode_ws_bytes how much
// workspace it needs.
bool decode_fits(int64_t M, const NF4View& w, int r);
size_t decode_ws_bytes(int64_t K, int r);
// Adapter merge / unmerge (merge.hip): out = bf16(base +/- s B A), base the
// dequantized NF4 weight or a bf16 weight; merge_fits says whether the 32-bit
// offsets hold for a shape.
bool merge_fits(int64_t N, int64_t K, int r);
hipError_t launch_merge(const NF4View& w, const u16* A, const u16* B, int r, float s, u16* out,
                        hipStream_t st);
hipError_t launch_unmerge(const u16* w_in, int64_t N, int64_t K, const u16* A, const u16* B, int r,
                          float s, u16* out, hipStream_t st);

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, float* ws, hipStream_t st);

// Workspace (fp32 elements) the skinny partial sums of one call need.
int64_t skinny_partial_elems(int64_t I, int64_t C, int r);

}  // namespace qln
