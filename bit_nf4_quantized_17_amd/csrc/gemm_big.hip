// gemm_big.hip -- the two large fused GEMMs of the QLoRA linear layer:
//
//   forward  Y  = X W'^T + s T B^T      (contraction over k, W' rows are output columns)
//   backward dX = dY W' + s U A          (contraction over n, W' columns are output columns)
//
// W' is the bf16 dequantized NF4 weight, produced tile by tile inside the
// kernel: a thread turns one 64-code block into bf16 exactly as
// nf4_dequantize does (w' = bf16(fl32(L[code] * scale))), through a per-block
// 16-entry bf16 table held in registers and looked up with byte permutes, and
// writes it to LDS with 16-byte stores.  Ultralytics glossary "QLoRA", "How
// QLoRA works": dequantize NF4 to bfloat16 right before the matrix product,
// gradients flow through the dequantized weights.
//
// Tiling (gfx950): 512 threads = 8 waves (two per SIMD, so one wave's MFMAs
// overlap the other's dequantization), output tile 256 x 256, contraction
// step 64.  Each wave owns a 128 x 64 eighth as 4 x 2 accumulators of
// v_mfma_f32_32x32x16_bf16 (128 accumulator registers).  LDS holds two stages
// of both operand tiles (about 144 KiB); global loads run two stages ahead in
// registers, so one barrier per step separates writing stage k+1 from
// reading stage k.  A thread produces a quarter of an A-tile column chunk and
// half of one 64-code weight block per step.  The forward's weight tile is [n][k] (contraction
// contiguous: plain 16-byte fragment reads); the backward's is [n][k] with
// n the contraction, read with ds_read_b64_tr_b16 (within each 16-lane group
// lane i receives element i%4 of the rows addressed by lanes 4j + i/4, which
// yields the column fragment the MFMA needs).
//
// The LoRA term is a prologue: the accumulators start as (s T) B^T or
// (s U) A, with s T / s U rounded to bf16 on the way to LDS (rank r <= 128 in
// steps of 64), then the base product accumulates on top.
//
// Dual projection (forward only): two weights of one shape that read the
// same X, such as the gate and up projections of a Llama-style MLP (the
// models the Transformers "Bitsandbytes" and Ultralytics pages fine-tune), in
// one kernel.  A tile's 256 weight rows are 128 output columns of each
// weight, interleaved in 32-row slices (gate n0..n0+31, up n0..n0+31, gate
// n0+32.., ...), so each wave's two 32-column accumulator blocks hold the
// gate and up sums of the same outputs, and the X tile is read once for both.
// The two LoRA terms share one prologue of contraction 2r: the A side is
// [T_gate | T_up] and a gate row of the B side is [B_gate[n] | 0], an up row
// [0 | B_up[n]].  The epilogue writes both outputs, or silu(g) * u.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "device.h"

namespace qln {
namespace big {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int APITCH = BK + 8;          // A tile [256][72] bf16 (144-byte rows)
constexpr int FPITCH = BK + 8;          // forward W tile [256 n][72]
constexpr int TPITCH = BN + 32;         // backward W tile [64 n][288] (576-byte rows)
constexpr int A_ELEMS = BM * APITCH;    // 18432
constexpr int BF_ELEMS = BN * FPITCH;   // 18432
constexpr int BT_ELEMS = BK * TPITCH;   // 17408
constexpr int NTHREADS = 512;

enum { MODE_FWD = 0, MODE_DX = 1 };

template <int MODE>
constexpr int b_elems() { return MODE == MODE_FWD ? BF_ELEMS : BT_ELEMS; }
// epilogue staging: each wave's 128 x 64 bf16 block, rows padded to 72
constexpr int EPITCH = 72;
constexpr int E_ELEMS = 128 * EPITCH;
template <int MODE>
constexpr size_t lds_bytes() {
  const size_t main = (size_t)2 * (A_ELEMS + b_elems<MODE>()) * 2;
  const size_t epi = (size_t)(NTHREADS / 64) * E_ELEMS * 2;
  return main > epi ? main : epi;
}

struct BigArgs {
  const u16* a; int64_t lda; bool a_vec;   // X [M][K] or dY [M][N]
  NF4View w;
  int64_t M, J, C;                         // output M x J, contraction C
  const float* la;                         // T or U, fp32 [M][r]
  const u16* lb;                           // B [N][r] (forward) or A [r][K] (backward)
  int r; float s; bool la_vec; bool lb_vec;
  u16* out; int64_t ldo; bool out_vec;   // out_vec: 16-byte aligned rows
  // dual projection only: the second weight, its T and B, its output
  NF4View w2; const float* la2; const u16* lb2; u16* out2;
};

enum { DUAL_NONE = 0, DUAL_SEPARATE = 1, DUAL_SWIGLU = 2 };

// dual projection: tile row t (0..255) holds output column n0 + dual_col(t)
// of the gate weight (dual_src(t) == 0) or of the up weight (1)
__device__ __forceinline__ int dual_col(int t) { return 32 * (t >> 6) + (t & 31); }
__device__ __forceinline__ int dual_src(int t) { return (t >> 5) & 1; }

typedef __attribute__((address_space(3))) short lds_short;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// ---------------------------------------------------------------------------
// dequantization of one 64-code block (32 bytes) into 32 bf16 pairs
// ---------------------------------------------------------------------------
// The two lanes that share a block (lanes 2i and 2i + 1 of a wave) build its
// table together: lane parity p scales the 8 levels 8p .. 8p + 7 and takes
// the other 8 from its partner with a DPP move.  Entries 0..7 of a lane's
// table are its own levels, so lane 1 of a pair looks codes up with bit 3
// flipped (the flip argument of dequant8), which lands every code on its own
// level.
struct Table {
  uint32_t lo[4], hi[4];   // low / high bytes of the 16 bf16 values, 4 per word
};

__device__ __forceinline__ uint32_t dpp_pair_swap(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_QUAD_XOR1, 0xF, 0xF, false);
}

// mv: this lane's 8 levels; sc: the block's scale
__device__ __forceinline__ Table make_table(const float (&mv)[8], float sc) {
  uint32_t P[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) P[j] = pack_bf16x2(mv[2 * j] * sc, mv[2 * j + 1] * sc);
  Table t;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    t.lo[q] = __builtin_amdgcn_perm(P[2 * q + 1], P[2 * q], 0x06040200u);
    t.hi[q] = __builtin_amdgcn_perm(P[2 * q + 1], P[2 * q], 0x07050301u);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    t.lo[2 + q] = dpp_pair_swap(t.lo[q]);
    t.hi[2 + q] = dpp_pair_swap(t.hi[q]);
  }
  return t;
}

// four 4-bit indices (one per byte) -> their bf16 low bytes and high bytes.
// Byte selectors past 12 read as 0xFF, so each half of the table is looked
// up with the other half's indices pushed past 16 and the two are AND-ed.
__device__ __forceinline__ void lookup4(const Table& t, uint32_t idx, uint32_t& lo, uint32_t& hi) {
  // idx | ((idx << 1) & 0x10101010) as one three-input bit operation
  const uint32_t selA = __builtin_amdgcn_bitop3_b32(idx, idx << 1, 0x10101010u, 0xF8);  // 8..15 -> 24..31 (0xFF)
  const uint32_t selB = selA ^ 0x18181818u;                // indices 0..7 -> 24..31, 8..15 -> 0..7
  lo = __builtin_amdgcn_perm(t.lo[1], t.lo[0], selA) & __builtin_amdgcn_perm(t.lo[3], t.lo[2], selB);
  hi = __builtin_amdgcn_perm(t.hi[1], t.hi[0], selA) & __builtin_amdgcn_perm(t.hi[3], t.hi[2], selB);
}

// 8 codes (one word, element e in bits 4e..4e+3) -> 4 words of bf16 pairs in
// element order.  The codes are first regrouped one per byte in element order
// (bytes of c and c >> 4 interleaved, then masked), so that each lookup's
// bytes pair up directly into two output words.
__device__ __forceinline__ void dequant8(const Table& t, uint32_t c, uint32_t flip, uint32_t o[4]) {
  const uint32_t c4 = c >> 4;
  const uint32_t i03 = (__builtin_amdgcn_perm(c4, c, 0x05010400u) ^ flip) & 0x0F0F0F0Fu;   // codes 0..3
  const uint32_t i47 = (__builtin_amdgcn_perm(c4, c, 0x07030602u) ^ flip) & 0x0F0F0F0Fu;   // codes 4..7
  uint32_t l, h;
  lookup4(t, i03, l, h);
  o[0] = __builtin_amdgcn_perm(h, l, 0x05010400u);
  o[1] = __builtin_amdgcn_perm(h, l, 0x07030602u);
  lookup4(t, i47, l, h);
  o[2] = __builtin_amdgcn_perm(h, l, 0x05010400u);
  o[3] = __builtin_amdgcn_perm(h, l, 0x07030602u);
}

// ---------------------------------------------------------------------------
// Main-loop operand loads go through buffer resources: a load whose byte
// offset is past the buffer's end returns zeros, so rows beyond M, rows of W
// beyond N and the stages past the last one need no branches.  (A row read
// past the contraction length C of the backward's dY runs into the next row;
// those values meet W rows beyond N, which read as zero codes with a zero
// scale, so they add nothing.)
// ---------------------------------------------------------------------------
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct Bufs {
  __amdgpu_buffer_rsrc_t a, codes, qscale, dscale;
  uint32_t qor, dshift;   // scale format: E4M3 code OR-ed in (QOR_U8: integer scales), group shift of dscale
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct StageA { uint4 v[4]; };                    // A tile: 4 x 16 bytes per thread
struct StageW { uint4 c; uint32_t q; float d; };  // half a block's codes, raw scale byte, group constant

// A tile rows m0 + tid/8 + 64q, contraction c0 + 8*(tid%8) .. +8
__device__ __forceinline__ void load_a(StageA& st, const Bufs& b, uint32_t row_off0,
                                       uint32_t row_step, uint32_t c0) {
#pragma unroll
  for (int q = 0; q < 4; ++q) st.v[q] = bload16(b.a, row_off0 + q * row_step + 2 * c0);
}

// the thread's half block: row n, columns k + 32*half .. +32.  The scale is
// decoded only when the block is dequantized (one step later), so nothing
// waits for these loads now; a stage past the last one (live == false) gets
// group constant 0, so it multiplies as a zero tile.
__device__ __forceinline__ void load_w(StageW& st, const Bufs& b, uint32_t n, uint32_t k, uint32_t half,
                                       uint32_t K, bool live) {
  st.c = bload16(b.codes, n * (K / 2) + k / 2 + 16 * half);
  const uint32_t blk = n * (K / 64) + k / 64;
  st.q = __builtin_amdgcn_raw_buffer_load_b8(b.qscale, blk, 0, 0);
  // a dead stage reads past the end of the group constants, which returns 0
  st.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       b.dscale, live ? 4 * (blk >> b.dshift) : 0xFFFFFFF0u, 0, 0));
}

// fl32(E4M3(q) * d); with fp32 scales q reads 0 from an empty buffer and the
// OR makes it E4M3(1.0), so the product is the stored scale exactly; with
// uint8-linear scales (qor == QOR_U8) fl32(q * d)
constexpr uint32_t QOR_U8 = 0x100u;
__device__ __forceinline__ float stage_scale(const StageW& st, uint32_t qor) {
  const float v = qor == QOR_U8 ? (float)(st.q & 0xFFu)
                                : __builtin_amdgcn_cvt_f32_fp8((int)(st.q | qor), 0);
  return v * st.d;
}

__device__ __forceinline__ void store_a(const StageA& st, u16* sA, int tid) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint4*>(sA + (tid / 8 + 64 * q) * APITCH + (tid % 8) * 8) = st.v[q];
}

// LoRA prologue A-side tile: s times fp32 T or U, rounded to bf16 (guarded loads)
__device__ __forceinline__ void lora_a_tile(const float* src, int64_t ld, int64_t rows,
                                            int64_t C, int64_t m0, int64_t c0, bool vec,
                                            float s, u16* sA, int tid) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t row = m0 + tid / 8 + 64 * q;
    const int64_t c = c0 + (tid % 8) * 8;
    float x[8];
    if (row < rows && c + 8 <= C && vec) {
      const float4 u = *reinterpret_cast<const float4*>(src + row * ld + c);
      const float4 v = *reinterpret_cast<const float4*>(src + row * ld + c + 4);
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (row < rows && c + e < C) ? src[row * ld + c + e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= s;
    *reinterpret_cast<uint4*>(sA + (tid / 8 + 64 * q) * APITCH + (tid % 8) * 8) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
  }
}

// Dual prologue, A side: columns c < r of the contraction come from T_gate,
// columns r .. 2r - 1 from T_up (both fp32 [M][r]), times s, rounded to bf16.
__device__ __forceinline__ void lora_a_tile_dual(const float* la, const float* la2, int r,
                                                 int64_t rows, int64_t m0, int64_t c0, bool vec,
                                                 float s, u16* sA, int tid) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t row = m0 + tid / 8 + 64 * q;
    const int64_t c = c0 + (tid % 8) * 8;
    float x[8];
    if (vec && row < rows && c + 8 <= 2 * r) {  // r % 8 == 0: a chunk lies in one source
      const float* src = c < r ? la + row * r + c : la2 + row * r + (c - r);
      const float4 u = *reinterpret_cast<const float4*>(src);
      const float4 v = *reinterpret_cast<const float4*>(src + 4);
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t ce = c + e;
        x[e] = row >= rows || ce >= 2 * r ? 0.0f : ce < r ? la[row * r + ce] : la2[row * r + ce - r];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= s;
    *reinterpret_cast<uint4*>(sA + (tid / 8 + 64 * q) * APITCH + (tid % 8) * 8) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
  }
}

// where the thread's 32 dequantized values go: forward tile [256 n][FPITCH],
// block row tid/2; backward tile [64 n][TPITCH], block (tid/2) = 4 per row
template <int MODE>
__device__ __forceinline__ u16* w_dst(u16* sB, int tid) {
  const int blk = tid >> 1, half = tid & 1;
  if constexpr (MODE == MODE_FWD) return sB + blk * FPITCH + 32 * half;
  else return sB + (blk >> 2) * TPITCH + 64 * (blk & 3) + 32 * half;
}

// Backward tile swizzle: in row n, 16-byte chunk c (8 bf16) is stored at chunk
// c ^ x with x = 2 * bit 4 of c ^ (n & 1), a permutation inside each aligned
// group of four chunks.  A thread stores four consecutive chunks of a row and
// eight threads fill a row, so without it the chunks 16 apart (256 bytes)
// and those of the next row fell on the same LDS banks; with it the 16 lanes
// of one store cycle use 16 distinct 4-bank groups, and the transposing reads
// (4 rows x 4 aligned chunks a half-wave) still cover 64 distinct banks.
__device__ __forceinline__ uint32_t t_swz(uint32_t chunk, uint32_t row) {
  return ((chunk >> 3) & 2u) ^ (row & 1u);
}
// the XOR of the thread's own chunks (all four share it)
template <int MODE>
__device__ __forceinline__ uint32_t w_swz(int tid) {
  if constexpr (MODE == MODE_FWD) return 0u;
  else return t_swz(4u * (uint32_t)(tid & 7), (uint32_t)(tid >> 3));
}

// dequantize the thread's half block and store its 32 bf16 values at dst
__device__ __forceinline__ void store_w(const StageW& st, const float (&mv)[8], uint32_t flip,
                                        uint32_t qor, u16* dst, uint32_t swz) {
  const Table t = make_table(mv, stage_scale(st, qor));
  const uint32_t c[4] = {st.c.x, st.c.y, st.c.z, st.c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t o[4];
    dequant8(t, c[i], flip, o);
    *reinterpret_cast<uint4*>(dst + 8 * ((uint32_t)i ^ swz)) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// LoRA prologue operand of the B side, bf16, in the weight tile's layout:
// forward B [J][r] row j0 + tid/2, columns c0 + 32*(tid%2) .. +32; backward
// A [r][J] row c0 + (tid/2)/4, columns j0 + 64*((tid/2)%4) + 32*(tid%2) .. +32.
template <int MODE>
__device__ __forceinline__ void lora_b_tile(const BigArgs& p, u16* sB, int64_t j0, int64_t c0,
                                            int tid) {
  u16* dst = w_dst<MODE>(sB, tid);
  const int blk = tid >> 1, half = tid & 1;
  int64_t row, col0, rows, cols, ld;
  if constexpr (MODE == MODE_FWD) {
    row = j0 + blk; col0 = c0 + 32 * half; rows = p.J; cols = p.r; ld = p.r;
  } else {
    row = c0 + (blk >> 2); col0 = j0 + 64 * (blk & 3) + 32 * half; rows = p.r; cols = p.J; ld = p.J;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = col0 + 8 * q;
    uint32_t v[4] = {0, 0, 0, 0};
    if (row < rows && c + 8 <= cols && p.lb_vec) {
      const uint4 u = *reinterpret_cast<const uint4*>(p.lb + row * ld + c);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else if (row < rows) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c + e < cols) v[e >> 1] |= (uint32_t)p.lb[row * ld + c + e] << (16 * (e & 1));
    }
    *reinterpret_cast<uint4*>(dst + 8 * ((uint32_t)q ^ w_swz<MODE>(tid))) = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// Dual prologue, B side, in the forward weight tile's layout: tile row t is
// [B_gate[n] | 0] for a gate row and [0 | B_up[n]] for an up row, n = n0 +
// dual_col(t); the thread fills row tid/2, columns c0 + 32*(tid%2) .. +32.
__device__ __forceinline__ void lora_b_tile_dual(const BigArgs& p, u16* sB, int64_t n0, int64_t c0,
                                                 int tid) {
  u16* dst = sB + (tid >> 1) * FPITCH + 32 * (tid & 1);
  const int t = tid >> 1, src = dual_src(t);
  const int64_t n = n0 + dual_col(t);
  const u16* lb = src ? p.lb2 : p.lb;
  const int64_t lo = src ? p.r : 0;  // this row's nonzero contraction range: lo .. lo + r - 1
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t c = c0 + 32 * (tid & 1) + 8 * q;
    uint32_t v[4] = {0, 0, 0, 0};
    if (n < p.J) {
      if (p.lb_vec && c >= lo && c + 8 <= lo + p.r) {
        const uint4 u = *reinterpret_cast<const uint4*>(lb + n * p.r + (c - lo));
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e >= lo && c + e < lo + p.r)
            v[e >> 1] |= (uint32_t)lb[n * p.r + (c + e - lo)] << (16 * (e & 1));
      }
    }
    *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// ---------------------------------------------------------------------------
// MFMA on one LDS stage: wave (wm, wn) owns rows wm*128 .. +128 and columns
// wn*64 .. +64 of the tile
// ---------------------------------------------------------------------------
template <int MODE>
__device__ __forceinline__ bf16x8_t read_b(const u16* sB, int wn, int b, int ks, int lane) {
  if constexpr (MODE == MODE_FWD) {
    return *reinterpret_cast<const bf16x8_t*>(
        sB + (wn * 64 + b * 32 + (lane & 31)) * FPITCH + ks * 16 + (lane >> 5) * 8);
  } else {
    const int L = lane & 15;
    const int col = wn * 64 + b * 32 + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
    const int row = ks * 16 + 8 * (lane >> 5) + (L >> 2);
    // rows row and row + 4 have the same parity, so the same swizzle
    const int scol = col ^ (8 * (int)t_swz((uint32_t)col >> 3, (uint32_t)row));
    const lds_short* base = (const lds_short*)(sB);
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + row * TPITCH + scol));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + (row + 4) * TPITCH + scol));
    typedef short s16x8_t __attribute__((ext_vector_type(8)));
    s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

template <int MODE>
__device__ __forceinline__ void frags(bf16x8_t (&fa)[4], bf16x8_t (&fb)[2], const u16* sA,
                                      const u16* sB, int wm, int wn, int ks, int lane) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
    fa[a] = *reinterpret_cast<const bf16x8_t*>(
        sA + (wm * 128 + a * 32 + (lane & 31)) * APITCH + ks * 16 + (lane >> 5) * 8);
#pragma unroll
  for (int b = 0; b < 2; ++b) fb[b] = read_b<MODE>(sB, wn, b, ks, lane);
}

template <int MODE>
__device__ __forceinline__ void mma_stage(f32x16_t (&acc)[4][2], const u16* sA, const u16* sB,
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    bf16x8_t fa[4], fb[2];
    frags<MODE>(fa, fb, sA, sB, wm, wn, ks, lane);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  }
}

// One contraction step with the producer work for the next stage woven in:
// for each 16-wide substep ks, the fragments of ks+1 are read while the 8
// MFMAs of ks issue, then a quarter of the next stage is written to the other
// LDS buffer (one 16-byte A chunk and 8 dequantized weights).  Loads of the
// stage after next are woven in too: the A chunk is reloaded right after it
// is stored, the weight block's scale bytes right after its table is built
// and its codes once they are dequantized, so the per-CU address unit sees a
// steady trickle instead of one burst per step.
struct NextLoads {
  const Bufs* bf;
  uint32_t a_base, a_step, a_c0;   // A stage to load into ra (contraction start)
  uint32_t wn, wk, whalf, K;       // weight half block to load into w
  bool wlive;
};

template <int MODE>
__device__ __forceinline__ void step_pipelined(f32x16_t (&acc)[4][2], const u16* sA,
                                               const u16* sB, int wm, int wn, int lane,
                                               StageA& ra, StageW& w,
                                               u16* sA_next, u16* wdst_next, int tid,
                                               const NextLoads& nl, const float (&mv)[8],
                                               uint32_t flip, uint32_t wswz) {
  bf16x8_t fa[2][4], fb[2][2];
  frags<MODE>(fa[0], fb[0], sA, sB, wm, wn, 0, lane);
  const Table t = make_table(mv, stage_scale(w, nl.bf->qor));
  const uint32_t c[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
  {
    // the scale byte and group constant of the weight block after next
    const uint32_t blk = nl.wn * (nl.K / 64) + nl.wk / 64;
    w.q = __builtin_amdgcn_raw_buffer_load_b8(nl.bf->qscale, blk, 0, 0);
    w.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        nl.bf->dscale, nl.wlive ? 4 * (blk >> nl.bf->dshift) : 0xFFFFFFF0u,
                                        0, 0));
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int cur = ks & 1;
    if (ks < 3) frags<MODE>(fa[cur ^ 1], fb[cur ^ 1], sA, sB, wm, wn, ks + 1, lane);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][a], fb[cur][b], acc[a][b],
                                                            0, 0, 0);
    {
      uint32_t o[4];
      dequant8(t, c[ks], flip, o);
      *reinterpret_cast<uint4*>(wdst_next + 8 * ((uint32_t)ks ^ wswz)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(sA_next + (tid / 8 + 64 * ks) * APITCH + (tid % 8) * 8) = ra.v[ks];
      ra.v[ks] = bload16(nl.bf->a, nl.a_base + ks * nl.a_step + 2 * nl.a_c0);
    }
    if (ks == 3) w.c = bload16(nl.bf->codes, nl.wn * (nl.K / 2) + nl.wk / 2 + 16 * nl.whalf);
#ifndef QLN_NO_INTERLEAVE
    // keep the dequantization's VALU work between the MFMAs (up to five VALU
    // per MFMA in the forward, six in the backward, as measured best)
    constexpr int ILV_VALU = MODE == MODE_FWD ? 5 : 6;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, ILV_VALU, 0);   // then VALU
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                  // next fragments
      else if (i < 7) __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);             // LDS stores
      else __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                         // global loads
    }
#endif
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int MODE, int DUAL>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_big(BigArgs p) {
  extern __shared__ __attribute__((aligned(16))) u16 smem[];
  u16* sA[2] = {smem, smem + A_ELEMS};
  u16* sB[2] = {smem + 2 * A_ELEMS, smem + 2 * A_ELEMS + b_elems<MODE>()};

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  // output column tile start (a dual tile covers BN / 2 columns of each weight)
  const int64_t j0 = (int64_t)blockIdx.y * (DUAL ? BN / 2 : BN);

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  // ---- LoRA prologue: acc = sum_{c < r} bf16(s la(m, c)) lb(j, c) ----
  for (int64_t c0 = 0; c0 < (DUAL ? 2 * p.r : p.r); c0 += BK) {
    __syncthreads();
    if constexpr (DUAL) {
      lora_a_tile_dual(p.la, p.la2, p.r, p.M, m0, c0, p.la_vec, p.s, sA[0], tid);
      lora_b_tile_dual(p, sB[0], j0, c0, tid);
    } else {
      lora_a_tile(p.la, p.r, p.M, p.r, m0, c0, p.la_vec, p.s, sA[0], tid);
      lora_b_tile<MODE>(p, sB[0], j0, c0, tid);
    }
    __syncthreads();
    mma_stage<MODE>(acc, sA[0], sB[0], wm, wn, lane);
  }
  __syncthreads();

  // ---- main contraction ----
  // While stage kt is multiplied out of LDS buffer kt&1, the other buffer
  // receives stage kt+1 (A tile from registers loaded one step earlier, the
  // weight block dequantized from registers loaded two steps earlier).  Loads
  // of stages past the end read zeros or unused data and are never consumed.
  Bufs bf;
  bf.a = rsrc(p.a, (uint32_t)(p.M * p.lda * 2));
  // a dual tile's wave w produces rows of the gate weight (w even) or the up
  // weight (w odd): the choice is uniform across the wave
  const int wsrc = DUAL ? (__builtin_amdgcn_readfirstlane(wave) & 1) : 0;
  const NF4View& wv = wsrc ? p.w2 : p.w;
  bf.codes = rsrc(wv.codes, (uint32_t)(wv.N * wv.K / 2));
  bf.qscale = rsrc(wv.qscale, wv.fp32_scale ? 0u : (uint32_t)(wv.N * wv.K / 64));
  bf.dscale = rsrc(wv.dscale, (uint32_t)(4 * (wv.fp32_scale ? wv.N * wv.K / 64
                                                             : (wv.N * wv.K / 64 + 255) / 256)));
  bf.qor = wv.fp32_scale ? 0x38u : wv.u8_scale ? QOR_U8 : 0u;   // 0x38: E4M3 code of 1.0
  bf.dshift = wv.fp32_scale ? 0u : 8u;
  // this lane's half of the block table: levels 8p .. 8p + 7 for lane parity p
  const bool odd_lane = tid & 1;
  const uint32_t flip = odd_lane ? 0x08080808u : 0u;
  float mv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) mv[i] = odd_lane ? wv.lv[8 + i] : wv.lv[i];
  const uint32_t K = (uint32_t)p.w.K;
  // rows past M give offsets past the end (the host checks 32-bit room)
  const uint32_t a_base = (uint32_t)((m0 + tid / 8) * p.lda * 2) + 2 * 8 * (tid % 8);
  const uint32_t a_step = (uint32_t)(64 * p.lda * 2);
  const int wblk = tid >> 1;
  const uint32_t whalf = (uint32_t)(tid & 1);
  // weight block coordinates of this thread for contraction step kt
  auto w_n = [&](int64_t kt) -> uint32_t {
    if constexpr (DUAL) return (uint32_t)(j0 + dual_col(wblk));
    else if constexpr (MODE == MODE_FWD) return (uint32_t)(j0 + wblk);
    else return (uint32_t)(kt * BK + (wblk >> 2));
  };
  auto w_k = [&](int64_t kt) -> uint32_t {
    if constexpr (MODE == MODE_FWD) return (uint32_t)(kt * BK);
    else return (uint32_t)(j0 + 64 * (wblk & 3));
  };
  u16* wdst0 = w_dst<MODE>(sB[0], tid);
  u16* wdst1 = w_dst<MODE>(sB[1], tid);

  const int64_t nk = (p.C + BK - 1) / BK;
  StageA ra;
  StageW w0, w1;
  load_a(ra, bf, a_base, a_step, 0);
  load_w(w0, bf, w_n(0), w_k(0), whalf, K, true);
  store_a(ra, sA[0], tid);
  const uint32_t wswz = w_swz<MODE>(tid);
  store_w(w0, mv, flip, bf.qor, wdst0, wswz);
  load_a(ra, bf, a_base, a_step, BK);
  load_w(w1, bf, w_n(1), w_k(1), whalf, K, 1 < nk);
  load_w(w0, bf, w_n(2), w_k(2), whalf, K, 2 < nk);
  __syncthreads();
  // steps are taken in pairs; with an odd count the last pair's second step
  // multiplies a zero weight tile (no early exit: that would make the
  // compiler keep two copies of the accumulators)
  for (int64_t kt = 0; kt < nk; kt += 2) {
    // buffer 0 holds stage kt; ra = A(kt+1), w1 = W(kt+1), w0 = W(kt+2)
    {
      const NextLoads nl{&bf, a_base, a_step, (uint32_t)((kt + 2) * BK), w_n(kt + 3), w_k(kt + 3), whalf, K,
                         kt + 3 < nk};
      step_pipelined<MODE>(acc, sA[0], sB[0], wm, wn, lane, ra, w1, sA[1], wdst1, tid, nl, mv, flip, wswz);
    }
    __syncthreads();
    // buffer 1 holds stage kt+1; ra = A(kt+2), w0 = W(kt+2), w1 = W(kt+3)
    {
      const NextLoads nl{&bf, a_base, a_step, (uint32_t)((kt + 3) * BK), w_n(kt + 4), w_k(kt + 4), whalf, K,
                         kt + 4 < nk};
      step_pipelined<MODE>(acc, sA[1], sB[1], wm, wn, lane, ra, w0, sA[0], wdst0, tid, nl, mv, flip, wswz);
    }
    __syncthreads();
  }

  // ---- epilogue ----
  // Each wave rounds its 128 x 64 block to bf16 into its own LDS region
  // (lanes l and l^1 hold neighbouring columns of the same rows, so one DPP
  // swap per pair of values gives each lane a packed pair), then writes it
  // back out as 16-byte row segments.  The main loop's last barrier has freed
  // LDS; the regions are disjoint, and a wave's LDS operations complete in
  // order, so no barrier is needed.  With the SwiGLU epilogue the block is
  // 128 x 32: h = silu(g) * u of the wave's gate and up accumulators.
  u16* sE = smem + wave * E_ELEMS;
  const bool odd = lane & 1;
  constexpr int NBLK = DUAL == DUAL_SWIGLU ? 1 : 2;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        float x0 = acc[a][b][v], x1 = acc[a][b][v + 1];
        if constexpr (DUAL == DUAL_SWIGLU) {
          x0 = x0 / (1.0f + __expf(-x0)) * acc[a][1][v];
          x1 = x1 / (1.0f + __expf(-x1)) * acc[a][1][v + 1];
        }
        const float got = dpp_f32<DPP_QUAD_XOR1>(odd ? x0 : x1);
        const int row = a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3) + (odd ? 1 : 0);
        const int col = b * 32 + ((lane & 31) & ~1);
        *reinterpret_cast<uint32_t*>(sE + row * EPITCH + col) =
            odd ? pack_bf16x2(got, x1) : pack_bf16x2(x0, got);
      }
  // read back: 8 lanes per 64-column row (4 per 32-column row)
  constexpr int LPR = NBLK * 4;              // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per instruction
#pragma unroll
  for (int q = 0; q < 128 / RPI; ++q) {
    const int row = q * RPI + lane / LPR, col = (lane % LPR) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(sE + row * EPITCH + col);
    const int64_t i = m0 + wm * 128 + row;
    int64_t j;
    u16* out;
    if constexpr (DUAL == DUAL_SEPARATE) {
      j = j0 + wn * 32 + (col & 31);
      out = col < 32 ? p.out : p.out2;
    } else if constexpr (DUAL == DUAL_SWIGLU) {
      j = j0 + wn * 32 + col;
      out = p.out;
    } else {
      j = j0 + wn * 64 + col;
      out = p.out;
    }
    if (i < p.M) {
      u16* dst = out + i * p.ldo + j;
      if (p.out_vec && j + 8 <= p.J) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j + e < p.J) dst[e] = (u16)(w4[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

static bool vec_ok(const void* ptr, int64_t ld) {
  return ((uintptr_t)ptr % 16 == 0) && (ld % 8 == 0);
}

template <int MODE, int DUAL = DUAL_NONE>
static hipError_t launch(const BigArgs& p, hipStream_t st) {
  const hipError_t e = set_dynamic_lds((const void*)k_gemm_big<MODE, DUAL>, (int)lds_bytes<MODE>());
  if (e != hipSuccess) return e;
  const int64_t bn = DUAL ? BN / 2 : BN;
  dim3 grid((unsigned)((p.M + BM - 1) / BM), (unsigned)((p.J + bn - 1) / bn), 1);
  hipLaunchKernelGGL((k_gemm_big<MODE, DUAL>), grid, dim3(NTHREADS), lds_bytes<MODE>(), st, p);
  return hipGetLastError();
}

}  // namespace big

// The buffer-load kernels need 16-byte aligned activation rows and 32-bit
// byte offsets (with room for the tile overrun); other shapes take the
// tile-128 kernels of gemm.hip.
static bool fits_32bit(int64_t M, int64_t lda, const NF4View& w) {
  const int64_t lim = (int64_t)1 << 31;
  return (M + big::BM) * lda * 2 + 8 * big::BK * 2 < lim && (w.N + big::BN) * w.K / 2 < lim &&
         w.N * w.K / 64 < lim && 4 * scale_d_count(w) < lim;
}

hipError_t launch_fwd_main(const NF4View& w, const u16* X, int64_t M, const float* T,
                           const u16* B, int r, float s, u16* Y, hipStream_t st) {
  if (!big::vec_ok(X, w.K) || !fits_32bit(M, w.K, w))
    return launch_fwd_generic(w, X, M, T, B, r, s, Y, st);
  big::BigArgs p{};
  p.a = X; p.lda = w.K; p.a_vec = big::vec_ok(X, w.K);
  p.w = w;
  p.M = M; p.J = w.N; p.C = w.K;
  p.la = T; p.lb = B; p.r = r; p.s = s;
  p.la_vec = big::vec_ok(T, r * 2); p.lb_vec = big::vec_ok(B, r);
  p.out = Y; p.ldo = w.N; p.out_vec = big::vec_ok(Y, w.N);
  return big::launch<big::MODE_FWD>(p, st);
}

// Gate and up projections of one X in one kernel (epilogue: 1 = both outputs,
// 2 = bf16(silu(g) * u) into Yg).  M is cut into slices whose X fits the
// 32-bit buffer offsets.
hipError_t launch_fwd_dual(const NF4View& wg, const NF4View& wu, const u16* X, int64_t M,
                           const float* Tg, const float* Tu, const u16* Bg, const u16* Bu, int r,
                           float s, int epilogue, u16* Yg, u16* Yu, hipStream_t st) {
  const int64_t N = wg.N, K = wg.K;
  const int64_t lim = (int64_t)1 << 31;
  if ((N + big::BN) * K / 2 >= lim || N * K / 64 >= lim || 4 * scale_d_count(wg) >= lim ||
      4 * scale_d_count(wu) >= lim)
    return hipErrorInvalidValue;
  int64_t mstep = (lim - 8 * big::BK * 2) / (K * 2) - big::BM;
  mstep = mstep / big::BM * big::BM;
  if (mstep < big::BM) return hipErrorInvalidValue;
  for (int64_t m = 0; m < M; m += mstep) {
    const int64_t mc = std::min(mstep, M - m);
    big::BigArgs p{};
    p.a = X + m * K; p.lda = K; p.a_vec = true;
    p.w = wg; p.w2 = wu;
    p.M = mc; p.J = N; p.C = K;
    p.la = Tg + m * r; p.la2 = Tu + m * r;
    p.lb = Bg; p.lb2 = Bu; p.r = r; p.s = s;
    p.la_vec = r % 8 == 0 && big::vec_ok(Tg, 8) && big::vec_ok(Tu, 8);
    p.lb_vec = big::vec_ok(Bg, r) && big::vec_ok(Bu, r);
    p.out = Yg + m * N; p.out2 = epilogue == 1 ? Yu + m * N : nullptr; p.ldo = N;
    p.out_vec = big::vec_ok(Yg, N) && (epilogue != 1 || big::vec_ok(Yu, N));
    const hipError_t e = epilogue == 1 ? big::launch<big::MODE_FWD, big::DUAL_SEPARATE>(p, st)
                                       : big::launch<big::MODE_FWD, big::DUAL_SWIGLU>(p, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_dx_main(const NF4View& w, const u16* dY, int64_t M, const float* U,
                          const u16* A, int r, float s, u16* dX, hipStream_t st) {
  if (!big::vec_ok(dY, w.N) || !fits_32bit(M, w.N, w) || (w.N + big::BK) * w.K / 2 >= ((int64_t)1 << 31))
    return launch_dx_generic(w, dY, M, U, A, r, s, dX, st);
  big::BigArgs p{};
  p.a = dY; p.lda = w.N; p.a_vec = big::vec_ok(dY, w.N);
  p.w = w;
  p.M = M; p.J = w.K; p.C = w.N;
  p.la = U; p.lb = A; p.r = r; p.s = s;
  p.la_vec = big::vec_ok(U, r * 2); p.lb_vec = big::vec_ok(A, w.K);
  p.out = dX; p.ldo = w.K; p.out_vec = big::vec_ok(dX, w.K);
  return big::launch<big::MODE_DX>(p, st);
}

}  // namespace qln
