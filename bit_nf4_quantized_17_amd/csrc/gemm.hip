// gemm.hip -- bf16 MFMA GEMMs of the QLoRA linear layer.
//
// One kernel template computes  C[I][J] = sum_c Aop(i, c) * Bop(j, c)  with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation) on 256-thread workgroups.
// Operand tiles are staged through LDS as [row][64 + 8] bf16 (contraction
// contiguous, so every MFMA fragment is one 16-byte LDS read).  The operand
// producers:
//   CC    bf16 source [row][c] (contraction contiguous): 16-byte copies
//   T     bf16 source [c][row]: 16-byte loads along the row, written to LDS
//         transposed (a wave covers 64 consecutive c, so the 2-byte writes of
//         one instruction are contiguous)
//   NF4CC packed NF4 weight W[n][k] with c = k: each thread dequantizes half a
//         block (32 codes) into bf16 exactly as nf4_dequantize does
//   NF4T  packed NF4 weight W[n][k] with c = n (the backward's dX): 32 codes
//         of one row, written to LDS transposed
// Ultralytics glossary "QLoRA", "How QLoRA works": the forward dequantizes
// NF4 to bf16 right before the matrix product and adds the LoRA path; the
// backward computes gradients through the dequantized weights and only for
// the two LoRA matrices.
//
// The LoRA terms enter as a prologue of the main GEMMs: the accumulators
// start as s * (T B^T) (forward) or s * (U A) (dX), then the base product is
// accumulated on top.  The rank-r side products (T, U, dA, dB) run as split
// contractions writing fp32 partials that a second kernel sums in a fixed
// order (deterministic) and rounds to bf16.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "device.h"

namespace qln {

constexpr int BK = 64;
constexpr int PITCH = BK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int NTHREADS = 256;

enum { SRC_CC = 0, SRC_T = 1, SRC_NF4CC = 2, SRC_NF4T = 3, SRC_TF32S = 4,
       SRC_TR = 5,      // A from a [C][I] matrix, kept [c][i] in LDS, read with transposing loads
       SRC_TF32SR = 6   // B from an fp32 [C][J] matrix as hi + lo bf16, kept [c][j], transposing loads
};
enum { LORA_NONE = 0, LORA_FWD = 1, LORA_DX = 2 };
enum { OUT_BF16 = 0, OUT_F32 = 1 };

struct GemmArgs {
  // A operand (bf16), rows i
  const u16* a; int64_t lda; bool a_vec;
  // B operand: bf16 source, fp32 source (SRC_TF32S) or NF4 weight, rows j
  const void* b; int64_t ldb; bool b_vec;
  NF4View w;
  int64_t I, J, C;
  int64_t c_per_split;
  // LoRA prologue: accumulators start at s * sum_{c < r} la(i, c) * lb(j, c);
  // la is fp32 [I][r] (T or U), rounded to bf16 on its way to LDS
  const float* la; const u16* lb; int r; float s; bool la_vec; bool lb_vec;
  // output
  void* out; int64_t ldo; float out_scale;
};

__device__ __forceinline__ float nf4_level(const float* sL, uint32_t c) { return sL[c]; }

// ---------------------------------------------------------------------------
// producers: global -> registers (load) and registers -> LDS (store)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 load8_guarded(const u16* src, int64_t row, int64_t rows,
                                               int64_t ld, int64_t c, int64_t C, bool vec) {
  if (row < rows && c + 8 <= C && vec)
    return *reinterpret_cast<const uint4*>(src + row * ld + c);
  uint32_t w[4] = {0, 0, 0, 0};
  if (row < rows) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c + e < C) w[e >> 1] |= (uint32_t)src[row * ld + c + e] << (16 * (e & 1));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Tile of R rows x 64 contraction from a [rows][C] matrix (leading dim ld).
template <int R>
struct ProdCC {
  static constexpr int NV = R / 32;
  uint4 v[NV];
  __device__ void load(const u16* src, int64_t ld, int64_t rows, int64_t C, int64_t r0,
                       int64_t c0, bool vec, int tid) {
#pragma unroll
    for (int q = 0; q < NV; ++q)
      v[q] = load8_guarded(src, r0 + tid / 8 + 32 * q, rows, ld, c0 + (tid % 8) * 8, C, vec);
  }
  __device__ void store(u16* S, int tid) const {
#pragma unroll
    for (int q = 0; q < NV; ++q)
      *reinterpret_cast<uint4*>(S + (tid / 8 + 32 * q) * PITCH + (tid % 8) * 8) = v[q];
  }
};

// Tile of R rows x 64 contraction from a [C][cols] matrix (row index along
// the contiguous dimension): LDS row i receives column i0 + i.
template <int R>
struct ProdT {
  static constexpr int NV = R / 32;
  uint4 v[NV];
  __device__ void load(const u16* src, int64_t ld, int64_t C, int64_t cols, int64_t i0,
                       int64_t c0, bool vec, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int q = 0; q < NV; ++q)
      v[q] = load8_guarded(src, c0 + lane, C, ld, i0 + (wv + 4 * q) * 8, cols, vec);
  }
  __device__ void store(u16* S, int tid) const {
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int iseg = (wv + 4 * q) * 8;
      const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        S[(iseg + e) * PITCH + lane] = (u16)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
};

// Tiles of a matrix whose contiguous dimension is the output index (dY or X
// for dB and dA): loaded with whole 256-byte row segments (16 lanes per
// contraction row) and kept in LDS as [64 c][R + 8] rows, so both the global
// loads and the 16-byte LDS stores are contiguous; the MFMA fragments come out
// with the transposing LDS read (ds_read_b64_tr_b16).
template <int R>
constexpr int tr_pitch() { return R + 8; }

typedef __attribute__((address_space(3))) short lds_short_g;
typedef short s16x4_g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_g lds_s16x4_g;

// MFMA operand fragment of column block cb (32 columns) at contraction step ks
// from a [c][cols] bf16 tile: lane l receives 8 contraction values of column
// cb*32 + l%32 (within each 16-lane group, lane i gets element i%4 of the rows
// addressed by lanes 4j + i/4).
__device__ __forceinline__ bf16x8_t read_tr(const u16* S, int pitch, int col0, int ks, int lane) {
  const int L = lane & 15;
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
  const int row = ks * 16 + 8 * (lane >> 5) + (L >> 2);
  const lds_short_g* base = (const lds_short_g*)S;
  const s16x4_g lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_g*)(base + row * pitch + col));
  const s16x4_g hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_g*)(base + (row + 4) * pitch + col));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// bf16 [C][cols] source, R = 128 output columns: thread t loads row
// c0 + t/16 + 16q (q < 4), columns i0 + 8 (t % 16) .. +8
template <int R>
struct ProdTR {
  static_assert(R == 128, "16 lanes x 8 columns per row");
  uint4 v[4];
  __device__ void load(const u16* src, int64_t ld, int64_t C, int64_t cols, int64_t i0,
                       int64_t c0, bool vec, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = load8_guarded(src, c0 + tid / 16 + 16 * q, C, ld, i0 + (tid % 16) * 8, cols, vec);
  }
  __device__ void store(u16* S, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(S + (tid / 16 + 16 * q) * tr_pitch<R>() + (tid % 16) * 8) = v[q];
  }
};

// fp32 [C][cols] source, R (32, 64 or 128) output columns, split into hi =
// bf16(x) and lo = bf16(x - hi): thread t loads row c0 + t/16 + 16q (q < 4),
// R/16 consecutive columns
template <int R>
struct ProdTF32SR {
  static constexpr int E = R / 16;
  float x[4][E];
  __device__ void load(const float* src, int64_t ld, int64_t C, int64_t cols, int64_t j0,
                       int64_t c0, bool vec, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t c = c0 + tid / 16 + 16 * q, j = j0 + (tid % 16) * E;
      if (vec && c < C && j + E <= cols) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          const float2 f = *reinterpret_cast<const float2*>(src + c * ld + j + e);
          x[q][e] = f.x;
          x[q][e + 1] = f.y;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) x[q][e] = (c < C && j + e < cols) ? src[c * ld + j + e] : 0.0f;
      }
    }
  }
  __device__ void store(u16* Shi, u16* Slo, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t hi[E / 2], lo[E / 2];
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        const float h0 = bf16_to_f32(f32_to_bf16(x[q][e])), h1 = bf16_to_f32(f32_to_bf16(x[q][e + 1]));
        hi[e / 2] = pack_bf16x2(h0, h1);
        lo[e / 2] = pack_bf16x2(x[q][e] - h0, x[q][e + 1] - h1);
      }
      const int off = (tid / 16 + 16 * q) * tr_pitch<R>() + (tid % 16) * E;
#pragma unroll
      for (int e = 0; e < E / 2; ++e) {
        *reinterpret_cast<uint32_t*>(Shi + off + 2 * e) = hi[e];
        *reinterpret_cast<uint32_t*>(Slo + off + 2 * e) = lo[e];
      }
    }
  }
};

// fp32 tile of R rows x 64 contraction from a [rows][C] fp32 matrix, rounded
// to bf16 (RNE) on the way to LDS.
template <int R>
struct ProdCCF32 {
  static constexpr int NV = R / 32;
  uint4 v[NV];
  __device__ void load(const float* src, int64_t ld, int64_t rows, int64_t C, int64_t r0,
                       int64_t c0, bool vec, int tid) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int64_t row = r0 + tid / 8 + 32 * q, c = c0 + (tid % 8) * 8;
      float x[8];
      if (row < rows && c + 8 <= C && vec) {
        const float4 a = *reinterpret_cast<const float4*>(src + row * ld + c);
        const float4 b = *reinterpret_cast<const float4*>(src + row * ld + c + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (row < rows && c + e < C) ? src[row * ld + c + e] : 0.0f;
      }
      v[q] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                        pack_bf16x2(x[6], x[7]));
    }
  }
  __device__ void store(u16* S, int tid) const {
#pragma unroll
    for (int q = 0; q < NV; ++q)
      *reinterpret_cast<uint4*>(S + (tid / 8 + 32 * q) * PITCH + (tid % 8) * 8) = v[q];
  }
};

// fp32 tile of R rows x 64 contraction from a [C][cols] fp32 matrix, split
// into hi = bf16(x) and lo = bf16(x - hi): the sum of the two MFMA products
// sees x to about 2^-17 relative precision.
template <int R>
struct ProdTF32S {
  static constexpr int NV = R / 32;
  float x[NV][8];
  __device__ void load(const float* src, int64_t ld, int64_t C, int64_t cols, int64_t i0,
                       int64_t c0, bool vec, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    const int64_t c = c0 + lane;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int64_t i = i0 + (wv + 4 * q) * 8;
      if (c < C && i + 8 <= cols && vec) {
        const float4 a = *reinterpret_cast<const float4*>(src + c * ld + i);
        const float4 b = *reinterpret_cast<const float4*>(src + c * ld + i + 4);
        x[q][0] = a.x; x[q][1] = a.y; x[q][2] = a.z; x[q][3] = a.w;
        x[q][4] = b.x; x[q][5] = b.y; x[q][6] = b.z; x[q][7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[q][e] = (c < C && i + e < cols) ? src[c * ld + i + e] : 0.0f;
      }
    }
  }
  __device__ void store(u16* Shi, u16* Slo, int tid) const {
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int iseg = (wv + 4 * q) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u16 hi = f32_to_bf16(x[q][e]);
        const u16 lo = f32_to_bf16(x[q][e] - bf16_to_f32(hi));
        Shi[(iseg + e) * PITCH + lane] = hi;
        Slo[(iseg + e) * PITCH + lane] = lo;
      }
    }
  }
};

// dequantize 32 packed codes (16 bytes) with block scale sc into 16 bf16 pairs
__device__ __forceinline__ void dequant32(const uint4& c, float sc, const float* sL,
                                          uint32_t o[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    o[i] = pack_bf16x2(nf4_level(sL, byte & 15u) * sc, nf4_level(sL, byte >> 4) * sc);
  }
}

// restored block scale: fl32(E4M3(q) * d), or the stored fp32 scale
__device__ __forceinline__ float block_scale(const NF4View& w, int64_t blk) {
  return w.fp32_scale ? w.dscale[blk]
                      : (w.u8_scale ? (float)w.qscale[blk] : e4m3_decode(w.qscale[blk])) * w.dscale[blk >> 8];
}

// NF4 weight, rows j = n (128 of them), contraction c = k (one 64-block):
// two threads per row, 32 codes each.
struct ProdNF4CC {
  uint4 v;
  float sc;
  __device__ void load(const NF4View& w, int64_t n0, int64_t k0, int tid) {
    const int64_t n = n0 + tid / 2;
    const int half = tid & 1;
    if (n < w.N) {
      v = *reinterpret_cast<const uint4*>(w.codes + n * (w.K / 2) + k0 / 2 + half * 16);
      sc = block_scale(w, n * (w.K / 64) + k0 / 64);
    } else {
      v = make_uint4(0, 0, 0, 0);
      sc = 0.0f;
    }
  }
  __device__ void store(u16* S, const float* sL, int tid) const {
    uint32_t o[16];
    dequant32(v, sc, sL, o);
    u16* dst = S + (tid / 2) * PITCH + (tid & 1) * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2],
                                                          o[4 * q + 3]);
  }
};

// NF4 weight, rows j = k (128 columns of W), contraction c = n (64 rows of W):
// thread (lane, wave) takes 32 codes of row c0 + lane at columns
// j0 + 32*wave .. +32 and writes them to LDS transposed.
struct ProdNF4T {
  uint4 v;
  float sc;
  __device__ void load(const NF4View& w, int64_t j0, int64_t c0, int tid) {
    const int lane = tid & 63, wv = tid >> 6;
    const int64_t n = c0 + lane;
    const int64_t k = j0 + 32 * wv;
    if (n < w.N && k < w.K) {
      v = *reinterpret_cast<const uint4*>(w.codes + n * (w.K / 2) + k / 2);
      sc = block_scale(w, n * (w.K / 64) + k / 64);
    } else {
      v = make_uint4(0, 0, 0, 0);
      sc = 0.0f;
    }
  }
  __device__ void store(u16* S, const float* sL, int tid) const {
    const int lane = tid & 63, wv = tid >> 6;
    uint32_t o[16];
    dequant32(v, sc, sL, o);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[(32 * wv + 2 * i) * PITCH + lane] = (u16)(o[i] & 0xFFFFu);
      S[(32 * wv + 2 * i + 1) * PITCH + lane] = (u16)(o[i] >> 16);
    }
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int ASRC, int BSRC, int LORA, int OUT, bool STORE_T>
__global__ __launch_bounds__(NTHREADS) void k_gemm(GemmArgs p) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  constexpr int SA_E = ASRC == SRC_TR ? BK * (BM + 8) : BM * PITCH;
  constexpr int SB_E = BSRC == SRC_TF32SR ? BK * (BN + 8) : BN * PITCH;
  __shared__ __attribute__((aligned(16))) u16 sA[SA_E];
  __shared__ __attribute__((aligned(16))) u16 sB[SB_E];
  constexpr bool SPLIT = (BSRC == SRC_TF32S || BSRC == SRC_TF32SR);
  __shared__ __attribute__((aligned(16))) u16 sB2[SPLIT ? SB_E : 8];
  __shared__ float sL[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t i0 = (int64_t)blockIdx.x * BM;
  const int64_t j0 = (int64_t)blockIdx.y * BN;
  const int64_t cs0 = (int64_t)blockIdx.z * p.c_per_split;
  const int64_t cs1 = min(p.C, cs0 + p.c_per_split);

  if (tid < 16) sL[tid] = p.w.lv[tid];   // the weight's codebook (unused without a weight)

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  auto mma_tile = [&]() {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t fa[TM], fb[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        if constexpr (ASRC == SRC_TR)
          fa[a] = read_tr(sA, BM + 8, wm * (BM / WM) + a * 32, ks, lane);
        else
          fa[a] = *reinterpret_cast<const bf16x8_t*>(
              sA + (wm * (BM / WM) + a * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        if constexpr (BSRC == SRC_TF32SR)
          fb[b] = read_tr(sB, BN + 8, wn * (BN / WN) + b * 32, ks, lane);
        else
          fb[b] = *reinterpret_cast<const bf16x8_t*>(
              sB + (wn * (BN / WN) + b * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8);
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
      if constexpr (SPLIT) {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          if constexpr (BSRC == SRC_TF32SR)
            fb[b] = read_tr(sB2, BN + 8, wn * (BN / WN) + b * 32, ks, lane);
          else
            fb[b] = *reinterpret_cast<const bf16x8_t*>(
                sB2 + (wn * (BN / WN) + b * 32 + (lane & 31)) * PITCH + ks * 16 + (lane >> 5) * 8);
        }
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
      }
    }
  };

  // ---- LoRA prologue ----
  if constexpr (LORA != LORA_NONE) {
    for (int64_t c0 = 0; c0 < p.r; c0 += BK) {
      ProdCCF32<BM> la;
      la.load(p.la, p.r, p.I, p.r, i0, c0, p.la_vec, tid);
      if constexpr (LORA == LORA_FWD) {
        ProdCC<BN> lb;  // B [J][r]
        lb.load(p.lb, p.r, p.J, p.r, j0, c0, p.lb_vec, tid);
        __syncthreads();
        la.store(sA, tid);
        lb.store(sB, tid);
      } else {
        ProdT<BN> lb;   // A [r][J]
        lb.load(p.lb, p.J, p.r, p.J, j0, c0, p.lb_vec, tid);
        __syncthreads();
        la.store(sA, tid);
        lb.store(sB, tid);
      }
      __syncthreads();
      mma_tile();
    }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][b][v] *= p.s;
  }

  // ---- main contraction ----
  using PA = typename std::conditional<
      ASRC == SRC_CC, ProdCC<BM>,
      typename std::conditional<ASRC == SRC_TR, ProdTR<BM>, ProdT<BM>>::type>::type;
  PA pa;
  ProdCC<BN> pbcc;
  ProdT<BN> pbt;
  ProdTF32S<BN> pbs;
  ProdTF32SR<BN> pbr;
  ProdNF4CC pn;
  ProdNF4T pnt;
  const u16* bsrc = reinterpret_cast<const u16*>(p.b);

  auto load_stage = [&](int64_t c0) {
    if constexpr (ASRC == SRC_CC) pa.load(p.a, p.lda, p.I, p.C, i0, c0, p.a_vec, tid);
    else pa.load(p.a, p.lda, p.C, p.I, i0, c0, p.a_vec, tid);
    if constexpr (BSRC == SRC_CC) pbcc.load(bsrc, p.ldb, p.J, p.C, j0, c0, p.b_vec, tid);
    else if constexpr (BSRC == SRC_T) pbt.load(bsrc, p.ldb, p.C, p.J, j0, c0, p.b_vec, tid);
    else if constexpr (BSRC == SRC_TF32S)
      pbs.load(reinterpret_cast<const float*>(p.b), p.ldb, p.C, p.J, j0, c0, p.b_vec, tid);
    else if constexpr (BSRC == SRC_TF32SR)
      pbr.load(reinterpret_cast<const float*>(p.b), p.ldb, p.C, p.J, j0, c0, p.b_vec, tid);
    else if constexpr (BSRC == SRC_NF4CC) pn.load(p.w, j0, c0, tid);
    else pnt.load(p.w, j0, c0, tid);
  };
  auto store_stage = [&]() {
    pa.store(sA, tid);
    if constexpr (BSRC == SRC_CC) pbcc.store(sB, tid);
    else if constexpr (BSRC == SRC_T) pbt.store(sB, tid);
    else if constexpr (BSRC == SRC_TF32S) pbs.store(sB, sB2, tid);
    else if constexpr (BSRC == SRC_TF32SR) pbr.store(sB, sB2, tid);
    else if constexpr (BSRC == SRC_NF4CC) pn.store(sB, sL, tid);
    else pnt.store(sB, sL, tid);
  };

  if (cs0 < cs1) {
    load_stage(cs0);
    for (int64_t c0 = cs0; c0 < cs1; c0 += BK) {
      __syncthreads();
      store_stage();
      __syncthreads();
      if (c0 + BK < cs1) load_stage(c0 + BK);
      mma_tile();
    }
  }

  // ---- epilogue ----
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int64_t j = j0 + wn * (BN / WN) + b * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + wm * (BM / WM) + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (i < p.I && j < p.J) {
          if constexpr (OUT == OUT_F32) {
            float* o = reinterpret_cast<float*>(p.out);
            o[((int64_t)blockIdx.z * p.I + i) * p.J + j] = acc[a][b][v];
          } else {
            u16* o = reinterpret_cast<u16*>(p.out);
            const u16 h = f32_to_bf16(acc[a][b][v] * p.out_scale);
            if constexpr (STORE_T) o[j * p.ldo + i] = h;
            else o[i * p.ldo + j] = h;
          }
        }
      }
    }
}

// Sum split partials [splits][I][J] in order, scale, round to bf16; store
// [I][J] (ldo) or transposed [J][I] (ldo).
template <typename OutT>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int splits,
                                                int64_t I, int64_t J, float scale,
                                                OutT* __restrict__ out, int64_t ldo, bool trans) {
  const int64_t n = I * J;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += part[(int64_t)z * n + e];
    const int64_t i = e / J, j = e % J;
    OutT h;
    if constexpr (sizeof(OutT) == 2) h = f32_to_bf16(s * scale);
    else h = s * scale;
    if (trans) out[j * ldo + i] = h;
    else out[i * ldo + j] = h;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static bool vec_ok(const void* p, int64_t ld) {
  return ((uintptr_t)p % 16 == 0) && (ld % 8 == 0);
}

int rank_tile(int r) { return r <= 32 ? 32 : (r <= 64 ? 64 : 128); }

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups a skinny product aims for (two 128-row workgroups per CU):
// doubling it shortened no product and doubled the fixed-order reduction.
constexpr int64_t kSkinnyWorkgroups = 512;

SkinnyPlan skinny_plan(int64_t I, int64_t C) {
  const int64_t tiles = cdiv(I, 128);
  const int64_t ctiles = cdiv(C, BK);
  int64_t splits = std::max<int64_t>(1, cdiv(kSkinnyWorkgroups, tiles));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, ctiles / 4));
  splits = std::min<int64_t>(splits, 64);
  const int64_t per = cdiv(ctiles, splits) * BK;
  SkinnyPlan pl;
  pl.splits = (int)cdiv(C, per);
  pl.c_per_split = per;
  return pl;
}

int64_t skinny_partial_elems(int64_t I, int64_t C, int r) {
  const SkinnyPlan pl = skinny_plan(I, C);
  return (int64_t)pl.splits * I * r;
}

template <typename OutT>
static hipError_t launch_reduce(const float* part, int splits, int64_t I, int64_t J, float scale,
                                OutT* out, int64_t ldo, bool trans, hipStream_t st) {
  int64_t grid = std::min<int64_t>(cdiv(I * J, 256), 8192);
  hipLaunchKernelGGL(k_reduce<OutT>, dim3((unsigned)grid), dim3(256), 0, st, part, splits, I, J,
                     scale, out, ldo, trans);
  return hipGetLastError();
}

template <int ASRC, int BSRC>
static hipError_t launch_skinny(GemmArgs& p, hipStream_t st) {
  const SkinnyPlan pl = skinny_plan(p.I, p.C);
  p.c_per_split = pl.c_per_split;
  dim3 grid((unsigned)cdiv(p.I, 128), 1, (unsigned)pl.splits);
  const int rt = rank_tile((int)p.J);
  if (rt == 32)
    hipLaunchKernelGGL((k_gemm<128, 32, 4, 1, ASRC, BSRC, LORA_NONE, OUT_F32, false>), grid,
                       dim3(NTHREADS), 0, st, p);
  else if (rt == 64)
    hipLaunchKernelGGL((k_gemm<128, 64, 4, 1, ASRC, BSRC, LORA_NONE, OUT_F32, false>), grid,
                       dim3(NTHREADS), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemm<128, 128, 4, 1, ASRC, BSRC, LORA_NONE, OUT_F32, false>), grid,
                       dim3(NTHREADS), 0, st, p);
  return hipGetLastError();
}

static GemmArgs zero_args() {
  GemmArgs p;
  __builtin_memset(&p, 0, sizeof(p));
  p.out_scale = 1.0f;
  return p;
}

hipError_t launch_lora_down(const u16* X, const u16* A, int64_t M, int64_t K, int r,
                            float* ws, float* T, hipStream_t st) {
  GemmArgs p = zero_args();
  p.a = X; p.lda = K; p.a_vec = vec_ok(X, K);
  p.b = A; p.ldb = K; p.b_vec = vec_ok(A, K);
  p.I = M; p.J = r; p.C = K;
  p.out = ws;
  hipError_t e = launch_skinny<SRC_CC, SRC_CC>(p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(ws, skinny_plan(M, K).splits, M, r, 1.0f, T, r, false, st);
}

hipError_t launch_lora_u(const u16* dY, const u16* B, int64_t M, int64_t N, int r, float* ws,
                         float* U, hipStream_t st) {
  GemmArgs p = zero_args();
  p.a = dY; p.lda = N; p.a_vec = vec_ok(dY, N);
  p.b = B; p.ldb = r; p.b_vec = vec_ok(B, r);
  p.I = M; p.J = r; p.C = N;
  p.out = ws;
  hipError_t e = launch_skinny<SRC_CC, SRC_T>(p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(ws, skinny_plan(M, N).splits, M, r, 1.0f, U, r, false, st);
}

hipError_t launch_lora_db(const u16* dY, const float* T, int64_t M, int64_t N, int r, float s,
                          float* ws, u16* dB, hipStream_t st) {
  GemmArgs p = zero_args();
  p.a = dY; p.lda = N; p.a_vec = vec_ok(dY, N);
  p.b = T; p.ldb = r; p.b_vec = vec_ok(T, r * 2);
  p.I = N; p.J = r; p.C = M;
  p.out = ws;
  hipError_t e = launch_skinny<SRC_TR, SRC_TF32SR>(p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(ws, skinny_plan(N, M).splits, N, r, s, dB, r, false, st);
}

hipError_t launch_lora_da(const float* U, const u16* X, int64_t M, int64_t K, int r, float s,
                          float* ws, u16* dA, hipStream_t st) {
  // dA^T [K][r] = X^T U, stored transposed into dA [r][K]
  GemmArgs p = zero_args();
  p.a = X; p.lda = K; p.a_vec = vec_ok(X, K);
  p.b = U; p.ldb = r; p.b_vec = vec_ok(U, r * 2);
  p.I = K; p.J = r; p.C = M;
  p.out = ws;
  hipError_t e = launch_skinny<SRC_TR, SRC_TF32SR>(p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(ws, skinny_plan(K, M).splits, K, r, s, dA, K, true, st);
}

// Tile-128 fused GEMMs for the shapes the buffer-load kernels of gemm_big.hip
// do not take (activation rows that are not 16-byte aligned, or operands of
// 2 GiB and more): same math, guarded loads.
hipError_t launch_fwd_generic(const NF4View& w, const u16* X, int64_t M, const float* T,
                           const u16* B, int r, float s, u16* Y, hipStream_t st) {
  GemmArgs p = zero_args();
  p.a = X; p.lda = w.K; p.a_vec = vec_ok(X, w.K);
  p.w = w;
  p.I = M; p.J = w.N; p.C = w.K; p.c_per_split = w.K;
  p.la = T; p.lb = B; p.r = r; p.s = s; p.la_vec = vec_ok(T, r * 2); p.lb_vec = vec_ok(B, r);
  p.out = Y; p.ldo = w.N;
  dim3 grid((unsigned)cdiv(M, 128), (unsigned)cdiv(w.N, 128), 1);
  hipLaunchKernelGGL((k_gemm<128, 128, 2, 2, SRC_CC, SRC_NF4CC, LORA_FWD, OUT_BF16, false>), grid,
                     dim3(NTHREADS), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_dx_generic(const NF4View& w, const u16* dY, int64_t M, const float* U,
                          const u16* A, int r, float s, u16* dX, hipStream_t st) {
  GemmArgs p = zero_args();
  p.a = dY; p.lda = w.N; p.a_vec = vec_ok(dY, w.N);
  p.w = w;
  p.I = M; p.J = w.K; p.C = w.N; p.c_per_split = w.N;
  p.la = U; p.lb = A; p.r = r; p.s = s; p.la_vec = vec_ok(U, r * 2); p.lb_vec = vec_ok(A, w.K);
  p.out = dX; p.ldo = w.K;
  dim3 grid((unsigned)cdiv(M, 128), (unsigned)cdiv(w.K, 128), 1);
  hipLaunchKernelGGL((k_gemm<128, 128, 2, 2, SRC_CC, SRC_NF4T, LORA_DX, OUT_BF16, false>), grid,
                     dim3(NTHREADS), 0, st, p);
  return hipGetLastError();
}


}  // namespace qln
