// quant.hip -- NF4 quantization (absmax per 64, nearest-level encode, pack,
// double quantization of the scales to E4M3 per 256 blocks) and streaming
// dequantization to bf16.  The second level of the scales is E4M3 (vnread)
// or, in the uint8-linear reading of the Ultralytics bullet ("8 bits"), an
// integer grid 0 .. 255 times max / 255; or the scales stay fp32.
//
// Method: Ultralytics glossary "QLoRA", "How QLoRA works" (NF4 bullet, double
// quantization bullet, the encoding snippet); vnread "Grokking QLoRA",
// "Double Quantization" (FP8 second level).  Both kernels are HBM-bound
// streams; the encode avoids a per-element IEEE division (see k_quantize).
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.h"
#include "device.h"

namespace qln {

// ---------------------------------------------------------------------------
// Host: decision points of the nearest-level rule, derived from the level
// table by walking fp32 values around each midpoint.
// ---------------------------------------------------------------------------
static float level(const uint32_t* bits, int i) { return __builtin_bit_cast(float, bits[i]); }

static bool takes_upper(const uint32_t* bits, float v, int j) {
  volatile float du = level(bits, j + 1) - v;
  volatile float dl = v - level(bits, j);
  return std::fabs(du) < std::fabs(dl);  // a tie keeps the lower code
}

static EncodeCuts make_cuts(const uint32_t* bits) {
  EncodeCuts cuts;
  for (int j = 0; j < 15; ++j) {
    float v = (float)(((double)level(bits, j) + (double)level(bits, j + 1)) * 0.5);
    while (takes_upper(bits, std::nextafterf(v, -2.0f), j)) v = std::nextafterf(v, -2.0f);
    while (!takes_upper(bits, v, j)) v = std::nextafterf(v, 2.0f);
    cuts.cut[j] = v;
  }
  cuts.zero_code = 0;  // the code of v = 0
  for (int j = 0; j < 15; ++j) cuts.zero_code += cuts.cut[j] <= 0.0f ? 1 : 0;
  return cuts;
}

const EncodeCuts& encode_cuts(int codebook) {
  static EncodeCuts cuts[2];
  static std::once_flag once;
  std::call_once(once, [] {
    cuts[CODEBOOK_NF4] = make_cuts(kNF4LevelBits);
    cuts[CODEBOOK_INT4] = make_cuts(kINT4LevelBits);
  });
  return cuts[codebook == CODEBOOK_INT4 ? CODEBOOK_INT4 : CODEBOOK_NF4];
}

// ---------------------------------------------------------------------------
// Quantize.  One workgroup (256 threads) per group of 256 blocks (16384
// contiguous fp32, 64 KiB).  Each wave load instruction reads 1 KiB of
// contiguous weights: four blocks, 16 lanes per block, 4 elements per lane;
// each wave reads its own contiguous quarter of the group, and a lane issues
// all 16 of its loads before any arithmetic.  The packed codes
// (two bytes per lane and load) and the group's 8-bit scales are collected in
// LDS and leave as 16-byte nontemporal stores, which costs HBM less than
// narrow stores interleaved with the read stream.
//
// Exact encode without a per-element division: with y = RN(1/a) the product
// q = RN(x*y) lies within 2 ulp of RN(x/a).  The code of v is the number of
// decision points cut[j] <= v; an LDS table of 1/128-wide bins over [-1, 1]
// holds, per bin, the only decision point that can fall inside it (decision
// points are >= 0.079 apart) and the count below it.  Whenever q is within
// 2^-20 of that decision point, or the block scale is outside [2^-100, 2^100]
// (including an all-zero block), the lane redoes its elements with an IEEE
// division, so the result always equals code(RN(x/a)).  The same holds for any
// codebook whose decision points are at least 1/128 apart (NF4, INT4).
//
// FP32 (no double quantization, Transformers "Bitsandbytes" 4-bit section):
// the group's exact block absmax values go to dscale[b] as fp32 and qscale is
// not written.
// ---------------------------------------------------------------------------
constexpr int QBINS = 256;
constexpr float BIN_PAD = 0x1p-12f;
constexpr float NEAR_EPS = 0x1p-20f;

struct BinEntry {
  float cut;   // the decision point in the (padded) bin, or 4.0 if none
  int base;    // number of decision points below the padded bin
};

// clamped bin of a value in [-1, 1] (slow path)
__device__ __forceinline__ int bin_of(float q) {
  int b = (int)((q + 1.0f) * 128.0f);
  return min(max(b, 0), QBINS - 1);
}

template <int FMT>
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ qscale,
                                                  float* __restrict__ dscale,
                                                  float* __restrict__ absmax_out,
                                                  EncodeCuts cuts) {
  // entry QBINS repeats entry QBINS - 1, for q a hair above 1 on the fast path
  __shared__ BinEntry s_bin[QBINS + 1];
  __shared__ uint16_t s_codes[256 * 16];  // the group's packed codes, 32 bytes per block
  __shared__ uint32_t s_q[64];            // the group's 8-bit scales
  __shared__ float s_amax[256];
  __shared__ float s_wmax[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256;
  const int nbg = (int)min<int64_t>(256, nblocks - b0);

  // wave w streams its own 16 KiB: load p covers blocks 4 (16w + p) .. 4 (16w + p) + 3
  f32x4_t v[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int bi = (wave * 16 + p) * 4 + (lane >> 4);
    if (bi < nbg) {
      v[p] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(W + (b0 + bi) * 64 + (lane & 15) * 4));
    } else {
      v[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  // bin table, built while the loads are in flight
  for (int i = tid; i <= QBINS; i += 256) {
    const int ib = min(i, QBINS - 1);
    const float lo = -1.0f + (float)ib * (1.0f / 128.0f) - BIN_PAD;
    const float hi = -1.0f + (float)(ib + 1) * (1.0f / 128.0f) + BIN_PAD;
    int base = 0;
    float cut = 4.0f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const float c = cuts.cut[j];
      base += (c < lo) ? 1 : 0;
      cut = (c >= lo && c <= hi) ? c : cut;
    }
    s_bin[i].cut = cut;
    s_bin[i].base = base;
  }

  __syncthreads();  // bin table ready

#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int bi = (wave * 16 + p) * 4 + (lane >> 4);
    const float x[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
    const float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    const float a = max16(m);
    const bool safe = (a >= 0x1p-100f) && (a <= 0x1p100f);
    // correctly rounded reciprocal; 0 for an unsafe scale keeps the fast
    // path's bin index in range (that lane takes the slow path anyway)
    const float y = safe ? 1.0f / a : 0.0f;
    uint32_t word = 0;
    bool near = !safe;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = x[e] * y;
      // |q| <= 1 + 2^-23, so fma(q, 128, 128) = RN(q + 1) * 128 truncates to
      // 0 .. 256 with no clamp
      const BinEntry be = s_bin[(int)__builtin_fmaf(q, 128.0f, 128.0f)];
      const float dlt = q - be.cut;  // zero only when q == cut (denormals kept)
      word |= (uint32_t)(be.base + (dlt >= 0.0f ? 1 : 0)) << (4 * e);
      near |= fabsf(dlt) <= NEAR_EPS;
    }
    if (near) {  // rare: exact quotients for this lane's 4 elements
      word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int c = cuts.zero_code;  // all-zero block: the code of v = 0
        if (a > 0.0f) {
          const float q = x[e] / a;
          const BinEntry be = s_bin[bin_of(q)];
          c = be.base + (q >= be.cut ? 1 : 0);
        }
        word |= (uint32_t)c << (4 * e);
      }
    }
    s_codes[bi * 16 + (lane & 15)] = (uint16_t)word;  // even element in the low nibble
    if (bi < nbg && (lane & 15) == 0) {
      s_amax[bi] = a;
      if (absmax_out) absmax_out[b0 + bi] = a;
    }
  }
  __syncthreads();

  for (int i = tid; i < nbg * 2; i += 256)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(&s_codes[i * 8]),
                                reinterpret_cast<u32x4_t*>(codes + b0 * 32) + i);

  const float a_t = tid < nbg ? s_amax[tid] : 0.0f;
  if constexpr (FMT == SCALE_FP32) {  // the scales themselves, no double quantization
    if (tid < nbg) dscale[b0 + tid] = a_t;
    return;
  }
  // double quantization of this group's block scales
  const float wm = wave_max(a_t);
  if (lane == 0) s_wmax[wave] = wm;
  __syncthreads();
  const float c = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  if constexpr (FMT == SCALE_U8) {
    // uint8-linear: the nearest of 0, d, ..., 255 d with d = max / 255
    // (the quotient rounded half to even; IEEE division)
    const float d = c / 255.0f;
    if (tid == 0) dscale[g] = d;
    reinterpret_cast<uint8_t*>(s_q)[tid] = (uint8_t)(d == 0.0f ? 0u : (uint32_t)fminf(rintf(a_t / d), 255.0f));
  } else {
    const float d = c / 448.0f;
    if (tid == 0) dscale[g] = d;
    reinterpret_cast<uint8_t*>(s_q)[tid] = (uint8_t)(d == 0.0f ? 0u : e4m3_encode(a_t / d));
  }
  __syncthreads();
  if (nbg == 256) {
    if (tid < 16)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(&s_q[tid * 4]),
                                  reinterpret_cast<u32x4_t*>(qscale + b0) + tid);
  } else if (tid < nbg) {
    qscale[b0 + tid] = reinterpret_cast<const uint8_t*>(s_q)[tid];
  }
}

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, int codebook, int fmt,
                           uint8_t* codes, uint8_t* qscale, float* dscale, float* absmax,
                           hipStream_t s) {
  const int64_t nb = N * K / 64;
  const int64_t ng = (nb + 255) / 256;
  if (fmt == SCALE_FP32)
    hipLaunchKernelGGL(k_quantize<SCALE_FP32>, dim3((unsigned)ng), dim3(256), 0, s, W, nb, codes, qscale,
                       dscale, absmax, encode_cuts(codebook));
  else if (fmt == SCALE_U8)
    hipLaunchKernelGGL(k_quantize<SCALE_U8>, dim3((unsigned)ng), dim3(256), 0, s, W, nb, codes, qscale,
                       dscale, absmax, encode_cuts(codebook));
  else
    hipLaunchKernelGGL(k_quantize<SCALE_E4M3>, dim3((unsigned)ng), dim3(256), 0, s, W, nb, codes, qscale,
                       dscale, absmax, encode_cuts(codebook));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: w' = bf16_RNE(fl32(L[code] * fl32(v(q) * d))), v the E4M3
// value of the scale byte or (uint8-linear) the byte itself.  One
// workgroup (4 waves) per group of 256 blocks, so d is one scalar load; wave w
// writes its own contiguous 64 blocks (8 KiB of bf16).  In step j a lane takes
// 8 codes of block 8j + lane/8 (one 4-byte load) and writes their 8 bf16 values
// with one 16-byte store, so every load instruction reads 256 contiguous bytes
// and every store instruction writes 1 KiB.  All loads are issued before any
// arithmetic; the level table (the weight's codebook) sits in LDS.  FP32: the
// block scale is dscale[b] itself.
// ---------------------------------------------------------------------------
constexpr int DQ_STEPS = 8;  // 8 blocks per wave and step

struct Levels { float v[16]; };

template <int FMT>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ qscale,
                                                    const float* __restrict__ dscale,
                                                    int64_t nblocks, u16* __restrict__ out,
                                                    Levels lv) {
  __shared__ float s_L[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256 + wave * 64;               // first block of this wave
  const int64_t nbw = min<int64_t>(64, nblocks - b0);  // its blocks (<= 0 past the end)
  if (tid < 16) s_L[tid] = lv.v[tid];
  constexpr bool FP32 = FMT == SCALE_FP32;
  const float d = FP32 ? 0.0f : dscale[g];
  const auto rQ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(qscale), (short)0,
                                                    FP32 ? 0 : (int)nblocks, 0x00020000);
  uint32_t c[DQ_STEPS], qv[DQ_STEPS];
  float sv[DQ_STEPS];
#pragma unroll
  for (int j = 0; j < DQ_STEPS; ++j) {
    const int blk = j * 8 + (lane >> 3);
    if (blk < nbw) {
      c[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + (b0 + blk) * 32) +
                                        (lane & 7));
      if constexpr (FP32) sv[j] = dscale[b0 + blk];
    } else {
      c[j] = 0;
      sv[j] = 0.0f;
    }
    // the scale byte by a buffer load (past the blocks it reads 0), outside
    // the branch: a conversion placed in the branch would wait for each load
    if constexpr (!FP32)
      qv[j] = __builtin_amdgcn_raw_buffer_load_b8(rQ, blk < nbw ? (uint32_t)(b0 + blk) : 0x80000000u, 0, 0);
  }
  __syncthreads();  // level table ready
#pragma unroll
  for (int j = 0; j < DQ_STEPS; ++j) {
    const int blk = j * 8 + (lane >> 3);
    const float sc = FP32 ? sv[j] : (FMT == SCALE_U8 ? (float)qv[j] : e4m3_decode(qv[j])) * d;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (c[j] >> (8 * i)) & 0xFFu;  // even element in the low nibble
      o[i] = pack_bf16x2(s_L[byte & 15u] * sc, s_L[byte >> 4] * sc);
    }
    if (blk < nbw)
      __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]},
                                  reinterpret_cast<u32x4_t*>(out + (b0 + blk) * 64 + (lane & 7) * 8));
  }
}

hipError_t launch_dequantize(const NF4View& w, u16* out, hipStream_t s) {
  const int64_t nb = w.N * w.K / 64;
  const int64_t ng = (nb + 255) / 256;
  Levels lv;
  for (int i = 0; i < 16; ++i) lv.v[i] = w.lv[i];
  const int fmt = scale_fmt(w);
  if (fmt == SCALE_FP32)
    hipLaunchKernelGGL(k_dequantize<SCALE_FP32>, dim3((unsigned)ng), dim3(256), 0, s, w.codes, w.qscale,
                       w.dscale, nb, out, lv);
  else if (fmt == SCALE_U8)
    hipLaunchKernelGGL(k_dequantize<SCALE_U8>, dim3((unsigned)ng), dim3(256), 0, s, w.codes, w.qscale,
                       w.dscale, nb, out, lv);
  else
    hipLaunchKernelGGL(k_dequantize<SCALE_E4M3>, dim3((unsigned)ng), dim3(256), 0, s, w.codes, w.qscale,
                       w.dscale, nb, out, lv);
  return hipGetLastError();
}

}  // namespace qln
