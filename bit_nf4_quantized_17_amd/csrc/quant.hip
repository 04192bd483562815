// quant.hip -- NF4 quantization (absmax per 64, nearest-level encode, pack,
// double quantization of the scales to E4M3 per 256 blocks) and streaming
// dequantization to bf16.
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
static float level(int i) { return __builtin_bit_cast(float, kNF4LevelBits[i]); }

static bool takes_upper(float v, int j) {
  volatile float du = level(j + 1) - v;
  volatile float dl = v - level(j);
  return std::fabs(du) < std::fabs(dl);  // a tie keeps the lower code
}

const EncodeCuts& encode_cuts() {
  static EncodeCuts cuts;
  static std::once_flag once;
  std::call_once(once, [] {
    for (int j = 0; j < 15; ++j) {
      float v = (float)(((double)level(j) + (double)level(j + 1)) * 0.5);
      while (takes_upper(std::nextafterf(v, -2.0f), j)) v = std::nextafterf(v, -2.0f);
      while (!takes_upper(v, j)) v = std::nextafterf(v, 2.0f);
      cuts.cut[j] = v;
    }
  });
  return cuts;
}

// ---------------------------------------------------------------------------
// Quantize.  One workgroup (256 threads) per group of 256 blocks (16384
// contiguous fp32, 64 KiB).  A wave pass covers 8 consecutive blocks: 8 lanes
// per block, 8 consecutive elements per lane (two 16-byte loads), so each
// lane emits one 32-bit word of packed codes.
//
// Exact encode without a per-element division: with y = RN(1/a) the product
// q = RN(x*y) lies within 2 ulp of RN(x/a).  The code of v is the number of
// decision points cut[j] <= v; a 256-bin LDS table over [-1, 1] holds, per
// bin, the only decision point that can fall inside it (bins are 1/128 wide,
// decision points >= 0.079 apart) and the count below it.  Whenever q is
// within 2^-20 of that decision point, or the block scale is outside
// [2^-100, 2^100] (including an all-zero block), the lane redoes the element
// with an IEEE division, so the result always equals code(RN(x/a)).
// ---------------------------------------------------------------------------
constexpr int QBINS = 256;
constexpr float BIN_PAD = 0x1p-12f;
constexpr float NEAR_EPS = 0x1p-20f;

struct BinEntry {
  float cut;   // the decision point in the (padded) bin, or 4.0 if none
  int base;    // number of decision points below the padded bin
};

__device__ __forceinline__ int bin_of(float q) {
  int b = (int)((q + 1.0f) * 128.0f);
  return min(max(b, 0), QBINS - 1);
}

__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t nblocks,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ qscale,
                                                  float* __restrict__ dscale,
                                                  float* __restrict__ absmax_out,
                                                  EncodeCuts cuts) {
  __shared__ BinEntry s_bin[QBINS];
  __shared__ float s_amax[256];
  __shared__ float s_wmax[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t g = blockIdx.x;
  const int64_t b0 = g * 256;
  const int nbg = (int)min<int64_t>(256, nblocks - b0);

  // issue all loads first, then build the bin table while they are in flight
  f32x4_t v[8][2];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    int bi = p * 32 + wave * 8 + (lane >> 3);
    if (bi < nbg) {
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(W + (b0 + bi) * 64 + (lane & 7) * 8);
      v[p][0] = __builtin_nontemporal_load(src);
      v[p][1] = __builtin_nontemporal_load(src + 1);
    } else {
      v[p][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      v[p][1] = v[p][0];
    }
  }
  for (int i = tid; i < QBINS; i += 256) {
    float lo = -1.0f + (float)i * (1.0f / 128.0f) - BIN_PAD;
    float hi = -1.0f + (float)(i + 1) * (1.0f / 128.0f) + BIN_PAD;
    int base = 0;
    float cut = 4.0f;
    for (int j = 0; j < 15; ++j) {
      float c = cuts.cut[j];
      if (c < lo) base++;
      else if (c <= hi) cut = c;
    }
    s_bin[i].cut = cut;
    s_bin[i].base = base;
  }

  __syncthreads();  // bin table ready

#pragma unroll
  for (int p = 0; p < 8; ++p) {
    int bi = p * 32 + wave * 8 + (lane >> 3);
    float x[8] = {v[p][0].x, v[p][0].y, v[p][0].z, v[p][0].w,
                  v[p][1].x, v[p][1].y, v[p][1].z, v[p][1].w};
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
    const float a = max8(m);
    const bool safe = (a >= 0x1p-100f) && (a <= 0x1p100f);
    const float y = 1.0f / a;  // correctly rounded (IEEE division)
    uint32_t word = 0;
    bool near = !safe;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = x[e] * y;
      BinEntry be = s_bin[bin_of(q)];
      int c = be.base + (q >= be.cut ? 1 : 0);
      near |= fabsf(q - be.cut) <= NEAR_EPS;
      word |= (uint32_t)c << (4 * e);
    }
    if (near) {  // rare: exact quotients for this lane's 8 elements
      word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int c = 7;  // all-zero block: the exact zero level
        if (a > 0.0f) {
          float q = x[e] / a;
          BinEntry be = s_bin[bin_of(q)];
          c = be.base + (q >= be.cut ? 1 : 0);
        }
        word |= (uint32_t)c << (4 * e);
      }
    }
    if (bi < nbg) {
      __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(codes + (b0 + bi) * 32 + (lane & 7) * 4));
      if ((lane & 7) == 0) {
        s_amax[bi] = a;
        if (absmax_out) absmax_out[b0 + bi] = a;
      }
    }
  }
  __syncthreads();

  // double quantization of this group's block scales
  const float a_t = tid < nbg ? s_amax[tid] : 0.0f;
  const float wm = wave_max(a_t);
  if (lane == 0) s_wmax[wave] = wm;
  __syncthreads();
  const float c = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));
  const float d = c / 448.0f;
  if (tid == 0) dscale[g] = d;
  if (tid < nbg) qscale[b0 + tid] = (uint8_t)(d == 0.0f ? 0u : e4m3_encode(a_t / d));
}

hipError_t launch_quantize(const float* W, int64_t N, int64_t K, uint8_t* codes,
                           uint8_t* qscale, float* dscale, float* absmax, hipStream_t s) {
  const int64_t nb = N * K / 64;
  const int64_t ng = (nb + 255) / 256;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)ng), dim3(256), 0, s, W, nb, codes, qscale,
                     dscale, absmax, encode_cuts());
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: w' = bf16_RNE(fl32(L[code] * fl32(E4M3(q) * d))).  Each thread
// converts 16 consecutive elements (8 code bytes -> 32 output bytes); the
// level table sits in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ qscale,
                                                    const float* __restrict__ dscale,
                                                    int64_t nchunks, u16* __restrict__ out) {
  __shared__ float s_L[16];
  if (threadIdx.x < 16) s_L[threadIdx.x] = __uint_as_float(kNF4LevelBits[threadIdx.x]);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; ch < nchunks; ch += stride) {
    const int64_t blk = ch >> 2;  // 4 chunks of 16 per block of 64
    const float sc = e4m3_decode(qscale[blk]) * dscale[blk >> 8];
    const u32x2_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(codes) + ch);
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t byte = ((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu;
      o[i] = pack_bf16x2(s_L[byte & 15u] * sc, s_L[byte >> 4] * sc);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + ch * 16);
    __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, dst);
    __builtin_nontemporal_store(u32x4_t{o[4], o[5], o[6], o[7]}, dst + 1);
  }
}

hipError_t launch_dequantize(const NF4View& w, u16* out, hipStream_t s) {
  const int64_t nchunks = w.N * w.K / 16;
  int64_t grid = (nchunks + 255) / 256;
  grid = std::min<int64_t>(grid, 256 * 64);
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)grid), dim3(256), 0, s, w.codes, w.qscale,
                     w.dscale, nchunks, out);
  return hipGetLastError();
}

}  // namespace qln
