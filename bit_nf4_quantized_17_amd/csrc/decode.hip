// decode.hip -- the forward at decode sizes (M <= 16 tokens), one kernel per
// call.  Ultralytics glossary "QLoRA", "How QLoRA works": the frozen layer
// dequantizes NF4 to bfloat16 for the matrix product and adds the LoRA path.
//
// At M <= 16 the layer is bound by streaming the packed weight (0.52 bytes
// per weight) from HBM, which leaves about three vector-ALU operations per
// weight at full bandwidth -- less than an exact per-element dequantization
// costs.  So this path factors the block scale out of the product:
//   Y[m][n] = sum_blocks s_b * ( sum_{k in block} X[m][k] * bf16(L[code]) )
//           + s_lora * sum_j T[m][j] B[n][j]
// bf16(L[code]) comes from an LDS table indexed by one code byte (two codes
// -> one bf16 pair), replicated 32 times so that a wave's lookups never share
// a bank; each 64-code block is one pair of v_mfma_f32_16x16x32_bf16 into a
// fresh accumulator, which is then scaled by the block's restored scale and
// added in fp32.  (The prefill and training kernels multiply the exactly
// dequantized bf16 weight instead; both round the weight's relative value
// once to bf16 precision.)
//
// Work split: a workgroup of 8 waves owns 64 output columns n (four 16-wide
// MFMA tiles; 16 for narrow weights) over the full contraction K; wave w
// takes an eighth of the 64-blocks for all tiles, so each X / A fragment it
// loads from L2 serves four weight tiles, keeps the code loads of 4 blocks x
// 4 tiles in flight, and the eight partial results are summed in LDS in wave
// order.  For ranks above 32, T comes from the split-contraction kernel first.  T = X A^T (needed by every workgroup for its LoRA term) is computed
// alongside from the same X fragments; workgroup 0 also writes it to T_save.
#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"

namespace qln {
namespace dec {

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int LUT_COPIES = 32;
constexpr int MAX_RQ = 2;       // rank tiles of 16 computed here (r <= 32)

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct DecArgs {
  const u16* X; int64_t M;          // X [M][K], M <= 16
  NF4View w;                        // W [N][K]
  const u16* A; const u16* B; int r; float s;
  u16* Y; float* T_save;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One workgroup = 8 waves on TILES 16-column tiles of Y; wave w takes blocks
// [w*nbk/8, (w+1)*nbk/8) of the contraction for all TILES tiles, four blocks
// at a time.  The weight stream is read coalesced -- lane l loads the 32 code
// bytes of block l%4 of row l/4 (each row's 4 blocks are 128 contiguous
// bytes) and that block's two scale bytes -- then passes through a
// wave-private LDS staging area to reach the MFMA layout.  The next batch's
// loads are issued before the current batch is multiplied.
constexpr int STG_PITCH = 144;                 // bytes per staged row (128 + 16)
constexpr int STG_BYTES = 16 * STG_PITCH;      // codes of one tile x 4 blocks
constexpr int STG_SC = 16 * 4 * 4;             // scales of one tile x 4 blocks

// TIN: T was computed beforehand (ranks above 32) and is read from T_save.
template <int TILES, bool TIN>
__global__ __launch_bounds__(NTHREADS) void k_decode(DecArgs p) {
  constexpr int LUT_WORDS = 256 * LUT_COPIES;
  constexpr int SLOTS = TILES + MAX_RQ;
  constexpr int RED_WORDS = WAVES * SLOTS * 64 * 4;
  constexpr int LUT_RED_WORDS = LUT_WORDS > RED_WORDS ? LUT_WORDS : RED_WORDS;
  // [table / cross-wave sums][per-wave staging of codes and scales]
  __shared__ __attribute__((aligned(16))) uint32_t smem[LUT_RED_WORDS + WAVES * TILES * (STG_BYTES + STG_SC) / 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int lrow = lane >> 2, lblk = lane & 3;          // this lane's load: row, block within the batch
  const int64_t n0 = (int64_t)blockIdx.x * 16 * TILES;
  const uint32_t K = (uint32_t)p.w.K;
  const int nbk = (int)(K / 64);
  const int rq = TIN ? 0 : (p.r + 15) / 16;   // rank tiles computed here

  for (int e = tid; e < LUT_WORDS; e += NTHREADS) {
    const int byte = e / LUT_COPIES;
    smem[e] = pack_bf16x2(__uint_as_float(kNF4LevelBits[byte & 15]),
                          __uint_as_float(kNF4LevelBits[byte >> 4]));
  }
  __syncthreads();

  uint8_t* stg = reinterpret_cast<uint8_t*>(smem + LUT_RED_WORDS) +
                 (size_t)wave * TILES * (STG_BYTES + STG_SC);

  const auto rX = rsrc(p.X, (uint32_t)(p.M * K * 2));
  const auto rA = rsrc(p.A, (uint32_t)(p.r * K * 2));
  const auto rC = rsrc(p.w.codes, (uint32_t)(p.w.N * K / 2));
  const auto rQ = rsrc(p.w.qscale, (uint32_t)(p.w.N * K / 64));
  const auto rD = rsrc(p.w.dscale, (uint32_t)(4 * ((p.w.N * K / 64 + 255) / 256)));

  f32x4_t acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t tacc[MAX_RQ];
#pragma unroll
  for (int q = 0; q < MAX_RQ; ++q) tacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int b0 = wave * nbk / WAVES, b1 = (wave + 1) * nbk / WAVES;
  const uint32_t lut_lane = (uint32_t)(lane & (LUT_COPIES - 1));
  const uint32_t xoff = (uint32_t)i16 * K * 2 + 32u * g;   // k = 64*blk + 16*g + 8*step + t
  uint32_t crow[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) crow[t] = (uint32_t)(n0 + 16 * t + lrow);

  struct Batch { u32x4v c0[TILES], c1[TILES]; uint32_t q[TILES]; float d[TILES]; };
  auto load_batch = [&](Batch& bt, int bb) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const uint32_t blk = (uint32_t)(bb + lblk);
      const uint32_t off = crow[t] * (K / 2) + 32u * blk;
      bt.c0[t] = __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 0);
      bt.c1[t] = __builtin_amdgcn_raw_buffer_load_b128(rC, off + 16, 0, 0);
      const uint32_t qb = crow[t] * (K / 64) + blk;
      bt.q[t] = __builtin_amdgcn_raw_buffer_load_b8(rQ, qb, 0, 0);
      bt.d[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, 4 * (qb >> 8), 0, 0));
    }
  };

  Batch cur, nxt;
  load_batch(cur, b0);
  for (int bb = b0; bb < b1; bb += 4) {
    load_batch(nxt, bb + 4);     // past b1: unused
    // stage this batch: codes [row][4 blocks x 32 B], scales [row][4 blocks]
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      uint8_t* st = stg + t * (STG_BYTES + STG_SC);
      *reinterpret_cast<u32x4v*>(st + lrow * STG_PITCH + 32 * lblk) = cur.c0[t];
      *reinterpret_cast<u32x4v*>(st + lrow * STG_PITCH + 32 * lblk + 16) = cur.c1[t];
      reinterpret_cast<float*>(st + STG_BYTES)[lrow * 4 + lblk] = e4m3_decode(cur.q[t]) * cur.d[t];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (bb + j >= b1) break;
      const uint32_t kb2 = (uint32_t)(bb + j) * 128u;   // byte offset of the block in a bf16 row
      const bf16x8_t x0 = ld16(rX, xoff + kb2);
      const bf16x8_t x1 = ld16(rX, xoff + kb2 + 16);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const uint8_t* st = stg + t * (STG_BYTES + STG_SC);
        const u32x2v c = *reinterpret_cast<const u32x2v*>(st + i16 * STG_PITCH + 32 * j + 8 * g);
        const float sc = reinterpret_cast<const float*>(st + STG_BYTES)[i16 * 4 + j];
        uint32_t wv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t byte = ((e < 4 ? c.x : c.y) >> (8 * (e & 3))) & 0xFFu;
          wv[e] = smem[byte * LUT_COPIES + lut_lane];
        }
        const bf16x8_t w0 = __builtin_bit_cast(bf16x8_t, u32x4v{wv[0], wv[1], wv[2], wv[3]});
        const bf16x8_t w1 = __builtin_bit_cast(bf16x8_t, u32x4v{wv[4], wv[5], wv[6], wv[7]});
        f32x4_t tmp = f32x4_t{0.f, 0.f, 0.f, 0.f};
        tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, w0, tmp, 0, 0, 0);
        tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, w1, tmp, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[t][e] += sc * tmp[e];
      }
#pragma unroll
      for (int q = 0; q < MAX_RQ; ++q) {
        if (q < rq) {
          const uint32_t aoff = (uint32_t)(16 * q + i16) * K * 2 + 32u * g + kb2;
          tacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x0, ld16(rA, aoff), tacc[q], 0, 0, 0);
          tacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x1, ld16(rA, aoff + 16), tacc[q], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    cur = nxt;
  }

  // ---- cross-wave sums (fixed wave order), LoRA term, store ----
  __syncthreads();   // the table is no longer read
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * SLOTS + t) * 64 + lane) * 4 + e] = acc[t][e];
#pragma unroll
  for (int q = 0; q < MAX_RQ; ++q)
    if (q < rq)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * SLOTS + TILES + q) * 64 + lane) * 4 + e] = tacc[q][e];
  __syncthreads();

  // the value of output (m, col) of slot `sl` sits in lane 16*(m/4) + col, element m%4
  auto total = [&](int sl, int m, int col) {
    const int idx = (16 * (m >> 2) + col) * 4 + (m & 3);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[(w * SLOTS + sl) * 64 * 4 + idx];
    return v;
  };

  auto t_at = [&](int m, int j) -> float {
    if constexpr (TIN) return p.T_save[m * p.r + j];
    else return total(TILES + j / 16, m, j % 16);
  };
  if (!TIN && blockIdx.x == 0) {
    for (int e = tid; e < 16 * p.r; e += NTHREADS) {
      const int m = e / p.r, j = e % p.r;
      if (m < p.M) p.T_save[m * p.r + j] = total(TILES + j / 16, m, j % 16);
    }
  }
  for (int e = tid; e < 256 * TILES; e += NTHREADS) {
    const int m = e / (16 * TILES), c = e % (16 * TILES);
    const int64_t nn = n0 + c;
    if (m < p.M && nn < p.w.N) {
      float lora = 0.0f;
      for (int j = 0; j < p.r; ++j) lora += t_at(m, j) * bf16_to_f32(p.B[nn * p.r + j]);
      p.Y[m * p.w.N + nn] = f32_to_bf16(total(c / 16, m, c % 16) + p.s * lora);
    }
  }
}

}  // namespace dec

bool decode_fits(int64_t M, const NF4View& w, int r) {
  const int64_t lim = (int64_t)1 << 31;
  return M <= 16 && w.N * w.K / 2 < lim && 16 * w.K * 2 < lim && (int64_t)r * w.K * 2 < lim;
}

template <bool TIN>
static void launch_tiles(const dec::DecArgs& p, int64_t N, hipStream_t st) {
  // as many 16-column tiles per workgroup as keeps at least 256 workgroups
  if (N >= 64 * 256)
    hipLaunchKernelGGL((dec::k_decode<4, TIN>), dim3((unsigned)((N + 63) / 64)), dim3(dec::NTHREADS),
                       0, st, p);
  else if (N >= 32 * 256)
    hipLaunchKernelGGL((dec::k_decode<2, TIN>), dim3((unsigned)((N + 31) / 32)), dim3(dec::NTHREADS),
                       0, st, p);
  else
    hipLaunchKernelGGL((dec::k_decode<1, TIN>), dim3((unsigned)((N + 15) / 16)), dim3(dec::NTHREADS),
                       0, st, p);
}

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, float* ws, hipStream_t st) {
  dec::DecArgs p;
  p.X = X; p.M = M; p.w = w; p.A = A; p.B = B; p.r = r; p.s = s; p.Y = Y; p.T_save = T_save;
  if (r <= 16 * dec::MAX_RQ) {           // T computed inside, from the same X fragments
    launch_tiles<false>(p, w.N, st);
    return hipGetLastError();
  }
  hipError_t e = launch_lora_down(X, A, M, w.K, r, ws, T_save, st);
  if (e != hipSuccess) return e;
  launch_tiles<true>(p, w.N, st);
  return hipGetLastError();
}

}  // namespace qln
