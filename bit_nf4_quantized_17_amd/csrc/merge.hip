// merge.hip -- the adapter folded into the weight, and taken out again.
// IBM "What is LoRA?": once training ends the low-rank update B A is merged
// into the pretrained weight, which then runs with no extra inference cost,
// and adapters are swapped per task; Ultralytics glossary "QLoRA",
// "Trade-offs": merging into the base needs it dequantized to 16 bit first.
//
//   merge    W_out[n][k] = bf16( W'[n][k]      + s sum_j B[n][j] A[j][k] )
//   unmerge  W_out[n][k] = bf16( W_in[n][k]    - s sum_j B[n][j] A[j][k] )
//
// with s = fl32(alpha / r) and W' the bf16 dequantized NF4 weight
// (bf16(fl32(L[code] * fl32(E4M3(q) * d))), as nf4_dequantize).  The rank-r
// sum is an fp32 MFMA product of the bf16 adapters; the base is added with
// one fused multiply-add and the result rounded once to bf16.
//
// One workgroup of 8 waves per 128 x 256 output tile.  The B rows of the tile
// ([128][r]) and the A columns ([r][256]) are staged in LDS (r padded to a
// multiple of 16 with zeros); each wave computes a 32 x 128 slice with
// v_mfma_f32_32x32x16_bf16, reading the A side with the transposing LDS read
// (ds_read_b64_tr_b16) because the contraction runs down A's columns.  The
// base of the tile (packed codes and scales, or the bf16 weight) is loaded
// into registers at the start, so its HBM latency overlaps the staging and
// the MFMAs.  The fp32 products then pass through LDS, 64 rows at a time, so
// that every output row segment is written with 16-byte stores.  The path is
// bound by HBM: it reads 0.52 bytes (merge) or 2 bytes (unmerge) and writes 2
// bytes per weight; the adapters are small and stay in the caches.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"
#include "device.h"

namespace qln {
namespace mrg {

constexpr int TN = 128, TK = 256, NTHREADS = 512;
constexpr int APITCH = TK + 16;      // A tile [RP][272] bf16 (transposing reads)
constexpr int SPITCH = TK + 4;       // fp32 staging [64][260]

typedef __attribute__((address_space(3))) short lds_short;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct MergeArgs {
  const uint8_t* codes; const uint8_t* qscale; const float* dscale;   // merge: the NF4 base
  bool fp32_scale, u8_scale; float lv[16];                            // its scale format, codebook
  const u16* w_in;                                                    // unmerge: the bf16 base
  int64_t N, K;
  const u16* A; const u16* B; int r; float s;                         // s already carries the sign
  u16* out;
};

__host__ __device__ inline int pad16(int r) { return (r + 15) / 16 * 16; }
__host__ __device__ inline int bpitch(int r) { return pad16(r) + 8; }
// dynamic LDS: B tile, A tile (both bf16), then reused as the fp32 staging
__host__ __device__ inline size_t lds_bytes(int r) {
  const size_t ab = ((size_t)TN * bpitch(r) + (size_t)pad16(r) * APITCH) * 2;
  const size_t st = (size_t)64 * SPITCH * 4;
  return ab > st ? ab : st;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// MFMA B-side fragment of a [contraction][columns] bf16 tile: for column block
// cb (32 columns) at contraction step ks, lane l receives 8 contraction values
// of column cb*32 + l%32, through two transposing 64-bit reads
__device__ __forceinline__ bf16x8_t read_cols(const u16* tile, int c0, int ks, int lane) {
  const int L = lane & 15;
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
  const int row = ks * 16 + 8 * (lane >> 5) + (L >> 2);
  const lds_short* base = (const lds_short*)(tile);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + row * APITCH + col));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (row + 4) * APITCH + col));
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// UNMERGE = false: the base is the NF4 weight; true: a bf16 weight
template <bool UNMERGE>
__global__ __launch_bounds__(NTHREADS) void k_merge(MergeArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ float levels[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wk = wave & 1;           // rows 32 wm .., columns 128 wk ..
  const int64_t n0 = (int64_t)blockIdx.y * TN, k0 = (int64_t)blockIdx.x * TK;
  const uint32_t K = (uint32_t)p.K, N = (uint32_t)p.N;
  const int r = p.r, RP = pad16(r), BP = bpitch(r);
  u16* sB = reinterpret_cast<u16*>(smem);                   // [TN][BP]
  u16* sA = sB + TN * BP;                                   // [RP][APITCH]
  float* stage = reinterpret_cast<float*>(smem);            // [64][SPITCH], after the MFMAs

  // ---- the base of this thread's output chunks, loaded first ----
  // half h (rows 64h .. 64h+63): chunk q = tid + 512 i (i < 4) is row q / 32,
  // columns 8 (q % 32) .. +8 of the tile
  uint32_t cw[2][4];          // merge: 8 codes per chunk
  uint32_t qb[2][4];          // merge: scale byte of the chunk's block
  float dg[2][4];             // merge: group constant
  u32x4v wv[2][4];            // unmerge: 8 bf16 per chunk
  {
    const auto rW = rsrc(UNMERGE ? (const void*)p.w_in : (const void*)p.codes,
                         UNMERGE ? N * K * 2u : N * K / 2u);
    const uint32_t nb = N * K / 64u;
    // fp32 scales: q reads 0 from an empty buffer and is OR-ed with E4M3(1.0)
    // below, d is the block's own scale
    const auto rQ = rsrc(p.qscale, UNMERGE || p.fp32_scale ? 0u : nb);
    const auto rD = rsrc(p.dscale, UNMERGE ? 0u : 4u * (p.fp32_scale ? nb : (nb + 255u) / 256u));
    const uint32_t dshift = p.fp32_scale ? 0u : 8u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHREADS * i;
        const uint32_t n = (uint32_t)n0 + 64u * h + (uint32_t)(q >> 5);
        const uint32_t k = (uint32_t)k0 + 8u * (uint32_t)(q & 31);
        const bool live = n < N && k < K;                  // rows and columns past the weight read nothing
        const uint32_t e = n * K + k;                      // the chunk's first element
        if constexpr (UNMERGE) {
          wv[h][i] = __builtin_amdgcn_raw_buffer_load_b128(rW, live ? 2u * e : 0x80000000u, 0, 0);
        } else {
          cw[h][i] = __builtin_amdgcn_raw_buffer_load_b32(rW, live ? e / 2u : 0x80000000u, 0, 0);
          const uint32_t blk = e / 64u;
          qb[h][i] = __builtin_amdgcn_raw_buffer_load_b8(rQ, live ? blk : 0x80000000u, 0, 0);
          dg[h][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rD, live ? 4u * (blk >> dshift) : 0x80000000u, 0, 0));
        }
      }
  }
  if (tid < 16) levels[tid] = p.lv[tid];

  // ---- stage B rows [n0, n0 + 128) x [0, RP) and A rows [0, RP) x [k0, k0 + 256) ----
  // (zeros past r, N and K: padded contraction terms then add exactly 0).
  // Every thread issues all its loads before its first store, so the staging
  // costs one memory round trip.
  {
    // B: thread t takes row t / 4, ranks 32 (t % 4) .. +32
    const auto rB = rsrc(p.B, N * (uint32_t)r * 2u);
    const int n = tid >> 2, j0 = 32 * (tid & 3);
    const bool row_live = n0 + n < p.N;
    if ((r & 7) == 0) {
      // rows of B are 16-byte aligned: four 16-byte loads
      u32x4v bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 8 * i;
        bv[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rB, row_live && j < r ? (uint32_t)((n0 + n) * r + j) * 2u : 0x80000000u, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j0 + 8 * i < RP) *reinterpret_cast<u32x4v*>(sB + n * BP + j0 + 8 * i) = bv[i];
    } else {
      uint32_t bv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int j = j0 + i;
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(
            rB, row_live && j < r ? (uint32_t)((n0 + n) * r + j) * 2u : 0x80000000u, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (j0 + i < RP) sB[n * BP + j0 + i] = (u16)bv[i];
    }
  }
  {
    // A: thread t takes columns 8 (t % 32) .. +8 of ranks t / 32 + 16 i
    const auto rA = rsrc(p.A, (uint32_t)r * K * 2u);
    const int c = tid & 31, jt = tid >> 5;
    const int64_t k = k0 + 8 * c;
    u32x4v av[QLN_MAX_RANK / 16];
#pragma unroll
    for (int i = 0; i < QLN_MAX_RANK / 16; ++i) {
      const int j = jt + 16 * i;
      av[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rA, j < r && k < p.K ? (uint32_t)(((int64_t)j * p.K + k) * 2) : 0x80000000u, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < QLN_MAX_RANK / 16; ++i) {
      const int j = jt + 16 * i;
      if (j < RP) *reinterpret_cast<u32x4v*>(sA + j * APITCH + 8 * c) = av[i];
    }
  }
  __syncthreads();

  // ---- the rank-r product: wave (wm, wk) computes rows 32 wm .., columns 128 wk .. ----
  f32x16_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;
  for (int ks = 0; ks < RP / 16; ++ks) {
    const bf16x8_t fa = *reinterpret_cast<const bf16x8_t*>(sB + (32 * wm + (lane & 31)) * BP + 16 * ks + 8 * (lane >> 5));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bf16x8_t fb = read_cols(sA, 128 * wk + 32 * b, ks, lane);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc[b], 0, 0, 0);
    }
  }

  // ---- add the base and store, 64 rows at a time through LDS ----
  // accumulator layout: lane l holds column l % 32 of each 32 x 32 block and
  // rows 8 (v / 4) + 4 (l / 32) + v % 4
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();   // the tiles (h = 0) or the previous half (h = 1) are no longer read
    if ((wm >> 1) == h) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = 32 * (wm & 1) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          stage[row * SPITCH + 128 * wk + 32 * b + (lane & 31)] = acc[b][v];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + NTHREADS * i;
      const int row = q >> 5, c8 = q & 31;
      const int64_t n = n0 + 64 * h + row, k = k0 + 8 * c8;
      if (n >= p.N || k >= p.K) continue;
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(stage + row * SPITCH + 8 * c8);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(stage + row * SPITCH + 8 * c8 + 4);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      float base[8];
      if constexpr (UNMERGE) {
        const u32x4v w = wv[h][i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          base[2 * e] = __uint_as_float(w[e] << 16);
          base[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      } else {
        // W' = bf16(L[code] * fl32(E4M3(q) * d)), element e in nibble e
        const float sb = (p.u8_scale ? (float)qb[h][i] : e4m3_decode((qb[h][i] | (p.fp32_scale ? 0x38u : 0u)) & 127u)) *
                         dg[h][i];
#pragma unroll
        for (int e = 0; e < 8; ++e) base[e] = bf16_to_f32(f32_to_bf16(levels[(cw[h][i] >> (4 * e)) & 15u] * sb));
      }
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(__builtin_fmaf(p.s, a[2 * e], base[2 * e]), __builtin_fmaf(p.s, a[2 * e + 1], base[2 * e + 1]));
      *reinterpret_cast<u32x4v*>(p.out + n * p.K + k) = u32x4v{o[0], o[1], o[2], o[3]};
    }
  }
}

template <bool UNMERGE>
static hipError_t launch(const MergeArgs& p, hipStream_t st) {
  const size_t lds = lds_bytes(p.r);
  const hipError_t attr =
      set_dynamic_lds(reinterpret_cast<const void*>(&k_merge<UNMERGE>), (int)lds_bytes(QLN_MAX_RANK));
  if (attr != hipSuccess) return attr;
  const dim3 grid((unsigned)((p.K + TK - 1) / TK), (unsigned)((p.N + TN - 1) / TN));
  hipLaunchKernelGGL((k_merge<UNMERGE>), grid, dim3(NTHREADS), lds, st, p);
  return hipGetLastError();
}

}  // namespace mrg

bool merge_fits(int64_t N, int64_t K, int r) {
  const int64_t lim = (int64_t)1 << 31;   // 32-bit buffer offsets
  return N * K * 2 < lim && (int64_t)r * K * 2 < lim && N * r * 2 < lim;
}

hipError_t launch_merge(const NF4View& w, const u16* A, const u16* B, int r, float s, u16* out,
                        hipStream_t st) {
  mrg::MergeArgs p{};
  p.codes = w.codes; p.qscale = w.qscale; p.dscale = w.dscale;
  p.fp32_scale = w.fp32_scale;
  p.u8_scale = w.u8_scale;
  for (int i = 0; i < 16; ++i) p.lv[i] = w.lv[i];
  p.N = w.N; p.K = w.K; p.A = A; p.B = B; p.r = r; p.s = s; p.out = out;
  return mrg::launch<false>(p, st);
}

hipError_t launch_unmerge(const u16* w_in, int64_t N, int64_t K, const u16* A, const u16* B, int r,
                          float s, u16* out, hipStream_t st) {
  mrg::MergeArgs p{};
  p.w_in = w_in; p.N = N; p.K = K; p.A = A; p.B = B; p.r = r; p.s = -s; p.out = out;
  return mrg::launch<true>(p, st);
}

}  // namespace qln
