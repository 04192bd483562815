// decode.hip -- the forward at decode sizes (M <= 16 tokens).  Ultralytics
// glossary "QLoRA", "How QLoRA works": the frozen layer dequantizes NF4 to
// bfloat16 for the matrix product and adds the LoRA path.
//
// At M <= 16 the layer is bound by streaming the packed weight (0.516 bytes
// per weight) from HBM, which leaves about three vector-ALU operations per
// weight at full bandwidth -- less than an exact per-element dequantization
// costs.  So this path factors the block scale out of the product:
//   Y[m][n] = sum_blocks s_b * ( sum_{k in block} X[m][k] * bf16(L[code]) )
//           + s_lora * sum_j T[m][j] B[n][j]
// bf16(L[code]) comes from an LDS table indexed by one code byte (two codes
// -> one bf16 pair), with one copy per lane so that lookups never share a
// bank; each 64-code block is one pair of v_mfma_f32_16x16x32_bf16 into a
// fresh accumulator, which is then scaled by the block's restored scale
// s_b = fl32(E4M3(q) * d) and added in fp32.  (The prefill and training
// kernels multiply the exactly dequantized bf16 weight instead; both round
// the weight's relative value once to bf16 precision.)
//
// Two kernels per call.  k_tpart computes T = X A^T as fixed split-K partial
// sums (a few dozen workgroups; A is read once).  k_decode streams the
// weight: one workgroup of 8 waves per 16*TILES output columns (W rows),
// sized so that the grid is about one workgroup per compute unit; each wave
// takes an eighth of the contraction (rotated by the workgroup index, so that
// the workgroups do not all stream the same column range of the weight at
// once) for all its tiles, so each X fragment it loads serves TILES weight
// tiles.  Codes are read straight from HBM into registers, 16 bytes a lane:
// lane (i, g) of a 16-row tile loads bytes 16g..16g+15 of a pair of blocks of
// row i, so the lower half-wave holds the first block and the upper half the
// second; two v_permlane32_swap exchanges then leave every lane with 16 codes
// of each block, at contraction offset 32(g&1) + 16(g>>1) inside the block,
// and X is loaded with the same permutation, which leaves each block's sum
// unchanged.  Each wave issues the next batch's loads one tile at a time
// between the tiles of the current batch, so that the per-CU address unit
// (about 16 bytes a clock, shared by the code and X loads) works through them
// while the wave computes instead of stalling its issue.
//
// The restored scales of all the workgroup's blocks, the LoRA factor B of its
// columns and T (summed from the partials in a fixed order; workgroup 0 also
// writes it to T_save) are put in LDS at the start, behind the first batch's
// loads.  The eight partial results are summed in LDS in wave order, so
// results do not depend on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <random>
#include <type_traits>

#include "common.h"
#include "device.h"

namespace qln {
namespace dec {

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int LUT_WORDS = 256 * 64;                   // one copy per lane, 64 KB (static LDS)
constexpr uint32_t MAX_DYN_LDS = 95u * 1024u;         // what is left of the 160 KB (1 KB for small statics)
constexpr int MAX_TILES = 8;
constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every range this path uses
constexpr int TP_WAVES = 4;             // waves of a k_tpart workgroup
constexpr int MAX_SPLIT = 16;           // T partials a decode workgroup sums

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

struct DecArgs {
  const u16* X; int64_t M;          // X [M][K], M <= 16
  NF4View w;                        // W [N][K]
  const u16* A; const u16* B; int r; float s;
  float* tpart; int nsplit;         // T partial sums [nsplit][16][r]
  uint32_t kchunk;                  // contraction elements per T split
  int tunits;                       // > 0: workgroups 0..tunits-1 also compute the T partials
  uint32_t* flags; uint32_t epoch;  // per T unit: set to epoch once its partials are written
  u16* Y; float* T_save;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------------------
// T partials: workgroup (q, s) sums X[m][k] A[16q + j][k] over k in split s
// (kchunk elements, a multiple of 64) into part[s][m][16q + j]; rows m >= M
// are zero and columns 16q + j >= r are skipped.  Four waves take 32-wide
// contraction steps in turn and are summed in LDS in wave order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * TP_WAVES) void k_tpart(const u16* X, int M, uint32_t K, const u16* A, int r,
                                                         uint32_t kchunk, float* part) {
  __shared__ float red[TP_WAVES][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i16 = lane & 15, g = lane >> 4;
  const int q = blockIdx.x;
  const uint32_t k0 = blockIdx.y * kchunk, k1 = min(K, k0 + kchunk);
  const auto rX = rsrc(X, (uint32_t)M * K * 2u);
  const auto rA = rsrc(A, (uint32_t)r * K * 2u);
  const uint32_t xrow = (uint32_t)i16 * K * 2u + 16u * (uint32_t)g;
  const uint32_t arow = (uint32_t)(16 * q + i16) * K * 2u + 16u * (uint32_t)g;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;   // steps in flight per wave
  for (uint32_t kk = k0 + 32u * wave; kk < k1; kk += 32u * TP_WAVES * U) {
    bf16x8_t xv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = kk + 32u * TP_WAVES * u;
      xv[u] = ld16(rX, k < k1 ? xrow + 2u * k : OOB);
      av[u] = ld16(rA, k < k1 ? arow + 2u * k : OOB);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[u], av[u], acc, 0, 0, 0);
  }
  // D layout: lane (col j = i16, rows 4g..4g+3)
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][(4 * g + e) * 16 + i16] = acc[e];
  __syncthreads();
  for (int e = threadIdx.x; e < 256; e += 64 * TP_WAVES) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < TP_WAVES; ++w) v += red[w][e];
    const int m = e >> 4, j = 16 * q + (e & 15);
    if (j < r) part[((size_t)blockIdx.y * 16 + m) * r + j] = v;
  }
}

// ---------------------------------------------------------------------------
// the weight stream
// ---------------------------------------------------------------------------
// Byte offsets of the dynamic LDS regions.  The same function runs on the
// host (to size the launch) and on the device.
struct Lds {
  uint32_t btab, ttab, tred, stab, red, total;
  uint32_t spitch;                  // floats per row of the scale table
};
__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }
__host__ __device__ inline Lds lds_layout(int tiles, int nbk, int r) {
  Lds L;
  const uint32_t rows = 16u * (uint32_t)tiles;
  // an even pitch of nbk + 2 or more keeps 8-byte reads aligned and puts the
  // 16 rows a wave reads at once in different banks
  L.spitch = ((uint32_t)nbk + 3u) & ~1u;
  L.btab = 0;                                               // B rows of this workgroup, bf16 [rows][r]
  L.ttab = align16(L.btab + rows * (uint32_t)r * 2u);       // T fp32 [16][r]
  L.tred = align16(L.ttab + 16u * (uint32_t)r * 4u);        // a T unit's per-wave sums [8][256]
  L.stab = L.tred + (uint32_t)WAVES * 256u * 4u;            // restored block scales fp32 [rows][spitch]
  L.red = L.stab;                                           // after the loop: per-wave partial sums
  const uint32_t end_s = L.stab + rows * L.spitch * 4u;
  const uint32_t end_r = L.red + (uint32_t)(WAVES * tiles) * 256u * 4u;
  L.total = end_s > end_r ? end_s : end_r;
  return L;
}

// Copy `len` bytes from buffer offset `goff` (16-byte aligned) to LDS `dst`
// (16-byte aligned): 16-byte loads, up to four per thread in flight before
// the stores, then single bytes for a tail under 16.
__device__ __forceinline__ void stage_bytes(uint8_t* dst, __amdgpu_buffer_rsrc_t src, uint32_t goff,
                                            uint32_t len, int tid) {
  const uint32_t nchunk = len >> 4;
  for (uint32_t base = (uint32_t)tid; base < nchunk; base += 4 * NTHREADS) {
    u32x4v v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = base + (uint32_t)(u * NTHREADS);
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(src, i < nchunk ? goff + 16u * i : OOB, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = base + (uint32_t)(u * NTHREADS);
      if (i < nchunk) *reinterpret_cast<u32x4v*>(dst + 16u * i) = v[u];
    }
  }
  const uint32_t tail = len & 15u;
  if ((uint32_t)tid < tail) {
    const uint32_t i = (nchunk << 4) + (uint32_t)tid;
    dst[i] = (uint8_t)__builtin_amdgcn_raw_buffer_load_b8(src, goff + i, 0, 0);
  }
}

// TILES: 16-column tiles per workgroup.  One batch = NP pairs of blocks.
template <int TILES>
__global__ __launch_bounds__(NTHREADS) void k_decode(DecArgs p) {
  constexpr int NP = TILES <= 3 ? 2 : 1;   // pairs per batch (two keep more bytes in flight)
  __shared__ __attribute__((aligned(16))) uint32_t lut[LUT_WORDS];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int ROWS = 16 * TILES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const uint32_t K = (uint32_t)p.w.K, RB = K / 2u;   // code bytes per row
  const int nbk = (int)(K / 64), npair = (nbk + 1) / 2;
  const uint32_t N = (uint32_t)p.w.N;
  const uint32_t n0 = blockIdx.x * (uint32_t)ROWS;
  const uint32_t rows_wg = min((uint32_t)ROWS, N - n0);
  const int r = p.r;
  const Lds L = lds_layout(TILES, nbk, r);

  const auto rX = rsrc(p.X, (uint32_t)p.M * K * 2u);
  const auto rC = rsrc(p.w.codes, N * RB);
  const uint32_t nb_all = N * (uint32_t)nbk;
  const auto rQ = rsrc(p.w.qscale, nb_all);
  const auto rD = rsrc(p.w.dscale, 4u * ((nb_all + 255u) / 256u));
  const auto rB = rsrc(p.B, N * (uint32_t)r * 2u);

  // this wave's pairs of blocks, and the per-lane load offsets
  const int wv = (wave + (int)blockIdx.x) & (WAVES - 1);
  const int p0 = wv * npair / WAVES, p1 = (wv + 1) * npair / WAVES;
  uint32_t crow[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) crow[t] = (n0 + 16u * t + (uint32_t)i16) * RB + 16u * (uint32_t)g;
  const uint32_t koff = 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1);   // after the swaps
  const uint32_t xrow = (uint32_t)i16 * K * 2u + 2u * koff;

  struct Batch {
    u32x4v c[NP][TILES];
    bf16x8_t x[NP][2][2];
  };
  // loads of one (pair u, tile t) slot of a batch; X rides with tile 0
  auto load_slot = [&](Batch& bt, int pr0, int u, int t) {
    const int pr = pr0 + u;
    const bool live = pr < p1;
    bt.c[u][t] = __builtin_amdgcn_raw_buffer_load_b128(rC, live ? crow[t] + 64u * (uint32_t)pr : OOB, 0, 0);
    if (t == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * pr + h;
        const uint32_t xo = live && kb < nbk ? xrow + 128u * (uint32_t)kb : OOB;
        bt.x[u][h][0] = ld16(rX, xo);     // rows >= M are past the buffer: zero
        bt.x[u][h][1] = ld16(rX, xo + 16u);
      }
    }
  };
  auto load_batch = [&](Batch& bt, int pr0) {
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
      for (int t = 0; t < TILES; ++t) load_slot(bt, pr0, u, t);
  };

  Batch cur, nxt;
  load_batch(cur, p0);

  // ---- a T unit: the partial T of rank tile q over contraction split sp ----
  if ((int)blockIdx.x < p.tunits) {
    const int rq = (r + 15) / 16;
    const int q = (int)blockIdx.x % rq, sp = (int)blockIdx.x / rq;
    const uint32_t k0 = (uint32_t)sp * p.kchunk, k1 = min(K, k0 + p.kchunk);
    const auto rA = rsrc(p.A, (uint32_t)r * K * 2u);
    const uint32_t txrow = (uint32_t)i16 * K * 2u + 16u * (uint32_t)g;
    const uint32_t tarow = (uint32_t)(16 * q + i16) * K * 2u + 16u * (uint32_t)g;
    f32x4_t tacc = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t kk = k0 + 32u * wave; kk < k1; kk += 32u * WAVES * 2) {
      const uint32_t ka = kk, kb = kk + 32u * WAVES;
      const bf16x8_t xa = ld16(rX, ka < k1 ? txrow + 2u * ka : OOB), aa = ld16(rA, ka < k1 ? tarow + 2u * ka : OOB);
      const bf16x8_t xb = ld16(rX, kb < k1 ? txrow + 2u * kb : OOB), ab = ld16(rA, kb < k1 ? tarow + 2u * kb : OOB);
      tacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, aa, tacc, 0, 0, 0);
      tacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, ab, tacc, 0, 0, 0);
    }
    float* tred = reinterpret_cast<float*>(smem + L.tred);
#pragma unroll
    for (int e = 0; e < 4; ++e) tred[wave * 256 + (4 * g + e) * 16 + i16] = tacc[e];   // (m, j) of the tile
    __syncthreads();
    if (tid < 256) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += tred[w * 256 + tid];
      const int m = tid >> 4, j = 16 * q + (tid & 15);
      // coherent (device-scope) stores: no cache-wide writeback needed
      if (j < r) __hip_atomic_store(p.tpart + ((size_t)sp * 16 + m) * r + j, v, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(p.flags + blockIdx.x, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- tables (their loads queue behind the first batch) ----
  {
    // word e holds the pair (byte & 15, byte >> 4) of byte e / 64: thread tid
    // writes bytes tid/64 + 8i, whose low nibble is tid/64 or tid/64 + 8
    const float lo0 = __uint_as_float(kNF4LevelBits[tid >> 6]);
    const float lo1 = __uint_as_float(kNF4LevelBits[(tid >> 6) + 8]);
#pragma unroll
    for (int i = 0; i < 32; ++i)
      lut[tid + NTHREADS * i] = pack_bf16x2((i & 1) ? lo1 : lo0, __uint_as_float(kNF4LevelBits[i >> 1]));
  }
  float* stab = reinterpret_cast<float*>(smem + L.stab);
  // the scale table's padding (columns past nbk, rows past this workgroup's
  // last row) is read by dead pairs and must be finite
  for (int lr = tid; lr < ROWS; lr += NTHREADS)
    for (uint32_t b = (uint32_t)nbk; b < L.spitch; ++b) stab[lr * L.spitch + b] = 0.0f;
  for (uint32_t e = (uint32_t)tid; e < ((uint32_t)ROWS - rows_wg) * L.spitch; e += NTHREADS)
    stab[rows_wg * L.spitch + e] = 0.0f;
  stage_bytes(smem + L.btab, rB, n0 * (uint32_t)r * 2u, rows_wg * (uint32_t)r * 2u, tid);
  float* ttab = reinterpret_cast<float*>(smem + L.ttab);
  {
    // restored scales of this workgroup's blocks [q0, q0 + len): 16 per step
    const uint32_t q0 = n0 * (uint32_t)nbk, len = rows_wg * (uint32_t)nbk;
    auto fill = [&](uint32_t c, const u32x4v& v, float da, float db, uint32_t ga) {
      const uint32_t f0 = 16u * c;
      uint32_t lr = f0 / (uint32_t)nbk, b = f0 - lr * (uint32_t)nbk;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (f0 + k < len) {
          const float d = ((q0 + f0 + k) >> 8) == ga ? da : db;
          stab[lr * L.spitch + b] = e4m3_decode((v[k >> 2] >> (8 * (k & 3))) & 127u) * d;
        }
        if (++b == (uint32_t)nbk) { b = 0; ++lr; }
      }
    };
    // 16 scale bytes per chunk; a chunk that runs past the workgroup's blocks
    // is read byte by byte (the qscale array may end there)
    auto load_q = [&](uint32_t c) -> u32x4v {
      const uint32_t f0 = 16u * c;
      if (f0 + 16u <= len) return __builtin_amdgcn_raw_buffer_load_b128(rQ, q0 + f0, 0, 0);
      u32x4v v = {0u, 0u, 0u, 0u};
      for (uint32_t k = 0; f0 + k < len; ++k)
        v[k >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rQ, q0 + f0 + k, 0, 0) << (8 * (k & 3));
      return v;
    };
    auto load_d = [&](uint32_t gi) -> float {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, 4u * gi, 0, 0));
    };
    const uint32_t nch = (len + 15u) / 16u;
    for (uint32_t c0 = (uint32_t)tid; c0 < nch; c0 += 2 * NTHREADS) {
      const uint32_t c1 = c0 + NTHREADS;
      const bool two = c1 < nch;
      const u32x4v v0 = load_q(c0);
      const u32x4v v1 = two ? load_q(c1) : u32x4v{0u, 0u, 0u, 0u};
      const uint32_t ga0 = (q0 + 16u * c0) >> 8, gb0 = (q0 + min(16u * c0 + 15u, len - 1u)) >> 8;
      const uint32_t ga1 = (q0 + 16u * c1) >> 8, gb1 = (q0 + min(16u * c1 + 15u, len - 1u)) >> 8;
      const float da0 = load_d(ga0), db0 = load_d(gb0);
      const float da1 = load_d(two ? ga1 : ga0), db1 = load_d(two ? gb1 : gb0);
      fill(c0, v0, da0, db0, ga0);
      if (two) fill(c1, v1, da1, db1, ga1);
    }
  }
  __syncthreads();

  // LDS address of (code byte e of word c, this lane's copy) = byte << 8 | lane * 4,
  // assembled by one byte permute
  const uint32_t lane4 = (uint32_t)lane * 4u;
  auto lookup = [&](uint32_t c, int e) -> uint32_t {
    const uint32_t addr = __builtin_amdgcn_perm(c, lane4, 0x0C0C0400u + ((uint32_t)e << 8));
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lut) + addr);
  };

  f32x4_t acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // multiply batch `bt` (pairs pr0..pr0+NP-1) while the next batch's loads
  // are issued one slot at a time between the tiles, so that the address
  // unit works through them while this wave computes
  auto step = [&](const Batch& bt, Batch& nb, int pr0, auto prefetch) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      // a pair past the row's end (the last batch of a wave may hold one) has
      // zero X; any finite scale then adds nothing
      const int prs = min(pr0 + u, npair - 1);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        if constexpr (decltype(prefetch)::value) load_slot(nb, pr0 + NP, u, t);
        // lower half-wave loaded block 2pr, upper half block 2pr+1: exchange
        // halves so that words 0,1 hold block 2pr and words 2,3 block 2pr+1
        const auto s02 = __builtin_amdgcn_permlane32_swap(bt.c[u][t].x, bt.c[u][t].z, false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(bt.c[u][t].y, bt.c[u][t].w, false, false);
        const uint32_t w[4] = {s02[0], s13[0], s02[1], s13[1]};
        const f32x2v sc = *reinterpret_cast<const f32x2v*>(stab + (16 * t + i16) * L.spitch + 2 * prs);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4v wa = {lookup(w[2 * h], 0), lookup(w[2 * h], 1), lookup(w[2 * h], 2), lookup(w[2 * h], 3)};
          const u32x4v wb = {lookup(w[2 * h + 1], 0), lookup(w[2 * h + 1], 1), lookup(w[2 * h + 1], 2),
                             lookup(w[2 * h + 1], 3)};
          f32x4_t tmp = f32x4_t{0.f, 0.f, 0.f, 0.f};
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt.x[u][h][0], __builtin_bit_cast(bf16x8_t, wa), tmp, 0, 0, 0);
          tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bt.x[u][h][1], __builtin_bit_cast(bf16x8_t, wb), tmp, 0, 0, 0);
          const float s = h ? sc.y : sc.x;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][e] += s * tmp[e];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // two batches ping-pong (no register copies, which would wait for the
  // loads); the tail issues no loads past this wave's last pair, since even a
  // load that returns zero costs address-unit time
  const std::integral_constant<bool, true> pf;
  const std::integral_constant<bool, false> nopf;
  int pr = p0;
  for (; pr + 2 * NP < p1; pr += 2 * NP) {
    step(cur, nxt, pr, pf);
    step(nxt, cur, pr + NP, pf);
  }
  if (pr + NP < p1) {
    step(cur, nxt, pr, pf);
    step(nxt, cur, pr + NP, nopf);
  } else if (pr < p1) {
    step(cur, nxt, pr, nopf);
  }

  // ---- cross-wave sums (fixed wave order), LoRA term, store ----
  __syncthreads();   // every wave is done with the scale table
  float* red = reinterpret_cast<float*>(smem + L.red);
  // slot layout [wave][tile][m][16]; lane (col i16, rows 4g..4g+3)
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * TILES + t) * 16 + 4 * g + e) * 16 + i16] = acc[t][e];
  // T: the partials of workgroups 0..tunits-1 (written early in this kernel;
  // by now long done -- they wait for nothing before publishing) or of the
  // separate k_tpart launch.  The wait is bounded: a unit that never reports
  // poisons this workgroup's output with NaN instead of hanging.
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (p.tunits > 0) {
    // coherent loads of the flags (no cache invalidation per poll); the
    // partials are then read with coherent loads too, issued only after the
    // barrier that follows every flag being seen
    for (int u = tid; u < p.tunits; u += NTHREADS) {
      int spins = 0;
      while (__hip_atomic_load(p.flags + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch) {
        __builtin_amdgcn_s_sleep(4);
        if (++spins > (1 << 22)) { s_bad = 1; break; }
      }
    }
    __syncthreads();
  }
  {
    // T = the partials summed in split order (all loads of an element in
    // flight at once); rows m >= M are zero
    for (int e = tid; e < 16 * r; e += NTHREADS) {
      float pv[MAX_SPLIT];
#pragma unroll
      for (int sp = 0; sp < MAX_SPLIT; ++sp)
        pv[sp] = sp < p.nsplit ? __hip_atomic_load(p.tpart + sp * 16 * r + e, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0.0f;
      float v = 0.0f;
#pragma unroll
      for (int sp = 0; sp < MAX_SPLIT; ++sp)
        if (sp < p.nsplit) v += pv[sp];
      ttab[e] = v;
      if (blockIdx.x == 0 && e < (int)p.M * r) p.T_save[e] = v;
    }
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  const u16* btab = reinterpret_cast<const u16*>(smem + L.btab);
  constexpr int COLS = 16 * TILES;
  for (int e = tid; e < (int)p.M * COLS; e += NTHREADS) {
    const int m = e / COLS, c = e - m * COLS;
    if ((uint32_t)c < rows_wg) {
      float base = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) base += red[((w * TILES + (c >> 4)) * 16 + m) * 16 + (c & 15)];
      float lora = 0.0f;
      if ((r & 7) == 0) {      // 8 terms per step from 16-byte LDS reads, in j order
        const f32x4_t* tv = reinterpret_cast<const f32x4_t*>(ttab + m * r);
        const u32x4v* bv = reinterpret_cast<const u32x4v*>(btab + c * r);
#pragma unroll 2
        for (int j8 = 0; j8 < r / 8; ++j8) {
          const f32x4_t t0 = tv[2 * j8], t1 = tv[2 * j8 + 1];
          const u32x4v b = bv[j8];
          const float bw[8] = {__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                               __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u),
                               __uint_as_float(b.z << 16), __uint_as_float(b.z & 0xFFFF0000u),
                               __uint_as_float(b.w << 16), __uint_as_float(b.w & 0xFFFF0000u)};
#pragma unroll
          for (int k = 0; k < 4; ++k) lora += t0[k] * bw[k];
#pragma unroll
          for (int k = 0; k < 4; ++k) lora += t1[k] * bw[4 + k];
        }
      } else {
        for (int j = 0; j < r; ++j) lora += ttab[m * r + j] * bf16_to_f32(btab[c * r + j]);
      }
      p.Y[(size_t)m * N + n0 + c] = bad ? (u16)0x7FC0u : f32_to_bf16(base + p.s * lora);
    }
  }
}

template <int TILES>
static hipError_t launch_one(const DecArgs& p, hipStream_t st) {
  const int nbk = (int)(p.w.K / 64);
  const Lds L = lds_layout(TILES, nbk, p.r);
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<TILES>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)MAX_DYN_LDS);
  });
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)((p.w.N + 16 * TILES - 1) / (16 * TILES));
  hipLaunchKernelGGL((k_decode<TILES>), dim3(grid), dim3(NTHREADS), L.total, st, p);
  return hipGetLastError();
}

static int device_cus() {
  static int cus = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  });
  return cus;
}

// tiles per workgroup: the fewest that keep the grid within one workgroup per
// compute unit (more tiles per workgroup share each X fragment more widely)
static int pick_tiles(int64_t N, int64_t K, int r) {
  const int64_t tiles = (N + 15) / 16;
  const int64_t cus = device_cus();
  int t = (int)std::min<int64_t>(MAX_TILES, std::max<int64_t>(1, (tiles + cus - 1) / cus));
  while (t > 1 && lds_layout(t, (int)(K / 64), r).total > MAX_DYN_LDS) --t;
  return t;
}

// Per-call epochs for the T-unit flags: a process-wide counter starting at a
// random value (so a workspace left over from another process is unlikely to
// hold a matching flag); 0 is skipped.
static uint32_t next_epoch() {
  static std::atomic<uint32_t> counter{0};
  static std::once_flag once;
  std::call_once(once, [] { counter.store(std::random_device{}()); });
  uint32_t e = counter.fetch_add(1) + 1;
  if (e == 0) e = counter.fetch_add(1) + 1;
  return e;
}

// Split of the contraction for the T partials: chunks of at least 512 (a
// multiple of 64), at most MAX_SPLIT of them.
struct TSplit {
  int nsplit;
  uint32_t kchunk;
};
static TSplit t_split(int64_t K) {
  int64_t chunk = std::max<int64_t>(512, (K + MAX_SPLIT - 1) / MAX_SPLIT);
  chunk = (chunk + 63) / 64 * 64;
  TSplit s;
  s.kchunk = (uint32_t)chunk;
  s.nsplit = (int)((K + chunk - 1) / chunk);
  return s;
}

}  // namespace dec

// workspace: T partials [nsplit][16][r] fp32, then one 32-bit flag per T unit
int64_t decode_workspace_elems(int64_t K, int r) {
  const dec::TSplit ts = dec::t_split(K);
  return (int64_t)ts.nsplit * 16 * r + (int64_t)ts.nsplit * ((r + 15) / 16) + 64;
}

bool decode_fits(int64_t M, const NF4View& w, int r) {
  const int64_t lim = (int64_t)1 << 31;
  if (!(M >= 1 && M <= 16 && w.N * w.K / 2 < lim && 16 * w.K * 2 < lim && (int64_t)r * w.K * 2 < lim &&
        w.N * r * 2 < lim))
    return false;
  return dec::lds_layout(1, (int)(w.K / 64), r).total <= dec::MAX_DYN_LDS;
}

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, float* ws, hipStream_t st) {
  const dec::TSplit ts = dec::t_split(w.K);
  const int tiles = dec::pick_tiles(w.N, w.K, r);
  const int64_t grid = (w.N + 16 * tiles - 1) / (16 * tiles);
  const int units = ((r + 15) / 16) * ts.nsplit;
  dec::DecArgs p;
  p.X = X; p.M = M; p.w = w; p.A = A; p.B = B; p.r = r; p.s = s;
  p.tpart = ws; p.nsplit = ts.nsplit; p.kchunk = ts.kchunk;
  p.flags = reinterpret_cast<uint32_t*>(ws + (int64_t)ts.nsplit * 16 * r);
  p.Y = Y; p.T_save = T_save;
  if (units <= grid) {
    // the first workgroups compute the T partials themselves; a fresh epoch
    // per call tells their flags from those a previous call left behind
    p.tunits = units;
    p.epoch = dec::next_epoch();
  } else {
    p.tunits = 0;
    p.epoch = 0;
    hipLaunchKernelGGL(dec::k_tpart, dim3((unsigned)((r + 15) / 16), (unsigned)ts.nsplit),
                       dim3(64 * dec::TP_WAVES), 0, st, X, (int)M, (uint32_t)w.K, A, r, ts.kchunk, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (tiles) {
    case 1: return dec::launch_one<1>(p, st);
    case 2: return dec::launch_one<2>(p, st);
    case 3: return dec::launch_one<3>(p, st);
    case 4: return dec::launch_one<4>(p, st);
    case 5: return dec::launch_one<5>(p, st);
    case 6: return dec::launch_one<6>(p, st);
    case 7: return dec::launch_one<7>(p, st);
    default: return dec::launch_one<8>(p, st);
  }
}

}  // namespace qln
