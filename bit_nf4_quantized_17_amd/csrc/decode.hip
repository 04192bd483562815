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
// k_decode streams the weight: one workgroup of 8 waves per 16*TILES output
// columns (W rows) and per part of the contraction, the grid sized to about
// one workgroup per compute unit.  Each wave takes an eighth of its part
// (rotated by the workgroup index, so that the workgroups do not all stream
// the same column range of the weight at once) for all its tiles, so each X
// fragment it loads serves TILES weight tiles.  Cutting the contraction into
// parts lets a workgroup cover more columns when the layer has few: the
// parts other than the last store their fp32 sums in the workspace, and the
// last part of each column group adds them, in part order, to its own.  T =
// X A^T is computed as fixed split-K partial sums by the first workgroups of
// the same launch (or, when there are more of them than workgroups, by a
// separate k_tpart launch first; A is read once).
//
// Codes are read straight from HBM into registers, 16 bytes a lane: lane
// (i, g) of a 16-row tile loads bytes 16g..16g+15 of a pair of blocks of row
// i, so the lower half-wave holds the first block and the upper half the
// second; two v_permlane32_swap exchanges then leave every lane with 16 codes
// of each block, at contraction offset 32(g&1) + 16(g>>1) inside the block,
// and X is loaded with the same permutation, which leaves each block's sum
// unchanged.  Each wave issues the next batch's loads one tile at a time
// between the tiles of the current batch, so that the per-CU address unit
// works through them while the wave computes instead of stalling its issue.
//
// Set-up data goes straight to LDS with direct-to-LDS loads issued before
// the first two batches (loads complete in order, so waiting for the set-up
// does not wait for the batches): each wave stages the 8-bit scales of its
// own block pairs for every row of the workgroup and the (at most two)
// second-level constants those blocks use, and restores each pair's scales
// s = fl32(E4M3(q) * d) inside the loop with the hardware fp8 conversion;
// the last part also stages the LoRA factor B of its columns.  T (summed
// from the partials in a fixed order; the first column group also writes it
// to T_save) is read at the end.  The eight waves' results are summed in LDS
// in wave order, so results do not depend on timing.  Producers (T units,
// parts other than the last) publish each sum as one coherent 64-bit word
// tagged with a per-call epoch, which the consumer polls directly; they have
// lower workgroup indices than every consumer and never wait, so the waits
// always end.
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
constexpr int MAX_KPARTS = 4;           // contraction parts of the weight stream

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

struct DecArgs {
  const u16* X; int64_t M;          // X [M][K], M <= 16
  NF4View w;                        // W [N][K]
  const u16* A; const u16* B; int r; float s;
  // Partial sums handed between workgroups are tagged words: epoch << 32 |
  // fp32 bits, written and read with coherent 64-bit accesses, so a consumer
  // sees a value and its readiness in one load and no fence is needed.
  uint64_t* tpart; int nsplit;      // T partial sums [nsplit][16][r]
  uint32_t kchunk;                  // contraction elements per T split
  int tunits;                       // > 0: workgroups 0..tunits-1 also compute the T partials
  uint32_t epoch;                   // this call's tag (never 0)
  int kparts, gcols;                // contraction parts x column groups = the grid
  uint64_t* ypart;                  // parts 0..kparts-2: partial Y [part][M][N]
  u16* Y; float* T_save;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// s_waitcnt for the vector-memory counter only: at most n loads outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// A workgroup barrier after this thread's LDS writes have completed, with no
// wait for its vector-memory loads (a plain __syncthreads would also wait for
// the outstanding direct-to-LDS loads, which the barrier here does not need)
__device__ __forceinline__ void barrier_lds_only() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ void put_tagged(uint64_t* dst, float v, uint32_t epoch) {
  __hip_atomic_store(dst, ((uint64_t)epoch << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* src) {
  return __hip_atomic_load(const_cast<uint64_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A first read that may be served by this die's cache: words that many
// workgroups read (the T partials) then come from memory about once per
// cache.  A stale copy carries an older tag, and the retries of await_tagged
// read coherently.
__device__ __forceinline__ uint64_t get_tagged_cached(const uint64_t* src) {
  return __hip_atomic_load(const_cast<uint64_t*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until every word of w[0..n) carries `epoch`, re-reading the others
// after a short sleep; gives up (returns false) after about 0.4 s, so that a
// producer that never writes cannot hang the caller.
template <int CAP>
__device__ __forceinline__ bool await_tagged(uint64_t (&w)[CAP], const uint64_t* const (&src)[CAP], int n,
                                             uint32_t epoch) {
  for (int spins = 0;; ++spins) {
    bool ready = true;
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (i < n && (uint32_t)(w[i] >> 32) != epoch) ready = false;
    if (ready) return true;
    if (spins > (1 << 20)) return false;
    __builtin_amdgcn_s_sleep(4);
#pragma unroll
    for (int i = 0; i < CAP; ++i)
      if (i < n && (uint32_t)(w[i] >> 32) != epoch) w[i] = get_tagged(src[i]);
  }
}

// ---------------------------------------------------------------------------
// T partials: workgroup (q, s) sums X[m][k] A[16q + j][k] over k in split s
// (kchunk elements, a multiple of 64) into part[s][m][16q + j]; rows m >= M
// are zero and columns 16q + j >= r are skipped.  Four waves take 32-wide
// contraction steps in turn and are summed in LDS in wave order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * TP_WAVES) void k_tpart(const u16* X, int M, uint32_t K, const u16* A, int r,
                                                         uint32_t kchunk, uint64_t* part, uint32_t epoch) {
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
    if (j < r) put_tagged(part + ((size_t)blockIdx.y * 16 + m) * r + j, v, epoch);
  }
}

// ---------------------------------------------------------------------------
// the weight stream
// ---------------------------------------------------------------------------
// Byte offsets of the dynamic LDS regions.  The same function runs on the
// host (to size the launch) and on the device.  Regions that receive
// direct-to-LDS loads are laid out in whole load instructions (64 lanes x 16
// or 4 bytes), so that the zeros written by out-of-range lanes stay inside
// them.
struct Lds {
  uint32_t btab, ttab, tred, qst, dst, tstage, tails, red, total;
  uint32_t qb;                      // staged scale bytes per row and wave (a multiple of 16)
  uint32_t rows_q, rows_d;          // row pitch of the scale-byte and dscale stages
};
__host__ __device__ inline uint32_t align_up(uint32_t x, uint32_t a) { return (x + a - 1u) / a * a; }
// ppw: the most block pairs a wave of the workgroup covers
__host__ __device__ inline Lds lds_layout(int tiles, int ppw, int r) {
  Lds L;
  const uint32_t rows = 16u * (uint32_t)tiles;
  L.qb = align_up(2u * (uint32_t)(ppw > 0 ? ppw : 1), 16u);
  L.rows_q = align_up(rows, 64u);
  L.rows_d = align_up(rows, 32u);
  L.btab = 0;                                                    // B rows, bf16 [rows][r]
  L.ttab = align_up(L.btab + rows * (uint32_t)r * 2u, 1024u);    // T fp32 [16][r]
  L.tred = align_up(L.ttab + 16u * (uint32_t)r * 4u, 16u);       // a T unit's per-wave sums [8][256]
  // until the loop ends: per wave, the 8-bit scales of its block pairs for
  // every row ([qb / 16][rows_q][16 bytes]) and the two dscale values its
  // rows can touch ([rows_d][2] fp32); a T unit's staged operands [8][4][1 KB];
  // the last elements of B.  After the loop: the per-wave partial sums
  // [8][tiles][1 KB].
  L.qst = L.tred + (uint32_t)WAVES * 256u * 4u;
  L.dst = L.qst + (uint32_t)WAVES * L.qb * L.rows_q;
  L.tstage = L.dst + (uint32_t)WAVES * L.rows_d * 8u;
  L.tails = L.tstage + (uint32_t)WAVES * 4096u;                  // 64 dwords
  L.red = L.qst;
  const uint32_t end_s = L.tails + 256u;
  const uint32_t end_r = L.red + (uint32_t)(WAVES * tiles) * 1024u;
  L.total = end_s > end_r ? end_s : end_r;
  return L;
}

// The split of a part's block pairs over the waves: wave w takes pairs
// [wp0 + 2 floor(w h / 8), wp0 + 2 floor((w + 1) h / 8)) of the part's
// [wp0, wp1), h = ceil((wp1 - wp0) / 2), so that every wave starts on an
// even pair (its first scale byte is then 4-byte aligned).
__host__ __device__ inline int wave_pairs_max(int npp) { return 2 * (((npp + 1) / 2 + WAVES - 1) / WAVES); }

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
  // column group and contraction part; parts other than the last hand their
  // fp32 partial sums to the last, which finishes the output
  const int kp = (int)blockIdx.x / p.gcols;
  const uint32_t n0 = (uint32_t)((int)blockIdx.x % p.gcols) * (uint32_t)ROWS;
  const uint32_t rows_wg = min((uint32_t)ROWS, N - n0);
  const bool last = kp == p.kparts - 1;
  const int wp0 = kp * npair / p.kparts, wp1 = (kp + 1) * npair / p.kparts;   // this part's pairs
  const int r = p.r;
  const Lds L = lds_layout(TILES, wave_pairs_max(wp1 - wp0), r);

  const auto rX = rsrc(p.X, (uint32_t)p.M * K * 2u);
  const auto rC = rsrc(p.w.codes, N * RB);
  const uint32_t nb_all = N * (uint32_t)nbk;
  const auto rQ = rsrc(p.w.qscale, nb_all);
  const uint32_t ng = (nb_all + 255u) / 256u;
  const auto rD = rsrc(p.w.dscale, 4u * ng);
  const auto rB = rsrc(p.B, N * (uint32_t)r * 2u);

  // this wave's pairs of blocks (computed from the wave index as a scalar,
  // so that the compiler sees them uniform and selects load addresses
  // without branching), and the per-lane load offsets
  const int wsc = __builtin_amdgcn_readfirstlane(wave);
  const int wv = (wsc + (int)blockIdx.x) & (WAVES - 1);
  const int hp = (wp1 - wp0 + 1) / 2;
  const int p0 = wp0 + 2 * (wv * hp / WAVES), p1 = min(wp1, wp0 + 2 * ((wv + 1) * hp / WAVES));
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
        const uint32_t xo = (live & (kb < nbk)) ? xrow + 128u * (uint32_t)kb : OOB;   // no short circuit: no branch
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

  typedef __attribute__((address_space(3))) void* lds_ptr;

  // ---- the lookup table (no loads) ----
  {
    // word e holds the pair (byte & 15, byte >> 4) of byte e / 64: thread tid
    // writes bytes tid/64 + 8i, whose low nibble is tid/64 or tid/64 + 8
    // levels of the weight's codebook (kernel arguments, scalar loads)
    const float lo0 = p.w.lv[wsc];
    const float lo1 = p.w.lv[wsc + 8];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      lut[tid + NTHREADS * i] = pack_bf16x2((i & 1) ? lo1 : lo0, p.w.lv[i >> 1]);
  }
  float* ttab = reinterpret_cast<float*>(smem + L.ttab);

  // ---- set-up loads, issued before the first batches and written straight
  //      to LDS: loads complete in order, so that waiting for these does not
  //      wait for the batches, and no register is tied up by them ----
  // (a) a T unit's first two contraction steps: the partial T of rank tile tq
  //     over contraction split tsp; lane (i16, g) stages 16 bytes of X row i16
  //     and of A row 16 tq + i16, as its MFMA operands
  const bool tunit = (int)blockIdx.x < p.tunits;
  const int rq = (r + 15) / 16;
  const int tq = (int)blockIdx.x % rq, tsp = (int)blockIdx.x / rq;
  const uint32_t tk0 = (uint32_t)tsp * p.kchunk, tk1 = min(K, tk0 + p.kchunk);
  const auto rA = rsrc(p.A, (uint32_t)r * K * 2u);
  const uint32_t txrow = (uint32_t)i16 * K * 2u + 16u * (uint32_t)g;
  const uint32_t tarow = (uint32_t)(16 * tq + i16) * K * 2u + 16u * (uint32_t)g;
  uint8_t* tst = smem + L.tstage + 4096u * (uint32_t)wsc;   // [X0, A0, X1, A1] x 1 KB
  if (tunit) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t k = tk0 + 32u * (uint32_t)(wsc + WAVES * h);
      if (k < tk1) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_ptr)(tst + 2048u * h), 16, txrow + 2u * k, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)(tst + 2048u * h + 1024u), 16, tarow + 2u * k, 0, 0, 0);
      }
    }
  }
  // (b) the LoRA factor B of this workgroup's columns (the last part only), in
  //     16-byte chunks that lie wholly inside B; the few elements after the
  //     last such chunk (at the end of B only) come as one 2-byte load a lane,
  //     which the hardware writes as a dword to the tails area
  const uint32_t bsize = N * (uint32_t)r * 2u;
  const uint32_t bgoff = n0 * (uint32_t)r * 2u, blen = last ? rows_wg * (uint32_t)r * 2u : 0u;
  const uint32_t bnch = min((blen + 15u) / 16u, (bsize - bgoff) / 16u);
  for (uint32_t u = (uint32_t)wsc; 64u * u < bnch; u += WAVES) {
    const uint32_t i = 64u * u + (uint32_t)lane;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(smem + L.btab + 1024u * u), 16,
                                             i < bnch ? bgoff + 16u * i : OOB, 0, 0, 0);
  }
  const uint32_t btail = blen > 16u * bnch ? (blen - 16u * bnch) / 2u : 0u;   // bf16 elements, < 8
  if (wsc == 0 && btail > 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr)(smem + L.tails), 2,
                                             (uint32_t)lane < btail ? bgoff + 16u * bnch + 2u * (uint32_t)lane : OOB,
                                             0, 0, 0);
  // (c) this wave's own scales: the 8-bit scales of its pairs for every row of
  //     the workgroup (row R, chunk h of 16 bytes at [h][R]), and for every row
  //     the dscale of the group holding the wave's first block and of the next
  //     group (a wave covers at most 256 blocks, so at most two groups).  K is
  //     a multiple of 256 and the wave starts on an even pair, so every scale
  //     load is 4-byte aligned and a dword that holds a wanted byte lies
  //     wholly inside the array.
  uint8_t* qst = smem + L.qst + (uint32_t)wsc * L.qb * L.rows_q;
  const float* dst = reinterpret_cast<const float*>(smem + L.dst + (uint32_t)wsc * L.rows_d * 8u);
  for (uint32_t h = 0; 16u * h < L.qb; ++h) {
#pragma unroll
    for (int jr = 0; jr < (16 * TILES + 63) / 64; ++jr) {
      const uint32_t R = 64u * jr + (uint32_t)lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rQ, (lds_ptr)(qst + (h * L.rows_q + 64u * jr) * 16u), 16,
                                               R < rows_wg ? (n0 + R) * (uint32_t)nbk + 2u * (uint32_t)p0 + 16u * h
                                                           : OOB,
                                               0, 0, 0);
    }
  }
#pragma unroll
  for (int jr = 0; jr < (32 * TILES + 63) / 64; ++jr) {
    const uint32_t R = 32u * jr + (uint32_t)(lane >> 1);
    const uint32_t g0 = ((n0 + R) * (uint32_t)nbk + 2u * (uint32_t)p0) >> 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rD, (lds_ptr)(dst + 64 * jr), 4,
                                             R < rows_wg ? 4u * (g0 + (uint32_t)(lane & 1)) : OOB, 0, 0, 0);
  }

  // the first two batches go out now, so that the memory system has work
  // while the rest is set up
  Batch cur, nxt;
  __builtin_amdgcn_sched_barrier(0);   // keep every set-up load ahead of the batches
  load_batch(cur, p0);
  load_batch(nxt, p0 + NP);
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds_only();   // the lookup table is complete
  // the set-up loads are complete once no more than the two batches' loads
  // are outstanding
  wait_vm<2 * NP * (TILES + 4)>();

  // ---- a T unit: finish its partial T ----
  if (tunit) {
    f32x4_t tacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t k = tk0 + 32u * (uint32_t)(wsc + WAVES * h);
      if (k < tk1) {
        const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(tst + 2048u * h + 16u * (uint32_t)lane);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(tst + 2048u * h + 1024u + 16u * (uint32_t)lane);
        tacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, av, tacc, 0, 0, 0);
      }
    }
    // further steps (a split longer than 16 steps) load behind the batches
    if (tk1 - tk0 > 64u * WAVES) {
      for (uint32_t kk = tk0 + 32u * (uint32_t)(wave + 2 * WAVES); kk < tk1; kk += 32u * WAVES * 2) {
        const uint32_t ka = kk, kb = kk + 32u * WAVES;
        const bf16x8_t xa = ld16(rX, ka < tk1 ? txrow + 2u * ka : OOB), aa = ld16(rA, ka < tk1 ? tarow + 2u * ka : OOB);
        const bf16x8_t xb = ld16(rX, kb < tk1 ? txrow + 2u * kb : OOB), ab = ld16(rA, kb < tk1 ? tarow + 2u * kb : OOB);
        tacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, aa, tacc, 0, 0, 0);
        tacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, ab, tacc, 0, 0, 0);
      }
      wait_vm<0>();
    }
    float* tred = reinterpret_cast<float*>(smem + L.tred);
#pragma unroll
    for (int e = 0; e < 4; ++e) tred[wave * 256 + (4 * g + e) * 16 + i16] = tacc[e];   // (m, j) of the tile
    __syncthreads();
    if (tid < 256) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += tred[w * 256 + tid];
      const int m = tid >> 4, j = 16 * tq + (tid & 15);
      if (j < r) put_tagged(p.tpart + ((size_t)tsp * 16 + m) * r + j, v, p.epoch);
    }
  }
  // wave 0 moves the last elements of B it staged into place (read in the
  // epilogue, after barriers)
  {
    const uint32_t* tl = reinterpret_cast<const uint32_t*>(smem + L.tails);
    if ((uint32_t)tid < btail) reinterpret_cast<uint16_t*>(smem + L.btab)[8u * bnch + (uint32_t)tid] = (uint16_t)tl[tid];
  }

  // per tile, this lane's row: its two dscale values and the first block
  // (relative to the row) that lies in the second group
  float d0[TILES], d1[TILES];
  int kb_sw[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const uint32_t R = 16u * t + (uint32_t)i16;
    const f32x2v dd = *reinterpret_cast<const f32x2v*>(dst + 2 * R);
    d0[t] = dd.x;
    d1[t] = dd.y;
    const uint32_t rb = (n0 + R) * (uint32_t)nbk;
    kb_sw[t] = (int)(256u * (((rb + 2u * (uint32_t)p0) >> 8) + 1u) - rb);
  }

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
      const int prs = min(pr0 + u, p1 - 1);
      const int jb = 2 * (prs - p0);   // the pair's first scale byte in the wave's stage
      const uint32_t qoff = (uint32_t)((jb >> 4) * (int)L.rows_q * 16 + (jb & 15));
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        if constexpr (decltype(prefetch)::value) load_slot(nb, pr0 + NP, u, t);
        // lower half-wave loaded block 2pr, upper half block 2pr+1: exchange
        // halves so that words 0,1 hold block 2pr and words 2,3 block 2pr+1
        const auto s02 = __builtin_amdgcn_permlane32_swap(bt.c[u][t].x, bt.c[u][t].z, false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(bt.c[u][t].y, bt.c[u][t].w, false, false);
        const uint32_t w[4] = {s02[0], s13[0], s02[1], s13[1]};
        // restored scales s = fl32(E4M3(q) * d) of blocks 2 prs and 2 prs + 1 of this lane's row
        const uint32_t q2 = *reinterpret_cast<const uint16_t*>(qst + (16u * t + (uint32_t)i16) * 16u + qoff);
        const auto e2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q2, false);
        const f32x2v sc = {e2[0] * (2 * prs < kb_sw[t] ? d0[t] : d1[t]),
                           e2[1] * (2 * prs + 1 < kb_sw[t] ? d0[t] : d1[t])};
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
  // loads): both are in flight at the first step, which therefore loads
  // nothing; the tail issues no loads past this wave's last pair, since even
  // a load that returns zero costs address-unit time
  const std::integral_constant<bool, true> pf;
  const std::integral_constant<bool, false> nopf;
  int pr = p0;
  if (pr < p1) {
    step(cur, nxt, pr, nopf);
    pr += NP;
    for (; pr + 2 * NP < p1; pr += 2 * NP) {
      step(nxt, cur, pr, pf);
      step(cur, nxt, pr + NP, pf);
    }
    if (pr + NP < p1) {
      step(nxt, cur, pr, pf);
      step(cur, nxt, pr + NP, nopf);
    } else if (pr < p1) {
      step(nxt, cur, pr, nopf);
    }
  }

  // ---- cross-wave sums (fixed wave order), LoRA term, store ----
  __syncthreads();   // every wave is done with its stages
  float* red = reinterpret_cast<float*>(smem + L.red);
  // slot layout [wave][tile][m][16]; lane (col i16, rows 4g..4g+3)
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[((wave * TILES + t) * 16 + 4 * g + e) * 16 + i16] = acc[t][e];
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  constexpr int COLS = 16 * TILES;
  const int cg = (int)blockIdx.x % p.gcols;
  if (!last) {
    // a part that is not the last: its sums (fixed wave order) go to the
    // workspace with coherent stores, then its flag is raised
    uint64_t* yp = p.ypart + (size_t)kp * (size_t)p.M * N;
    for (int e = tid; e < (int)p.M * COLS; e += NTHREADS) {
      const int m = e / COLS, c = e - m * COLS;
      if ((uint32_t)c < rows_wg) {
        float base = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) base += red[((w * TILES + (c >> 4)) * 16 + m) * 16 + (c & 15)];
        put_tagged(yp + (size_t)m * N + n0 + c, base, p.epoch);
      }
    }
    return;
  }
  // The last part waits for T (the partials of workgroups 0..tunits-1,
  // written early in this kernel, or of the separate k_tpart launch) and for
  // the other parts of its columns.  Every workgroup it waits for has a lower
  // index and waits for nothing itself.  The wait is bounded: a producer that
  // never reports poisons this workgroup's output with NaN instead of hanging.
  // The other parts' sums of this thread's outputs, all loads in flight at once:
  constexpr int EPT = (16 * COLS + NTHREADS - 1) / NTHREADS;
  constexpr int NQ = EPT * (MAX_KPARTS - 1);
  uint64_t yq[NQ];
  const uint64_t* yq_src[NQ];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + i * NTHREADS, m = e / COLS, c = e - m * COLS;
    const bool ok = e < (int)p.M * COLS && (uint32_t)c < rows_wg;
#pragma unroll
    for (int q = 0; q < MAX_KPARTS - 1; ++q) {
      const bool live = ok && q < p.kparts - 1;
      yq_src[i * (MAX_KPARTS - 1) + q] = p.ypart + ((size_t)q * p.M + (live ? m : 0)) * N + n0 + (live ? c : 0);
      yq[i * (MAX_KPARTS - 1) + q] = live ? get_tagged(yq_src[i * (MAX_KPARTS - 1) + q]) : (uint64_t)p.epoch << 32;
    }
  }
  {
    // T = the partials summed in split order; rows m >= M are zero
    for (int e = tid; e < 16 * r; e += NTHREADS) {
      uint64_t pv[MAX_SPLIT];
      const uint64_t* src[MAX_SPLIT];
#pragma unroll
      for (int sp = 0; sp < MAX_SPLIT; ++sp) {
        src[sp] = p.tpart + (sp < p.nsplit ? sp : 0) * 16 * r + e;
        pv[sp] = sp < p.nsplit ? get_tagged_cached(src[sp]) : (uint64_t)p.epoch << 32;
      }
      if (!await_tagged(pv, src, p.nsplit, p.epoch)) s_bad = 1;
      float v = 0.0f;
#pragma unroll
      for (int sp = 0; sp < MAX_SPLIT; ++sp)
        if (sp < p.nsplit) v += __uint_as_float((uint32_t)pv[sp]);
      ttab[e] = v;
      if (cg == 0 && e < (int)p.M * r) p.T_save[e] = v;
    }
  }
  if (!await_tagged(yq, yq_src, NQ, p.epoch)) s_bad = 1;
  __syncthreads();
  const bool bad = s_bad != 0;
  const u16* btab = reinterpret_cast<const u16*>(smem + L.btab);
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + i * NTHREADS, m = e / COLS, c = e - m * COLS;
    if (e < (int)p.M * COLS && (uint32_t)c < rows_wg) {
      // the parts in order, then this one's waves in order
      float base = 0.0f;
#pragma unroll
      for (int q = 0; q < MAX_KPARTS - 1; ++q)
        if (q < p.kparts - 1) base += __uint_as_float((uint32_t)yq[i * (MAX_KPARTS - 1) + q]);
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
  const int npair = (nbk + 1) / 2;
  const Lds L = lds_layout(TILES, wave_pairs_max((npair + p.kparts - 1) / p.kparts), p.r);
  const hipError_t attr = set_dynamic_lds(reinterpret_cast<const void*>(&k_decode<TILES>), (int)MAX_DYN_LDS);
  if (attr != hipSuccess) return attr;
  const unsigned grid = (unsigned)(p.gcols * p.kparts);
  hipLaunchKernelGGL((k_decode<TILES>), dim3(grid), dim3(NTHREADS), L.total, st, p);
  return hipGetLastError();
}

// compute units of the current device (queried once per device; 256, the
// MI355X count, if the query fails)
static int device_cus() {
  constexpr int MAX_DEV = 64;
  static std::atomic<int> cus[MAX_DEV];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Shape of the weight stream: TILES 16-column tiles per workgroup and the
// contraction cut into kparts parts.  The address unit of a compute unit is
// what bounds the stream (a 16-byte load of codes or of X costs it the same
// time), so the plan minimises the wave loads of the most loaded compute
// unit: each pair of blocks costs one code load per tile plus four X loads,
// shared by all the workgroup's tiles.  A part must cover a multiple of 16
// blocks of every row, so that its scale segments are 16-byte aligned.
struct Plan {
  int tiles, kparts;
};
static bool part_ok(int64_t K, int kparts) { return kparts == 1 || (K / 64) % (16 * kparts) == 0; }
static Plan plan(int64_t N, int64_t K, int r) {
  const int64_t cus = device_cus(), nbk = K / 64, npair = (nbk + 1) / 2;
  Plan best{0, 0};
  int64_t best_cost = -1;
  for (int kp = 1; kp <= MAX_KPARTS; kp *= 2) {
    if (!part_ok(K, kp)) continue;
    for (int t = 1; t <= MAX_TILES; ++t) {
      const int ppw = wave_pairs_max((int)((npair + kp - 1) / kp));
      if (ppw > 128 || lds_layout(t, ppw, r).total > MAX_DYN_LDS) continue;   // a wave spans <= 2 groups
      const int64_t grid = (N + 16 * t - 1) / (16 * t) * kp;
      // (+ a fixed charge per extra part for the hand-over of its sums)
      const int64_t cost = (grid + cus - 1) / cus * ((npair + kp - 1) / kp) * (t + 4) + 64 * (kp - 1);
      if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = Plan{t, kp}; }
    }
  }
  return best;
}

// Per-call tags of the partial sums: a process-wide counter starting at a
// random value (so a workspace left over from another process is unlikely to
// hold a matching tag); 0 is skipped.
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

// workspace, in 64-bit tagged words: T partials [nsplit][16][r] | the parts'
// sums [MAX_KPARTS - 1][M][N] when K allows more than one part
static int64_t dec_ws_words(int64_t M, int64_t N, int64_t K, int r) {
  const dec::TSplit ts = dec::t_split(K);
  const int64_t extra = dec::part_ok(K, 2) ? dec::MAX_KPARTS - 1 : 0;
  return (int64_t)ts.nsplit * 16 * r + extra * M * N;
}

int64_t decode_workspace_elems(int64_t M, int64_t N, int64_t K, int r) { return 2 * dec_ws_words(M, N, K, r); }

bool decode_fits(int64_t M, const NF4View& w, int r) {
  const int64_t lim = (int64_t)1 << 31;
  if (!(M >= 1 && M <= 16 && w.N * w.K / 2 < lim && 16 * w.K * 2 < lim && (int64_t)r * w.K * 2 < lim &&
        w.N * r * 2 < lim && (dec::MAX_KPARTS - 1) * M * w.N < lim))
    return false;
  // K a multiple of 256 keeps every wave's scale loads 4-byte aligned; the
  // kernel stages 8-bit block scales, so fp32 scales take the tiled path
  return !w.fp32_scale && (w.K / 64) % 4 == 0 && dec::plan(w.N, w.K, r).tiles > 0;
}

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, float* ws, hipStream_t st) {
  const dec::TSplit ts = dec::t_split(w.K);
  const dec::Plan pl = dec::plan(w.N, w.K, r);
  const int64_t gcols = (w.N + 16 * pl.tiles - 1) / (16 * pl.tiles);
  const int units = ((r + 15) / 16) * ts.nsplit;
  dec::DecArgs p;
  p.X = X; p.M = M; p.w = w; p.A = A; p.B = B; p.r = r; p.s = s;
  uint64_t* words = reinterpret_cast<uint64_t*>(ws);   // 16-byte aligned (checked by the caller)
  p.tpart = words; p.nsplit = ts.nsplit; p.kchunk = ts.kchunk;
  p.kparts = pl.kparts; p.gcols = (int)gcols;
  p.ypart = words + (int64_t)ts.nsplit * 16 * r;
  p.Y = Y; p.T_save = T_save;
  // a fresh tag per call tells this call's partial sums from those a
  // previous call left in the workspace
  p.epoch = dec::next_epoch();
  if (units <= gcols * pl.kparts) {
    p.tunits = units;   // the first workgroups compute the T partials themselves
  } else {
    p.tunits = 0;
    hipLaunchKernelGGL(dec::k_tpart, dim3((unsigned)((r + 15) / 16), (unsigned)ts.nsplit),
                       dim3(64 * dec::TP_WAVES), 0, st, X, (int)M, (uint32_t)w.K, A, r, ts.kchunk, p.tpart, p.epoch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (pl.tiles) {
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
