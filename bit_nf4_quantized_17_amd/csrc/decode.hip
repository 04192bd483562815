// decode.hip -- the forward at decode sizes (M <= 16 tokens).  Ultralytics
// glossary "QLoRA", "How QLoRA works": the frozen layer dequantizes NF4 to
// bfloat16 for the matrix product and adds the LoRA path.
//
// At M <= 16 the layer is bound by streaming the packed weight (0.516 bytes
// per weight) from HBM, which leaves about three vector-ALU operations per
// weight at full bandwidth -- less than an exact per-element dequantization
// costs.  So this path factors the block scale out of the product:
//   Y[m][n] = sum_blocks s_b * ( sum_{k in block} X[m][k] * bf16(L[code]) )
//           + s_lora * sum_j T[m][j] B[n][j],      T = X A^T (fp32)
// bf16(L[code]) comes from an LDS table indexed by one code byte (two codes
// -> one bf16 pair), with one copy per lane so that lookups never share a
// bank; each 64-code block is one pair of v_mfma_f32_16x16x32_bf16 into a
// fresh accumulator, which is then scaled by the block's restored scale
// s_b = fl32(v(q) * d) (v: the E4M3 value of the scale byte, or the byte
// as an integer for uint8-linear scales) and added in fp32.  (The prefill and training
// kernels multiply the exactly dequantized bf16 weight instead; both round
// the weight's relative value once to bf16 precision.)
//
// Two launches.  The first sums T = X A^T over S slices of the contraction
// (S x RT small workgroups, fp32 partials in the workspace).  The second
// streams the weight with no communication between workgroups: a workgroup
// owns 16 * TR consecutive output columns (W rows, TR <= 7) over the whole
// contraction, so it finishes its outputs itself; it adds up the S partials
// of T in a fixed order for its LoRA term.  Its grid is about one workgroup
// per compute unit.  The 8-bit block scales of its rows are one contiguous
// run of bytes, which it copies to LDS at the start.
//
// The eight waves split the contraction into chunks of 128 (two blocks, 64
// code bytes of a row), wave w taking every eighth chunk from chunk w, and
// run independently until the final sums: no LDS staging and no barrier in
// the stream.  Per chunk and
// 16-row tile a wave loads the codes straight into registers -- lane
// (n = lane % 16, g = lane / 16) takes bytes [16 g, 16 g + 16) of row n --
// and one v_permlane32_swap per register pair moves them so that registers
// x, y of every lane hold block 0 of the chunk and z, w block 1 (the swap
// exchanges the upper lanes of one register with the lower lanes of the
// other).  Each register then feeds one MFMA whose 32 contraction slots all
// lie in one block; the X fragments are loaded in the same contraction
// order (lane group g, register v: chunk offset 64 [v in z, w] + 8 [v in y,
// w] + 32 (g & 1) + 16 (g >> 1)).  Loads run D chunks ahead in a register
// ring.  Since the waves run at the same pace, the two halves of each
// 128-byte line reach L2 close together and the line is fetched from HBM
// once (measured: a wave that read both halves itself, one chunk apart,
// fetched 1.7 times the weight's bytes).  The workgroups start at different
// groups of chunks (if every workgroup read the same column window of its
// rows at the same time, the requests would pile onto a few memory
// channels).  The
// eight waves' sums are added in LDS in wave order, so results do not depend
// on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "device.h"

namespace qln {
namespace dec {

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int LUT_WORDS = 256 * 64;     // 256 byte values x 64 lanes, 64 KB (static LDS)
constexpr int CHUNK = 128;              // contraction elements per chunk (two blocks)
constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every range this path uses
constexpr int MAX_R = 32;               // ranks the fused T handles (two 16-rank tiles)
constexpr int MAX_TR = 7;               // 16-row tiles per workgroup
constexpr int MAX_DYN_LDS = 94 * 1024;  // dynamic LDS limit set on the kernels (they use <= 65 KB)
constexpr int MAX_S = 16;               // slices of the T partials

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

struct DecArgs {
  const u16* X; int M;                      // X [M][K], M <= 16
  const uint8_t* codes; const uint8_t* qscale; const float* dscale;
  uint32_t N, K;
  float lv[16];                             // the codebook's levels
  const float* tpart; int S, RT;            // T partials [S][16][16 RT]
  const u16* B; int r; float s;
  u16* Y; float* T_save;
};

// Slices of the contraction for the T partials: up to MAX_S, each a
// multiple of 128 (four waves x 32) and at least 512 long.
static inline int t_slices(uint32_t K) {
  for (int s = MAX_S; s > 1; s /= 2)
    if (K % (128u * (uint32_t)s) == 0 && K / (uint32_t)s >= 512u) return s;
  return 1;
}

// T partials: workgroup (s, rt) sums X[m][k] A[16 rt + j][k] over k in slice
// s, its four waves taking a quarter each (32 per MFMA, lane (i, g) holding
// X[i][k0 + 8 g ..] and A[16 rt + i][k0 + 8 g ..]); the waves' sums are added
// in LDS in wave order and stored as part[s][m][16 rt + j] (rows m >= M and
// ranks j >= r read as zero).
__global__ __launch_bounds__(256) void k_decode_t(const u16* X, int M, const u16* A, int r, uint32_t K,
                                                  int S, int RT, float* part) {
  __shared__ float red[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int s = blockIdx.x, rt = blockIdx.y;
  const uint32_t len = K / (uint32_t)S / 4u;
  const uint32_t k0 = (uint32_t)s * (K / (uint32_t)S) + (uint32_t)wave * len + 8u * (uint32_t)g;
  const auto rX = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(X), (short)0, (int)((uint32_t)M * K * 2u), 0x00020000);
  const auto rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(A), (short)0, (int)((uint32_t)r * K * 2u), 0x00020000);
  const uint32_t xo = i16 < M ? (uint32_t)i16 * K * 2u + 2u * k0 : 0x80000000u;
  const uint32_t ao = 16 * rt + i16 < r ? (uint32_t)(16 * rt + i16) * K * 2u + 2u * k0 : 0x80000000u;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // eight steps of 32 in flight at a time (a slice is at least 128 a wave)
  for (uint32_t k = 0; k < len; k += 256u) {
    bf16x8_t xv[8], av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t kk = k + 32u * (uint32_t)u;
      xv[u] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rX, kk < len ? xo + 2u * kk : 0x80000000u, 0, 0));
      av[u] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rA, kk < len ? ao + 2u * kk : 0x80000000u, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[u], av[u], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[wave][(4 * g + e) * 16 + i16] = acc[e];
  __syncthreads();
  const int t = threadIdx.x, m = t >> 4, j = t & 15;
  const float v = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
  part[((size_t)s * 16 + (size_t)m) * (size_t)(16 * RT) + (size_t)(16 * rt + j)] = v;
}

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

// One wave's register loads of one chunk: per tile the codes of the lane's
// row, and the X fragments of the chunk's four MFMAs (shared by every tile).
template <int TR>
struct Chunk {
  u32x4v c[TR];           // row n0 + 16 t + lane % 16, code bytes [16 g, 16 g + 16) of the chunk
  bf16x8_t x[4];          // X[m = lane % 16][chunk offset of register v .. + 8], v = x, y, z, w
};

// Loads per chunk per wave, and D, the chunks loaded ahead: as deep as the
// register ring allows (at most 160 of the 256 registers a wave of a
// 512-lane workgroup may hold), at most 4, and within the 6-bit load
// counter.
template <int TR>
constexpr int lpc_of() { return TR + 4; }
template <int TR>
constexpr int depth_of() {
  constexpr int slot = 4 * TR + 16;          // registers of one ring slot
  int d = 160 / slot - 1;                    // the ring takes at most 160
  d = d < 1 ? 1 : d > 4 ? 4 : d;
  return d * lpc_of<TR>() > 60 ? 60 / lpc_of<TR>() : d;
}

template <int TR, bool U8>
__global__ __launch_bounds__(NTHREADS) void k_decode(DecArgs p) {
  constexpr int D = depth_of<TR>();
  constexpr int NS = D + 1;
  constexpr int LPC = lpc_of<TR>();
  __shared__ __attribute__((aligned(16))) uint32_t lut[LUT_WORDS];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const uint32_t K = p.K, N = p.N, RB = K / 2u, nbk = K / 64u;
  const uint32_t n0 = (uint32_t)blockIdx.x * 16u * (uint32_t)TR;

  // the row's C chunks form G groups of eight; at iteration i wave w takes
  // chunk w of group (i + rot) mod G, so the eight waves read the two
  // halves of each 128-byte line of their rows at about the same time (a
  // chunk number past C, in a ragged last group, is skipped)
  const int C = (int)(K / CHUNK);
  const int G = (C + WAVES - 1) / WAVES;
  const int rot = (int)(blockIdx.x % (uint32_t)G);
  auto chunk_of = [&](int i) { const int j = i + rot; return WAVES * (j >= G ? j - G : j) + wave; };

  const auto rC = rsrc(p.codes, N * RB);
  const auto rQ = rsrc(p.qscale, N * nbk);
  const auto rX = rsrc(p.X, (uint32_t)p.M * K * 2u);

  // this lane's code offset at chunk 0 of tile 0 (tile t adds 16 t rows;
  // rows past N fall past the buffer's range and read zeros)
  const uint32_t coff = (n0 + (uint32_t)i16) * RB + 16u * (uint32_t)g;
  const uint32_t qoff = (n0 + (uint32_t)i16) * nbk;   // the row's first scale byte
  // contraction offset of lane group g within a chunk's register x
  const uint32_t kg = 32u * (uint32_t)(g & 1) + 16u * (uint32_t)(g >> 1);
  const uint32_t xoff = i16 < p.M ? (uint32_t)i16 * K * 2u + 2u * kg : OOB;

  // ---- the workgroup's block scales, 16 TR nbk contiguous bytes from
  //      n0 nbk (at most 28 KB), 16 bytes a thread and pass; rows past N
  //      read zeros ----
  constexpr int QPASS = (16 * MAX_TR * 256 + 16 * NTHREADS - 1) / (16 * NTHREADS);
  const uint32_t qbytes = 16u * (uint32_t)TR * nbk;
  u32x4v qv[QPASS];
#pragma unroll
  for (int i = 0; i < QPASS; ++i) {
    const uint32_t o = 16u * (uint32_t)(tid + NTHREADS * i);
    qv[i] = __builtin_amdgcn_raw_buffer_load_b128(rQ, o < qbytes ? n0 * nbk + o : OOB, 0, 0);
  }

  // ---- the sum of the T partials for thread (m, j) = (tid / 32, tid % 32),
  //      in slice order ----
  float tpv[MAX_S];
  {
    const uint32_t m = (uint32_t)tid >> 5, j = (uint32_t)tid & 31u;
    const auto rT = rsrc(p.tpart, 4u * (uint32_t)p.S * 256u * (uint32_t)p.RT);
#pragma unroll
    for (int sl = 0; sl < MAX_S; ++sl)
      tpv[sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rT, sl < p.S && (int)j < p.r ? 4u * (((uint32_t)sl * 16u + m) * 16u * (uint32_t)p.RT + j) : OOB, 0, 0));
  }

  // issue iteration i's chunk into a ring slot.  Past the last iteration,
  // or past C in a ragged group, a wave reloads a chunk it has (an L2 hit)
  // rather than selecting other offsets, so that every iteration issues the
  // same loads from one code path and the waits below are constants.
  auto issue = [&](Chunk<TR>& f, int i) {
    const int cc = chunk_of(i < G ? i : G - 1);
    const uint32_t c = (uint32_t)(cc < C ? cc : C - 1);
    const uint32_t co = coff + 64u * c;
    // (the tile's offset goes into the per-lane offset, which is what the
    // buffer range check sees)
#pragma unroll
    for (int t = 0; t < TR; ++t)
      f.c[t] = __builtin_amdgcn_raw_buffer_load_b128(rC, co + 16u * (uint32_t)t * RB, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      f.x[v] = ld16(rX, xoff + 256u * c + 128u * (uint32_t)(v >> 1) + 16u * (uint32_t)(v & 1));
  };

  // ---- the lookup table, from the kernel arguments: word e holds the pair
  //      (byte & 15, byte >> 4) of byte e / 64; thread tid writes bytes
  //      wave + 8i (the wave's low level is picked with uniform selects) ----
  {
    float lo0 = p.lv[0], lo1 = p.lv[8];
#pragma unroll
    for (int k = 1; k < 8; ++k)
      if (wave == k) { lo0 = p.lv[k]; lo1 = p.lv[k + 8]; }
#pragma unroll
    for (int i = 0; i < 32; ++i) lut[tid + NTHREADS * i] = pack_bf16x2((i & 1) ? lo1 : lo0, p.lv[i >> 1]);
  }

  // ---- the LoRA factor B of this workgroup's rows: 16 TR rows x r bf16 =
  //      2 TR r 16-byte chunks at byte 32 TR r blockIdx, one per thread,
  //      held in registers until the epilogue (element by element: the
  //      chunk that holds the end of B may hold bytes past it, which read
  //      as zero) ----
  const uint32_t bsize = N * (uint32_t)p.r * 2u;
  const auto rB = rsrc(p.B, bsize);
  const uint32_t bchunks = 2u * (uint32_t)TR * (uint32_t)p.r;
  const uint32_t boff = 32u * (uint32_t)TR * (uint32_t)p.r * (uint32_t)blockIdx.x + 16u * (uint32_t)tid;
  u32x4v bchunk;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t o = boff + 4u * (uint32_t)i;
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rB, (uint32_t)tid < bchunks && o < bsize ? o : OOB, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rB, (uint32_t)tid < bchunks && o + 2u < bsize ? o + 2u : OOB, 0, 0);
    bchunk[i] = lo | (hi << 16);
  }

  // ---- the group constants of the workgroup's rows: row c's blocks lie in
  //      at most two groups of 256 (K <= 16384), g0 = (n nbk) >> 8 and
  //      g0 + 1; thread c < 16 TR loads both now and writes them to LDS
  //      after the prologue ----
  const auto rD = rsrc(p.dscale, 4u * ((N * nbk + 255u) / 256u));
  float dl0 = 0.0f, dl1 = 0.0f;
  if (tid < 16 * TR) {
    const uint32_t n = n0 + (uint32_t)tid;
    const uint32_t g0 = (n * nbk) >> 8;
    dl0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, n < N ? 4u * g0 : OOB, 0, 0));
    dl1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, n < N ? 4u * (g0 + 1u) : OOB, 0, 0));
  }

  // ---- prologue: the first D chunks, each group of loads kept whole and
  //      in order (the waits below count loads per chunk) ----
  Chunk<TR> f[NS];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < D; ++i) {
    issue(f[i], i);
    __builtin_amdgcn_sched_barrier(0);
  }

  // T, the scales, the rows of B and the group constants go to LDS now
  // (their loads are older than the prologue's); scales and constants share
  // the space of the per-wave sums, which are written only after every wave
  // has left the stream
  float* red = reinterpret_cast<float*>(smem);                 // [8 waves][TR][16 m][16 n]
  float* ttab = red + WAVES * TR * 256;                        // [16 m][MAX_R]
  u16* btab = reinterpret_cast<u16*>(ttab + 16 * MAX_R);       // B rows of the workgroup [16 TR][r]
  float* dtab = red;                                           // [16 TR rows][2]
  uint8_t* qtab = smem + 16 * 16 * MAX_TR;                     // [16 TR rows][nbk] scale bytes
  wait_vm<LPC * D>();
  {
    // T[m][j] for thread (m, j) = (tid / 32, tid % 32): slices past S hold zero
    float tval = 0.0f;
#pragma unroll
    for (int sl = 0; sl < MAX_S; ++sl) tval += tpv[sl];
    const int m = tid >> 5, j = tid & 31;
    ttab[m * MAX_R + j] = tval;
    if (blockIdx.x == 0 && m < p.M && j < p.r) p.T_save[m * p.r + j] = tval;
  }
  if ((uint32_t)tid < bchunks) *reinterpret_cast<u32x4v*>(reinterpret_cast<uint8_t*>(btab) + 16u * (uint32_t)tid) = bchunk;
  if (tid < 16 * TR) { dtab[2 * tid] = dl0; dtab[2 * tid + 1] = dl1; }
#pragma unroll
  for (int i = 0; i < QPASS; ++i) {
    const uint32_t o = 16u * (uint32_t)(tid + NTHREADS * i);
    if (o < qbytes) *reinterpret_cast<u32x4v*>(qtab + o) = qv[i];
  }

  __syncthreads();   // the lookup table is complete

  const uint32_t lane4 = (uint32_t)lane * 4u;
  // LDS address of (byte e of word c, this lane's copy) = byte << 8 | lane * 4
  auto lookup = [&](uint32_t c, int e) -> uint32_t {
    const uint32_t addr = __builtin_amdgcn_perm(c, lane4, 0x0C0C0400u + ((uint32_t)e << 8));
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lut) + addr);
  };
  auto operand = [&](uint32_t c) -> bf16x8_t {
    const u32x4v w = {lookup(c, 0), lookup(c, 1), lookup(c, 2), lookup(c, 3)};
    return __builtin_bit_cast(bf16x8_t, w);
  };

  f32x4_t acc[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const Chunk<TR>& f, int i) {
    if (i >= G) return;
    const int c = chunk_of(i);
    if (c >= C) return;
    const uint32_t kb = 2u * (uint32_t)c;   // first block of the chunk within the row
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      // registers x, y <- block kb, z, w <- block kb + 1 (see the header)
      const auto sxz = __builtin_amdgcn_permlane32_swap(f.c[t].x, f.c[t].z, false, false);
      const auto syw = __builtin_amdgcn_permlane32_swap(f.c[t].y, f.c[t].w, false, false);
      f32x4_t t0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, t1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
      t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[0], operand(sxz[0]), t0, 0, 0, 0);
      t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[1], operand(syw[0]), t0, 0, 0, 0);
      t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[2], operand(sxz[1]), t1, 0, 0, 0);
      t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[3], operand(syw[1]), t1, 0, 0, 0);
      // the row's first block in its second group
      const uint32_t kb_sw = 256u - ((qoff + 16u * (uint32_t)t * nbk) & 255u);
      const float2 dd = *reinterpret_cast<const float2*>(dtab + 2 * (16 * t + i16));
      const uint32_t q = *reinterpret_cast<const uint16_t*>(qtab + (uint32_t)(16 * t + i16) * nbk + kb);
      const float v0 = U8 ? (float)(q & 0xFFu) : __builtin_amdgcn_cvt_f32_fp8((int)q, 0);
      const float v1 = U8 ? (float)((q >> 8) & 0xFFu) : __builtin_amdgcn_cvt_f32_fp8((int)q, 1);
      const float s0 = v0 * (kb < kb_sw ? dd.x : dd.y);
      const float s1 = v1 * (kb + 1u < kb_sw ? dd.x : dd.y);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] += s0 * t0[e] + s1 * t1[e];
    }
  };

  // ---- the stream: chunks in groups of NS so that the register ring is
  //      indexed by constants.  At chunk i the loads of chunk i + D go out
  //      into the slot that chunk i - 1 used, and once this wave's loads of
  //      chunk i have landed (D later chunks may still be in flight) it is
  //      multiplied. ----
  for (int i0 = 0; i0 < G; i0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = i0 + j;
      __builtin_amdgcn_sched_barrier(0);
      issue(f[(j + D) % NS], i + D);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<LPC * D>();
      process(f[j], i);            // nothing past the last iteration or past C
    }
  }
  wait_vm<0>();

  // ---- sums over the waves (fixed order), LoRA term, store ----
  __syncthreads();   // every wave is done
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * TR + t) * 256 + (4 * g + e) * 16 + i16] = acc[t][e];
  __syncthreads();
  // one output (m, row c) per thread and pass; consecutive threads take
  // consecutive rows, so each store instruction covers a run of Y's row m
  const int R = 16 * TR;
  for (int o = tid; o < p.M * R; o += NTHREADS) {
    const int m = o / R, c = o - m * R;
    const uint32_t n = n0 + (uint32_t)c;
    if (n >= N) continue;
    const int t = c >> 4, ci = c & 15;
    float base = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) base += red[(w * TR + t) * 256 + m * 16 + ci];
    float lora = 0.0f;
    for (int j = 0; j < p.r; ++j) lora += ttab[m * MAX_R + j] * bf16_to_f32(btab[c * p.r + j]);
    p.Y[(size_t)m * N + n] = f32_to_bf16(base + p.s * lora);
  }
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

// Rows per workgroup: enough 16-row tiles (at most 7) that the grid is about
// one workgroup per compute unit.
struct Plan {
  int TR, RT;
};
static Plan plan(int64_t N, int r) {
  const int64_t cus = device_cus();
  Plan pl;
  pl.TR = (int)std::min<int64_t>(MAX_TR, std::max<int64_t>(1, (N + 16 * cus - 1) / (16 * cus)));
  pl.RT = (r + 15) / 16;
  return pl;
}

// dynamic LDS: per-wave sums [8][TR][256] and T [16][MAX_R] (fp32), which
// in the stream hold the group constants [16 MAX_TR][2] (fp32) and the
// scale bytes [16 TR][nbk]; then the workgroup's rows of B [16 TR][r] (bf16)
static uint32_t dyn_lds(const Plan& pl, int r, uint32_t K) {
  const uint32_t sums = 4u * ((uint32_t)WAVES * (uint32_t)pl.TR * 256u + 16u * MAX_R);
  const uint32_t stream = 16u * 16u * MAX_TR + 16u * (uint32_t)pl.TR * (K / 64u);
  return std::max(sums, stream) + 32u * (uint32_t)pl.TR * (uint32_t)r;
}

template <int TR, bool U8>
static hipError_t launch_one(const DecArgs& p, unsigned grid, uint32_t lds, hipStream_t st) {
  const hipError_t attr = set_dynamic_lds(reinterpret_cast<const void*>(&k_decode<TR, U8>), MAX_DYN_LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_decode<TR, U8>), dim3(grid), dim3(NTHREADS), lds, st, p);
  return hipGetLastError();
}

template <bool U8>
static hipError_t launch_tr(const Plan& pl, const DecArgs& p, unsigned grid, uint32_t lds, hipStream_t st) {
  switch (pl.TR) {
    case 1: return launch_one<1, U8>(p, grid, lds, st);
    case 2: return launch_one<2, U8>(p, grid, lds, st);
    case 3: return launch_one<3, U8>(p, grid, lds, st);
    case 4: return launch_one<4, U8>(p, grid, lds, st);
    case 5: return launch_one<5, U8>(p, grid, lds, st);
    case 6: return launch_one<6, U8>(p, grid, lds, st);
    case 7: return launch_one<7, U8>(p, grid, lds, st);
    default: return hipErrorInvalidConfiguration;
  }
}

}  // namespace dec

bool decode_fits(int64_t M, const NF4View& w, int r) {
  const int64_t lim = (int64_t)1 << 31;
  // 32-bit buffer offsets; K a multiple of 256 and at most 16384 (a row's
  // blocks lie in at most two groups of 256); 8-bit block scales (fp32
  // scales take the tiled path); at most two 16-rank tiles of T
  // (rows up to 16 * MAX_TR past N are addressed, and read as zeros)
  return M >= 1 && M <= 16 && r >= 1 && r <= dec::MAX_R && w.K % 256 == 0 && w.K <= 16384 &&
         !w.fp32_scale && (w.N + 16 * dec::MAX_TR) * (w.K / 2) + 1024 < lim &&
         (w.N + 16 * dec::MAX_TR) * (w.K / 64) + 1024 < lim && 16 * w.K * 2 < lim && (int64_t)r * w.K * 2 < lim &&
         w.N * r * 2 < lim && w.N * (w.K / 64) + 1024 < lim;
}

size_t decode_ws_bytes(int64_t K, int r) {
  if (K <= 0 || K % 256 || r < 1) return 0;
  const int S = dec::t_slices((uint32_t)K);
  return (size_t)S * 16u * 16u * (size_t)((r + 15) / 16) * sizeof(float);
}

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, float* ws, hipStream_t st) {
  const dec::Plan pl = dec::plan(w.N, r);
  const int S = dec::t_slices((uint32_t)w.K);
  hipLaunchKernelGGL(dec::k_decode_t, dim3((unsigned)S, (unsigned)pl.RT), dim3(256), 0, st, X, (int)M, A, r,
                     (uint32_t)w.K, S, pl.RT, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dec::DecArgs p;
  p.X = X; p.M = (int)M;
  p.codes = w.codes; p.qscale = w.qscale; p.dscale = w.dscale;
  p.N = (uint32_t)w.N; p.K = (uint32_t)w.K;
  for (int i = 0; i < 16; ++i) p.lv[i] = w.lv[i];
  p.tpart = ws; p.S = S;
  p.RT = pl.RT;
  p.B = B; p.r = r; p.s = s;
  p.Y = Y; p.T_save = T_save;
  const unsigned grid = (unsigned)((w.N + 16 * pl.TR - 1) / (16 * pl.TR));
  const uint32_t lds = dec::dyn_lds(pl, r, (uint32_t)w.K);
  return w.u8_scale ? dec::launch_tr<true>(pl, p, grid, lds, st) : dec::launch_tr<false>(pl, p, grid, lds, st);
}

}  // namespace qln
