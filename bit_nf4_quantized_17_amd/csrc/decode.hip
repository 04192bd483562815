// decode.hip -- the forward at decode sizes (M <= 16 tokens).  Ultralytics
// glossary "QLoRA", "How QLoRA works": the frozen layer dequantizes NF4 to
// bfloat16 for the matrix product and adds the LoRA path.
//
// At M <= 16 the layer is bound by streaming the packed weight (0.516 bytes
// per weight) from HBM.  This path multiplies the same bf16 weight as the
// prefill kernels, w' = bf16(fl32(L[code] * s_b)) with s_b = fl32(v(q_b) d_g),
// dequantized in registers (about four vector-ALU operations per weight), and
// adds the LoRA term as their prologue does:
//   Y = X W'^T + bf16(s_lora T) B^T,      T = X A^T (fp32)
// (Taking the block scale out of the product -- bf16(L[code]) from a table,
// s_b applied to each block's partial sum -- costs less than one operation
// per weight, but it rounds the unscaled level instead of the weight: on
// weights with outliers that moves outputs past the elementwise tolerance
// already at K = 8192.)
//
// Two launches.  The first sums T = X A^T over S slices of the contraction
// (S x RT small workgroups, fp32 partials in the workspace).  The second
// streams the weight with no communication between workgroups: a workgroup
// owns 16 * TR consecutive output columns (W rows, TR <= 7) over the whole
// contraction, so it finishes its outputs itself; at the start it adds up
// the S partials of T in a fixed order for its LoRA term.  Its grid is about one
// workgroup per compute unit.  The 8-bit block scales of its rows are one
// contiguous run of bytes; at the start it restores them into an fp32 table
// in LDS, so a row's blocks may span any number of scale groups.
//
// The eight waves split the contraction into chunks of 128 (two blocks, 64
// code bytes of a row), wave w taking every eighth chunk from chunk w, and
// run independently until the final sums: no LDS staging and no barrier in
// the stream.  Per chunk and 16-row tile a wave loads the codes straight
// into registers -- lane (n = lane % 16, g = lane / 16) takes bytes
// [16 g, 16 g + 16) of row n, codes 32 g .. 32 g + 31 of the chunk, all in
// block g / 2 of it -- and register v (8 codes) of every lane becomes the
// weight operand of MFMA v, whose 32 contraction slots are codes 32 g + 8 v
// .. + 7 of the four lane groups.  A lane's 16 scaled levels are built by
// the two lanes of its row and block (lanes 16 apart: one scales levels
// 0 .. 7, the other 8 .. 15, and a v_permlane16_swap of each plane word with
// itself hands both lanes both halves) as low-byte and high-byte planes, and
// each code is looked up with byte permutes.  The even and the odd codes of
// a register are looked up separately, so an operand holds its elements in
// the order 0, 2, 4, 6, 1, 3, 5, 7; the X fragments (row m, the same 8
// contraction indices) are permuted the same way.  Loads run one chunk
// ahead in a two-slot register ring.  Since the waves run at the same pace, the two
// halves of each 128-byte line reach L2 close together and the line is
// fetched from HBM once (measured: a wave that read both halves itself, one
// chunk apart, fetched 1.7 times the weight's bytes).  The workgroups start
// at different groups of chunks (if every workgroup read the same column
// window of its rows at the same time, the requests would pile onto a few
// memory channels).  Wave t starts its sums of tile t from the LoRA term,
// and the eight waves' sums are added in LDS in wave order, so results do
// not depend on timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "device.h"

namespace qln {
namespace dec {

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int CHUNK = 128;              // contraction elements per chunk (two blocks)
constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every range this path uses
constexpr int MAX_R = QLN_MAX_RANK;     // ranks (T is kept [16][MAX_R] in LDS)
constexpr int MAX_TR = 7;               // 16-row tiles per workgroup
constexpr int MAX_DYN_LDS = 160 * 1024; // dynamic LDS limit set on the kernels (all of it)
constexpr uint32_t MAX_K = 65536;       // longest contraction
constexpr int MAX_S = 16;               // slices of the T partials
constexpr int QPASS = 4;                // 16-byte scale loads a thread
constexpr uint32_t QBYTES = 16u * NTHREADS * QPASS;   // scale bytes a workgroup can restore (32 KB)
constexpr int BCH = (16 * MAX_TR * (MAX_R + 8) / 8 + NTHREADS - 1) / NTHREADS;   // 16-byte B chunks a thread

// Row pitch of the restored block scales in LDS: K / 64 is a multiple of 4,
// so K / 64 + 2 is twice an odd number and the sixteen rows a lane group
// reads at one block index fall on sixteen different banks (a pitch of
// K / 64 put them all on one bank).
__host__ __device__ inline uint32_t scale_pitch(uint32_t K) { return K / 64u + 2u; }

// floats at the start of the dynamic LDS: the per-wave sums [8][TR][256]
// after the stream, the restored block scales [16 TR][scale_pitch] during it
__host__ __device__ inline uint32_t region0_floats(int TR, uint32_t K) {
  const uint32_t sums = (uint32_t)WAVES * 256u, scales = 16u * scale_pitch(K);
  return (sums > scales ? sums : scales) * (uint32_t)TR;
}

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

// A block's 16 bf16 weights bf16(fl32(L[c] * s)) as a low-byte and a
// high-byte plane (word j holds levels 4j .. 4j + 3).  lv8: this lane's
// levels, 0 .. 7 in even 16-lane rows and 8 .. 15 in odd ones; the two lanes
// 16 apart share a row and a block, and v_permlane16_swap of a word with
// itself returns the even row's word and the odd row's word in both lanes.
struct Table {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Table make_table(const float (&lv8)[8], float s) {
  uint32_t pk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(lv8[2 * j] * s, lv8[2 * j + 1] * s);
  Table t;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t lo = __builtin_amdgcn_perm(pk[2 * q + 1], pk[2 * q], 0x06040200u);
    const uint32_t hi = __builtin_amdgcn_perm(pk[2 * q + 1], pk[2 * q], 0x07050301u);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    t.lo[q] = l[0]; t.lo[2 + q] = l[1];
    t.hi[q] = h[0]; t.hi[2 + q] = h[1];
  }
  return t;
}

// four 4-bit indices (one per byte) -> their bf16 low bytes and high bytes.
// Byte selectors past 12 read as 0xFF, so each half of the table is looked
// up with the other half's indices pushed past 16 and the two are AND-ed.
__device__ __forceinline__ void lookup4(const Table& t, uint32_t idx, uint32_t& lo, uint32_t& hi) {
  const uint32_t selA = __builtin_amdgcn_bitop3_b32(idx, idx << 1, 0x10101010u, 0xF8);  // 8..15 -> 24..31 (0xFF)
  const uint32_t selB = selA ^ 0x18181818u;                // indices 0..7 -> 24..31, 8..15 -> 0..7
  lo = __builtin_amdgcn_perm(t.lo[1], t.lo[0], selA) & __builtin_amdgcn_perm(t.lo[3], t.lo[2], selB);
  hi = __builtin_amdgcn_perm(t.hi[1], t.hi[0], selA) & __builtin_amdgcn_perm(t.hi[3], t.hi[2], selB);
}

// 8 codes (element e in bits 4e .. 4e + 3) -> an MFMA operand of their bf16
// weights in the element order 0, 2, 4, 6, 1, 3, 5, 7
__device__ __forceinline__ bf16x8_t dequant8(const Table& t, uint32_t c) {
  uint32_t l, h;
  u32x4v o;
  lookup4(t, c & 0x0F0F0F0Fu, l, h);
  o[0] = __builtin_amdgcn_perm(h, l, 0x05010400u);
  o[1] = __builtin_amdgcn_perm(h, l, 0x07030602u);
  lookup4(t, (c >> 4) & 0x0F0F0F0Fu, l, h);
  o[2] = __builtin_amdgcn_perm(h, l, 0x05010400u);
  o[3] = __builtin_amdgcn_perm(h, l, 0x07030602u);
  return __builtin_bit_cast(bf16x8_t, o);
}

// 8 bf16 in element order -> the order 0, 2, 4, 6, 1, 3, 5, 7
__device__ __forceinline__ bf16x8_t evens_then_odds(bf16x8_t x) {
  const u32x4v w = __builtin_bit_cast(u32x4v, x);
  const u32x4v o = {__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                    __builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u)};
  return __builtin_bit_cast(bf16x8_t, o);
}

// One wave's register loads of one chunk: the X fragments of the chunk's four
// MFMAs (shared by every tile), then per tile the codes of the lane's row.
template <int TR>
struct Chunk {
  bf16x8_t x[4];          // X[m = lane % 16][chunk offset 32 g + 8 v .. + 8], v = 0 .. 3
  u32x4v c[TR];           // row n0 + 16 t + lane % 16, code bytes [16 g, 16 g + 16) of the chunk
};

// Loads per chunk per wave, and D, the chunks loaded ahead.  One: a wave
// takes longer to dequantize and multiply a chunk than the chunk's loads take
// to arrive, and a deeper ring only lengthens the start, where every
// workgroup's first requests arrive together (measured: D = 2 and the earlier
// register-budget depths were 4-20% slower than D = 1).
template <int TR>
constexpr int lpc_of() { return TR + 4; }
template <int TR>
constexpr int depth_of() { return 1; }

template <int TR, bool U8>
__global__ __launch_bounds__(NTHREADS) void k_decode(DecArgs p) {
  constexpr int D = depth_of<TR>();
  constexpr int NS = D + 1;
  constexpr int LPC = lpc_of<TR>();
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
  // X row m = lane % 16 at contraction offset 32 g of a chunk (rows past M read zero)
  const uint32_t xoff = i16 < p.M ? (uint32_t)i16 * K * 2u + 64u * (uint32_t)g : OOB;

  // ---- the workgroup's block scales, 16 TR nbk contiguous bytes from
  //      n0 nbk (at most QBYTES), 16 bytes a thread and pass, with the group
  //      constant of each thread's 16 (n0 nbk is a multiple of 16, so they
  //      lie in one group of 256); rows past N read zeros, and a wave whose
  //      16-byte pieces all lie past the run issues nothing ----
  const uint32_t qbytes = 16u * (uint32_t)TR * nbk;
  const auto rD = rsrc(p.dscale, 4u * ((N * nbk + 255u) / 256u));
  u32x4v qv[QPASS];
  float qd[QPASS];
#pragma unroll
  for (int i = 0; i < QPASS; ++i) {
    qv[i] = u32x4v{0u, 0u, 0u, 0u};
    qd[i] = 0.0f;
    if (16u * (uint32_t)(64 * wave + NTHREADS * i) >= qbytes) continue;
    const uint32_t o = 16u * (uint32_t)(tid + NTHREADS * i);
    qv[i] = __builtin_amdgcn_raw_buffer_load_b128(rQ, o < qbytes ? n0 * nbk + o : OOB, 0, 0);
    qd[i] = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rD, o < qbytes ? 4u * ((n0 * nbk + o) >> 8) : OOB, 0, 0));
  }

  // issue iteration i's chunk into a ring slot.  Past the last iteration,
  // or past C in a ragged group, a wave reloads a chunk it has (an L2 hit)
  // rather than selecting other offsets, so that every iteration issues the
  // same loads from one code path (the waits count loads in issue order).
  auto issue = [&](Chunk<TR>& f, int i) {
    const int cc = chunk_of(i < G ? i : G - 1);
    const uint32_t c = (uint32_t)(cc < C ? cc : C - 1);
    const uint32_t co = coff + 64u * c;
    // (the tile's offset goes into the per-lane offset, which is what the
    // buffer range check sees)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      f.x[v] = ld16(rX, xoff + 256u * c + 16u * (uint32_t)v);
#pragma unroll
    for (int t = 0; t < TR; ++t)
      f.c[t] = __builtin_amdgcn_raw_buffer_load_b128(rC, co + 16u * (uint32_t)t * RB, 0, 0);
  };

  // ---- this lane's eight levels, 0 .. 7 in even 16-lane rows and 8 .. 15
  //      in odd ones ----
  float lv8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) lv8[e] = (g & 1) ? p.lv[8 + e] : p.lv[e];

  // ---- the LoRA factor B of this workgroup's rows, zero-padded to
  //      [16 TR][BP] bf16 (BP = RP + 8, RP = r rounded up to 32): 16-byte
  //      chunk q is row q / (BP / 8), ranks 8 (q % (BP / 8)) .. + 8, up to
  //      BCH chunks a thread (a whole chunk in one load when r % 8 == 0,
  //      else element by element; ranks past r and rows past N read zero) ----
  const uint32_t RP = ((uint32_t)p.r + 31u) & ~31u, BP = RP + 8u, BQ = BP / 8u;
  const uint32_t bsize = N * (uint32_t)p.r * 2u;
  const auto rB = rsrc(p.B, bsize);
  const uint32_t bchunks = 16u * (uint32_t)TR * BQ;
  const bool bvec = (p.r & 7) == 0;
  u32x4v bch[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    bch[i] = u32x4v{0u, 0u, 0u, 0u};
    if ((uint32_t)(64 * wave + NTHREADS * i) >= bchunks) continue;   // nothing of this wave's
    const uint32_t q = (uint32_t)(tid + NTHREADS * i);
    const uint32_t c = q / BQ, j0 = 8u * (q - c * BQ);
    const uint32_t row0 = ((n0 + c) * (uint32_t)p.r + j0) * 2u;   // byte offset of (row, j0)
    const bool live = q < bchunks && n0 + c < N && j0 < (uint32_t)p.r;
    if (bvec) {
      bch[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, live ? row0 : OOB, 0, 0);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t j = j0 + 2u * (uint32_t)w;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
            rB, live && j < (uint32_t)p.r ? row0 + 4u * (uint32_t)w : OOB, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
            rB, live && j + 1u < (uint32_t)p.r ? row0 + 4u * (uint32_t)w + 2u : OOB, 0, 0);
        bch[i][w] = lo | (hi << 16);
      }
    }
  }

  // ---- T = the sum of its partials in slice order, kept [16 m][MAX_R] in
  //      LDS; entry e = (m, j) of [16][RP] is thread e % NTHREADS's, and
  //      ranks past r and rows past M hold zero.  The loads go out now,
  //      before the first chunk's, and are summed while the chunk is on its
  //      way; a wave whose entries all lie in rows past M, and every slice
  //      past S, issues nothing. ----
  const auto rT = rsrc(p.tpart, 4u * (uint32_t)p.S * 256u * (uint32_t)p.RT);
  constexpr int TP = 16 * MAX_R / NTHREADS;
  const uint32_t RW = 16u * (uint32_t)p.RT;   // width of a partial's rows
  float tp[TP][MAX_S];
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const uint32_t e = (uint32_t)(tid + NTHREADS * i), m = e / RP, j = e - m * RP;
    const uint32_t e0 = (uint32_t)(64 * wave + NTHREADS * i);
    const bool wave_live = e0 < 16u * RP && e0 / RP < (uint32_t)p.M;
#pragma unroll
    for (int sl = 0; sl < MAX_S; ++sl) {
      tp[i][sl] = 0.0f;
      if (!wave_live || sl >= p.S) continue;
      tp[i][sl] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rT, m < (uint32_t)p.M && j < (uint32_t)p.r ? 4u * (((uint32_t)sl * 16u + m) * RW + j) : OOB, 0, 0));
    }
  }

  // ---- the first D chunks, each group of loads kept whole and in order
  //      (the waits below count loads per chunk) ----
  Chunk<TR> f[NS];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < D; ++i) {
    issue(f[i], i);
    __builtin_amdgcn_sched_barrier(0);
  }

  // The restored scales, T and the rows of B go to LDS now (their loads are
  // older than the first chunk's); the scales share the space of the
  // per-wave sums, which are written only after every wave has left the
  // stream
  const uint32_t SP = scale_pitch(K);
  float* red = reinterpret_cast<float*>(smem);                 // [8 waves][TR][16 m][16 n]
  float* stab = red;                                           // [16 TR rows][SP] block scales
  float* ttab = red + region0_floats(TR, K);                   // [16 m][MAX_R]
  u16* btab = reinterpret_cast<u16*>(ttab + 16 * MAX_R);       // B rows of the workgroup [16 TR][BP]
  wait_vm<LPC * D>();
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const uint32_t q = (uint32_t)(tid + NTHREADS * i);
    if (q < bchunks) *reinterpret_cast<u32x4v*>(btab + 8u * q) = bch[i];
  }
  // s_b = fl32(v(q_b) * d_g): v the E4M3 value of the byte, or the byte as an
  // integer for uint8-linear scales.  Scale j of the run is row j / nbk,
  // block j % nbk; four consecutive scales from a multiple of 4 share a row.
#pragma unroll
  for (int i = 0; i < QPASS; ++i) {
    const uint32_t o = 16u * (uint32_t)(tid + NTHREADS * i);
    if (o < qbytes) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t q = qv[i][w];
        const uint32_t j = o + 4u * (uint32_t)w, row = j / nbk;
        float sv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t qb = q >> (8 * b);
          const float v = U8 ? (float)(qb & 0xFFu) : __builtin_amdgcn_cvt_f32_fp8((int)qb, 0);
          sv[b] = v * qd[i];
        }
        float* dst = stab + j + 2u * row;   // row * SP + j % nbk, 8-byte aligned
        reinterpret_cast<float2*>(dst)[0] = float2{sv[0], sv[1]};
        reinterpret_cast<float2*>(dst)[1] = float2{sv[2], sv[3]};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const uint32_t e = (uint32_t)(tid + NTHREADS * i), m = e / RP, j = e - m * RP;
    if (e >= 16u * RP) continue;
    float tval = 0.0f;
#pragma unroll
    for (int sl = 0; sl < MAX_S; ++sl) tval += tp[i][sl];
    ttab[m * MAX_R + j] = tval;
    if (blockIdx.x == 0 && m < (uint32_t)p.M && j < (uint32_t)p.r) p.T_save[m * (uint32_t)p.r + j] = tval;
  }

  __syncthreads();   // the restored scales, T and B are complete

  // ---- the LoRA term of tile t, bf16(s T) B^T (contraction over the
  //      ranks, 32 per MFMA: lane (i, g) holds bf16(s T[i][32 c + 8 g ..])
  //      and B[n0 + 16 t + i][32 c + 8 g ..]), starts wave t's sums of tile
  //      t; the stream's products are added to it ----
  f32x4_t acc[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (wave != t) continue;
    for (uint32_t c = 0; c < RP / 32u; ++c) {
      const f32x4_t* tr = reinterpret_cast<const f32x4_t*>(ttab + i16 * MAX_R + 32u * c + 8u * (uint32_t)g);
      const f32x4_t ta = tr[0], tb = tr[1];
      const u32x4v tv = {pack_bf16x2(p.s * ta[0], p.s * ta[1]), pack_bf16x2(p.s * ta[2], p.s * ta[3]),
                         pack_bf16x2(p.s * tb[0], p.s * tb[1]), pack_bf16x2(p.s * tb[2], p.s * tb[3])};
      const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(btab + (uint32_t)(16 * t + i16) * BP + 32u * c +
                                                             8u * (uint32_t)g);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, tv), bv, acc[t], 0, 0, 0);
    }
  }

  auto process = [&](const Chunk<TR>& f, int i) {
    if (i >= G) return;
    const int c = chunk_of(i);
    if (c >= C) return;
    // the lane's block within the row: two per chunk, lane groups 0, 1 in the
    // first; the chunk's block scales of every tile are read up front
    const uint32_t kb = 2u * (uint32_t)c + ((uint32_t)g >> 1);
    float sc[TR];
#pragma unroll
    for (int t = 0; t < TR; ++t) sc[t] = stab[(uint32_t)(16 * t + i16) * SP + kb];
    bf16x8_t xp[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) xp[v] = evens_then_odds(f.x[v]);
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const Table tb = make_table(lv8, sc[t]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xp[0], dequant8(tb, f.c[t].x), acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xp[1], dequant8(tb, f.c[t].y), acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xp[2], dequant8(tb, f.c[t].z), acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xp[3], dequant8(tb, f.c[t].w), acc[t], 0, 0, 0);
    }
  };

  // ---- the stream: chunks in groups of NS so that the register ring is
  //      indexed by constants.  At chunk i the loads of chunk i + D go out
  //      into the slot that chunk i - 1 used, and chunk i is multiplied as it
  //      lands: a chunk's X fragments are loaded before its tiles, and each
  //      use of a loaded register waits only for its own load, so tile 0 is
  //      dequantized while the later tiles are still arriving. ----
  for (int i0 = 0; i0 < G; i0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = i0 + j;
      __builtin_amdgcn_sched_barrier(0);
      issue(f[(j + D) % NS], i + D);
      __builtin_amdgcn_sched_barrier(0);
      process(f[j], i);            // nothing past the last iteration or past C; each use of a
                                   // loaded register waits for its own load (X, then tile by tile)
    }
  }
  wait_vm<0>();
  __syncthreads();   // every wave has left the stream (the scales' space is reused)

  // ---- sums over the waves (fixed order), store ----
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
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[(w * TR + t) * 256 + m * 16 + ci];
    p.Y[(size_t)m * N + n] = f32_to_bf16(sum);
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

// dynamic LDS: the sums / restored scales, T [16][MAX_R] fp32, the
// workgroup's rows of B [16 TR][BP] bf16
static uint32_t dyn_lds(int TR, int r, uint32_t K) {
  const uint32_t bp = (((uint32_t)r + 31u) & ~31u) + 8u;
  return 4u * region0_floats(TR, K) + 4u * 16u * MAX_R + 2u * 16u * (uint32_t)TR * bp;
}

// Rows per workgroup: enough 16-row tiles (at most 7) that the grid is about
// one workgroup per compute unit, and no more than the dynamic LDS and the
// scale copy hold (K = 65536 allows two).
struct Plan {
  int TR, RT;
};
static Plan plan(int64_t N, int r, uint32_t K) {
  const int64_t cus = device_cus();
  Plan pl;
  pl.TR = (int)std::min<int64_t>(MAX_TR, std::max<int64_t>(1, (N + 16 * cus - 1) / (16 * cus)));
  while (pl.TR > 1 && (dyn_lds(pl.TR, r, K) > (uint32_t)MAX_DYN_LDS || 16u * (uint32_t)pl.TR * (K / 64u) > QBYTES))
    --pl.TR;
  pl.RT = (r + 15) / 16;
  return pl;
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
  // 32-bit buffer offsets; K a multiple of 256 (whole chunks for the eight
  // waves) and at most MAX_K (one 16-row tile's restored scales fit the LDS
  // and the scale copy); 8-bit block scales (fp32 scales take the tiled
  // path) (rows up to 16 * MAX_TR past N are addressed, and read as zeros)
  return M >= 1 && M <= 16 && r >= 1 && r <= dec::MAX_R && w.K % 256 == 0 && w.K <= dec::MAX_K &&
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
  const dec::Plan pl = dec::plan(w.N, r, (uint32_t)w.K);
  const uint32_t lds = dec::dyn_lds(pl.TR, r, (uint32_t)w.K);
  if (lds > (uint32_t)dec::MAX_DYN_LDS || 16u * (uint32_t)pl.TR * ((uint32_t)w.K / 64u) > dec::QBYTES)
    return hipErrorInvalidConfiguration;   // excluded by decode_fits and the plan; nothing launched
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
  return w.u8_scale ? dec::launch_tr<true>(pl, p, grid, lds, st) : dec::launch_tr<false>(pl, p, grid, lds, st);
}

}  // namespace qln
