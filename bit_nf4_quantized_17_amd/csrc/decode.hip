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
// s_b = fl32(E4M3(q) * d) and added in fp32.  (The prefill and training
// kernels multiply the exactly dequantized bf16 weight instead; both round
// the weight's relative value once to bf16 precision.)
//
// One launch, no communication between workgroups: a workgroup owns 16 * TR
// consecutive output columns (W rows, TR <= 7) over the whole contraction,
// so it finishes its outputs itself, and it computes T = X A^T itself too
// (A and X are small and stay in L2; the repeated reads cost far less than
// the HBM stream they overlap).  The grid is about one workgroup per
// compute unit.
//
// The contraction goes in steps of 512 (8 blocks), each workgroup starting
// at its own step (see the rotation below).  The eight waves load
// each step's codes and 8-bit scales together -- each 16-byte-lane
// instruction covers 4 rows x 256 contiguous bytes -- into registers NS - 1
// steps ahead, and when a step's loads have landed they write them into one
// of two LDS stages, with the 16-byte chunks of a row XOR-swizzled by the
// row index so that the MFMA-layout reads (16 rows x 8 bytes per 16 lanes)
// hit distinct banks.  Wave w then multiplies block w of the step for every
// tile, with its own X and A fragments of that block (read from L2 with the
// same lead), so X and A are each read once per workgroup.  A barrier per
// step hands the stage over.  Every load goes to registers, so the
// compiler's own waits count them exactly and never wait for a later step.
// The eight waves' sums are added in LDS in wave order, so results do not
// depend on timing.
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
constexpr int STEP = 512;               // contraction elements per step (8 blocks, one per wave)
constexpr uint32_t ROW_BYTES = 256;     // code bytes of one row in a step
constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every range this path uses
constexpr int MAX_R = 32;               // ranks the fused T handles (two 16-rank tiles)
constexpr int MAX_TR = 7;               // 16-row tiles per workgroup
constexpr int MAX_DYN_LDS = 94 * 1024;  // dynamic LDS limit set on the kernels (two stages use <= 60 KB)

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

struct DecArgs {
  const u16* X; int M;                      // X [M][K], M <= 16
  const uint8_t* codes; const uint8_t* qscale; const float* dscale;
  uint32_t N, K;
  float lv[16];                             // the codebook's levels
  const u16* A; const u16* B; int r; float s;
  u16* Y; float* T_save;
};

// LDS of one stage: codes [16 TR rows][256 B], then the 8-bit scales
// [32 ceil(TR / 2) rows][8 B] (whole 64-lane dword loads)
struct StageLayout {
  uint32_t codes_insts, qs_insts, qs_off, bytes;
};
__host__ __device__ inline StageLayout stage_layout(int TR) {
  StageLayout L;
  L.codes_insts = 4u * (uint32_t)TR;             // 1 KB each: 4 rows x 256 B
  L.qs_insts = ((uint32_t)TR + 1u) / 2u;         // 256 B each: 32 rows x 8 B
  L.qs_off = 1024u * L.codes_insts;
  L.bytes = L.qs_off + 256u * L.qs_insts;
  return L;
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
// A barrier that waits for this wave's LDS operations but not for its
// outstanding direct-to-LDS loads (a plain __syncthreads would wait for
// every stage in flight).
__device__ __forceinline__ void barrier_lds_only() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
}

// One wave's register loads of one step: the X and A fragments of its
// block, and its share of the step's codes and scale bytes.
template <int RT, int CPW>
struct Frags {
  bf16x8_t x[2];          // X[m = lane%16][64 kb + 16 (lane/16) + 8 h .. +8], h = 0, 1
  bf16x8_t a[RT][2];      // A[16 rt + lane%16][same]
  u32x4v c[CPW];          // code loads (16 bytes a lane)
  uint32_t q;             // scale load (4 bytes a lane)
};

// TR: 16-row tiles per workgroup; RT: 16-rank tiles of T.  Derived: CPW,
// code loads per wave per step (the step's 4 TR instructions over the eight
// waves), and NS, the register slots of the load ring (NS - 1 steps in
// flight: 4 for the narrower workgroups, whose steps are short, 2 when the
// slots are wide).
template <int TR>
constexpr int cpw_of() { return (4 * TR + WAVES - 1) / WAVES; }
template <int TR, int RT>
constexpr int ns_of() { return (RT == 1 && cpw_of<TR>() <= 2) ? 5 : 3; }

template <int TR, int RT>
__global__ __launch_bounds__(NTHREADS) void k_decode(DecArgs p) {
  constexpr int CPW = cpw_of<TR>();
  constexpr int NS = ns_of<TR, RT>();
  __shared__ __attribute__((aligned(16))) uint32_t lut[LUT_WORDS];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, qk = lane >> 4;
  const uint32_t K = p.K, N = p.N, RB = K / 2u, nbk = K / 64u;
  const uint32_t n0 = (uint32_t)blockIdx.x * 16u * (uint32_t)TR;
  const int nsteps = (int)((K + STEP - 1) / STEP);   // the last step may hold 4 blocks
  // Workgroups start at different steps of the contraction: if every
  // workgroup read the same 256-byte window of its rows at the same time,
  // the requests would pile onto a few memory channels (measured: 26.8 us
  // against 20.7 us for the 117 MB weight of a 28672 x 8192 layer).
  const int rot = (int)(blockIdx.x % (uint32_t)nsteps);
  auto kstep = [&](int st) { const int k = st + rot; return k >= nsteps ? k - nsteps : k; };
  const StageLayout SL = stage_layout(TR);
  uint8_t* junk = smem + 2u * SL.bytes;              // target of the padding loads

  const auto rC = rsrc(p.codes, N * RB);
  const auto rQ = rsrc(p.qscale, N * nbk);
  const auto rX = rsrc(p.X, (uint32_t)p.M * K * 2u);
  const auto rA = rsrc(p.A, (uint32_t)p.r * K * 2u);

  // ---- this wave's share of a step: code instructions wave, wave + 8, ...
  //      (CPW slots, the last may be padding) and scale instruction wave ----
  //  codes instruction ii: lane l takes row 4 ii + l/16 and writes its chunk
  //  slot l%16, which holds the row's memory chunk (l%16) ^ (row%16);
  //  scale instruction jj: lane l takes row 32 jj + l/2, dword l%2 of the
  //  step's 8 scale bytes.
  uint32_t src[CPW];   // per code slot: byte offset at step 0 (OOB: padding or rows past N)
  uint32_t dst[CPW];   // per code slot: LDS offset within a stage (NONE: padding)
  constexpr uint32_t NONE = 0xFFFFFFFFu;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const uint32_t ii = (uint32_t)(wave + 8 * c);
    const uint32_t row = 4u * ii + (uint32_t)(lane >> 4);
    const uint32_t chunk = (uint32_t)(lane & 15) ^ (row & 15u);
    const bool real = ii < SL.codes_insts;
    src[c] = (real && n0 + row < N) ? (n0 + row) * RB + 16u * chunk : OOB;
    dst[c] = real ? 1024u * ii : NONE;
  }
  uint32_t qsrc, qdst;
  {
    const uint32_t jj = (uint32_t)wave;
    const uint32_t row = 32u * jj + (uint32_t)(lane >> 1);
    const bool real = jj < SL.qs_insts;
    qsrc = (real && row < 16u * (uint32_t)TR && n0 + row < N) ? (n0 + row) * nbk + 4u * (uint32_t)(lane & 1) : OOB;
    qdst = real ? SL.qs_off + 256u * jj : NONE;
  }
  const uint32_t xoff = (uint32_t)i16 * K * 2u + 32u * (uint32_t)qk;
  uint32_t aoff[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) aoff[rt] = (uint32_t)(16 * rt + i16) * K * 2u + 32u * (uint32_t)qk;

  // issue step st into registers: this wave's X and A fragments (block
  // 8 st + wave), then its code and scale loads.  Every step issues the same
  // loads (padding slots load past the buffer), so that the waits are
  // constants; a step or block past the contraction reads past the buffers
  // (zeros, no memory traffic).
  auto issue = [&](Frags<RT, CPW>& f, int st) {
    const bool step_live = st < nsteps;
    const uint32_t ks = step_live ? (uint32_t)kstep(st) : 0u;
    const uint32_t kb = 8u * ks + (uint32_t)wave;
    const bool live = step_live && kb < nbk;
#pragma unroll
    for (int h = 0; h < 2; ++h) f.x[h] = ld16(rX, live ? xoff + 128u * kb + 16u * (uint32_t)h : OOB);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h) f.a[rt][h] = ld16(rA, live ? aoff[rt] + 128u * kb + 16u * (uint32_t)h : OOB);
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      f.c[c] = __builtin_amdgcn_raw_buffer_load_b128(rC, (src[c] == OOB || !step_live) ? OOB : src[c] + ROW_BYTES * ks,
                                                     0, 0);
    f.q = __builtin_amdgcn_raw_buffer_load_b32(rQ, (qsrc == OOB || !step_live) ? OOB : qsrc + 8u * ks, 0, 0);
  };
  // write a landed step's codes and scale bytes into LDS stage st % 2
  // (padding slots write to the junk area, so their loads stay live)
  auto stage_write = [&](const Frags<RT, CPW>& f, int st) {
    uint8_t* sbase = smem + (uint32_t)(st & 1) * SL.bytes;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      *reinterpret_cast<u32x4v*>((dst[c] == NONE ? junk : sbase + dst[c]) + 16u * (uint32_t)lane) = f.c[c];
    *reinterpret_cast<uint32_t*>((qdst == NONE ? junk : sbase + qdst) + 4u * (uint32_t)lane) = f.q;
  };
  constexpr int LPS = 2 + 2 * RT + CPW + 1;   // loads per step per wave

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
  //      held in registers until the epilogue ----
  //      (element by element: the chunk that holds the end of B may hold
  //      bytes past it, which read as zero)
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

  // ---- per tile: this lane's row, its two group constants and the first
  //      block (relative to the row) that uses the second (K <= 16384: a row
  //      spans at most two groups of 256 blocks); loaded first, so the wait
  //      for stage 0 covers them ----
  float d0[TR], d1[TR];
  uint32_t kb_sw[TR];
  const auto rD = rsrc(p.dscale, 4u * ((N * nbk + 255u) / 256u));
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const uint32_t n = n0 + 16u * (uint32_t)t + (uint32_t)i16;
    const uint32_t g0 = (n * nbk) >> 8;
    const bool ok = n < N;
    d0[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, ok ? 4u * g0 : OOB, 0, 0));
    d1[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rD, ok ? 4u * (g0 + 1u) : OOB, 0, 0));
    kb_sw[t] = 256u * (g0 + 1u) - n * nbk;
  }

  // ---- prologue: the first NS - 1 steps, each group of loads kept whole
  //      and in order (the waits below count loads per step) ----
  Frags<RT, CPW> f[NS];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    issue(f[i], i);
    __builtin_amdgcn_sched_barrier(0);
  }


  barrier_lds_only();   // the lookup table is complete

  const uint32_t lane4 = (uint32_t)lane * 4u;
  // LDS address of (byte e of word c, this lane's copy) = byte << 8 | lane * 4
  auto lookup = [&](uint32_t c, int e) -> uint32_t {
    const uint32_t addr = __builtin_amdgcn_perm(c, lane4, 0x0C0C0400u + ((uint32_t)e << 8));
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(lut) + addr);
  };

  f32x4_t acc[TR], tacc[RT];
#pragma unroll
  for (int t = 0; t < TR; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) tacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // block `wave` of step st for every tile; the chunk holding this lane's 16
  // codes is 2 wave + qk / 2, its 8-byte half qk % 2
  const uint32_t chunk = 2u * (uint32_t)wave + (uint32_t)(qk >> 1);
  const uint32_t half8 = 8u * (uint32_t)(qk & 1);
  auto process = [&](const Frags<RT, CPW>& f, int st) {
    if (st >= nsteps) return;
    const uint32_t kb = 8u * (uint32_t)kstep(st) + (uint32_t)wave;
    if (kb >= nbk) return;
    const uint8_t* sbase = smem + (uint32_t)(st & 1) * SL.bytes;
    // every tile's codes and scale byte first, then the lookups and MFMAs
    u32x2v cw[TR];
    uint32_t qb[TR];
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const uint32_t row = 16u * (uint32_t)t + (uint32_t)i16;
      cw[t] = *reinterpret_cast<const u32x2v*>(sbase + row * ROW_BYTES + 16u * (chunk ^ (row & 15u)) + half8);
      qb[t] = sbase[SL.qs_off + row * 8u + (uint32_t)wave];
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const float sc = __builtin_amdgcn_cvt_f32_fp8((int)qb[t], 0) * (kb < kb_sw[t] ? d0[t] : d1[t]);
      const u32x4v wa = {lookup(cw[t].x, 0), lookup(cw[t].x, 1), lookup(cw[t].x, 2), lookup(cw[t].x, 3)};
      const u32x4v wb = {lookup(cw[t].y, 0), lookup(cw[t].y, 1), lookup(cw[t].y, 2), lookup(cw[t].y, 3)};
      f32x4_t tmp = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[0], __builtin_bit_cast(bf16x8_t, wa), tmp, 0, 0, 0);
      tmp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[1], __builtin_bit_cast(bf16x8_t, wb), tmp, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] += sc * tmp[e];
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      tacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[0], f.a[rt][0], tacc[rt], 0, 0, 0);
      tacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[1], f.a[rt][1], tacc[rt], 0, 0, 0);
    }
  };

  // ---- the stream: steps in groups of NS so that the register ring is
  //      indexed by constants.  At step st the loads of steps st .. st +
  //      NS - 2 are in flight; once this wave's loads of step st have
  //      landed, it writes its codes into LDS stage st % 2, the barrier makes
  //      every wave's share visible (and guarantees that step st - 2, which
  //      used the same stage, is done everywhere), the loads of step st +
  //      NS - 1 go out into the slot after step st's, and step st is
  //      multiplied. ----
  for (int st0 = 0; st0 < nsteps; st0 += NS) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int st = st0 + i;
      wait_vm<LPS * (NS - 2)>();   // step st has landed (NS - 2 later steps may be in flight)
      stage_write(f[i], st);
      barrier_lds_only();
      __builtin_amdgcn_sched_barrier(0);
      issue(f[(i + NS - 1) % NS], st + NS - 1);
      __builtin_amdgcn_sched_barrier(0);
      process(f[i], st);           // nothing for a step past the end
    }
  }
  wait_vm<0>();

  // ---- sums over the waves (fixed order), LoRA term, store ----
  __syncthreads();   // every wave is done with the stages
  const int rt_count = (p.r + 15) / 16;
  const int TT = TR + RT;
  float* red = reinterpret_cast<float*>(smem);                 // [8 waves][TT][16 m][16 n]
  float* ttab = red + WAVES * TT * 256;                        // [16 m][MAX_R]
  u16* btab = reinterpret_cast<u16*>(ttab + 16 * MAX_R);       // B rows of the workgroup [16 TR][r]
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * TT + t) * 256 + (4 * qk + e) * 16 + i16] = acc[t][e];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(wave * TT + TR + rt) * 256 + (4 * qk + e) * 16 + i16] = tacc[rt][e];
  if ((uint32_t)tid < bchunks) *reinterpret_cast<u32x4v*>(reinterpret_cast<uint8_t*>(btab) + 16u * (uint32_t)tid) = bchunk;
  __syncthreads();
  for (int e = tid; e < 16 * MAX_R; e += NTHREADS) {
    const int m = e / MAX_R, j = e - m * MAX_R;
    float v = 0.0f;
    if (j < p.r && (j >> 4) < rt_count) {
      for (int w = 0; w < WAVES; ++w) v += red[(w * TT + TR + (j >> 4)) * 256 + m * 16 + (j & 15)];
      if (blockIdx.x == 0 && m < p.M) p.T_save[m * p.r + j] = v;
    }
    ttab[e] = v;
  }
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
    for (int w = 0; w < WAVES; ++w) base += red[(w * TT + t) * 256 + m * 16 + ci];
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

// dynamic LDS: two stages and the padding loads' target, and after the loop
// the per-wave sums [8][TR + RT][256], T [16][MAX_R] (fp32) and the
// workgroup's rows of B [16 TR][r] (bf16)
static uint32_t dyn_lds(const Plan& pl, int r) {
  const uint32_t stages = 2u * stage_layout(pl.TR).bytes + 1024u;
  const uint32_t red = 4u * ((uint32_t)WAVES * (uint32_t)(pl.TR + pl.RT) * 256u + 16u * MAX_R) +
                       32u * (uint32_t)pl.TR * (uint32_t)r;
  return std::max(stages, red);
}

template <int TR, int RT>
static hipError_t launch_one(const DecArgs& p, unsigned grid, uint32_t lds, hipStream_t st) {
  const hipError_t attr = set_dynamic_lds(reinterpret_cast<const void*>(&k_decode<TR, RT>), MAX_DYN_LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_decode<TR, RT>), dim3(grid), dim3(NTHREADS), lds, st, p);
  return hipGetLastError();
}

template <int RT>
static hipError_t launch_rt(const Plan& pl, const DecArgs& p, unsigned grid, uint32_t lds, hipStream_t st) {
  switch (pl.TR) {
    case 1: return launch_one<1, RT>(p, grid, lds, st);
    case 2: return launch_one<2, RT>(p, grid, lds, st);
    case 3: return launch_one<3, RT>(p, grid, lds, st);
    case 4: return launch_one<4, RT>(p, grid, lds, st);
    case 5: return launch_one<5, RT>(p, grid, lds, st);
    case 6: return launch_one<6, RT>(p, grid, lds, st);
    case 7: return launch_one<7, RT>(p, grid, lds, st);
    default: return hipErrorInvalidConfiguration;
  }
}

static hipError_t launch_plan(const Plan& pl, const DecArgs& p, unsigned grid, uint32_t lds, hipStream_t st) {
  return pl.RT == 2 ? launch_rt<2>(pl, p, grid, lds, st) : launch_rt<1>(pl, p, grid, lds, st);
}

}  // namespace dec

bool decode_fits(int64_t M, const NF4View& w, int r) {
  const int64_t lim = (int64_t)1 << 31;
  // 32-bit buffer offsets; K a multiple of 256 and at most 16384 (a row's
  // blocks lie in at most two groups of 256); 8-bit block scales (fp32
  // scales take the tiled path); at most two 16-rank tiles of T
  return M >= 1 && M <= 16 && r >= 1 && r <= dec::MAX_R && w.K % 256 == 0 && w.K <= 16384 &&
         !w.fp32_scale && w.N * w.K / 2 + 1024 < lim && 16 * w.K * 2 < lim && (int64_t)r * w.K * 2 < lim &&
         w.N * r * 2 < lim && w.N * (w.K / 64) + 1024 < lim;
}

hipError_t launch_decode(const NF4View& w, const u16* X, int64_t M, const u16* A, const u16* B,
                         int r, float s, u16* Y, float* T_save, hipStream_t st) {
  const dec::Plan pl = dec::plan(w.N, r);
  dec::DecArgs p;
  p.X = X; p.M = (int)M;
  p.codes = w.codes; p.qscale = w.qscale; p.dscale = w.dscale;
  p.N = (uint32_t)w.N; p.K = (uint32_t)w.K;
  for (int i = 0; i < 16; ++i) p.lv[i] = w.lv[i];
  p.A = A; p.B = B; p.r = r; p.s = s;
  p.Y = Y; p.T_save = T_save;
  const unsigned grid = (unsigned)((w.N + 16 * pl.TR - 1) / (16 * pl.TR));
  const uint32_t lds = dec::dyn_lds(pl, r);
  return dec::launch_plan(pl, p, grid, lds, st);
}

}  // namespace qln
