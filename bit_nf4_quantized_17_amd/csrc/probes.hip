// probes.hip -- context kernels for the benchmark, in their own library
// (libqlora_probes.so); nothing in the QLoRA path uses them.  They measure
// what the chip itself delivers, for comparison with the path's kernels:
//   - a dense bf16 MFMA loop (v_mfma_f32_32x32x16_bf16 on register operands,
//     four independent accumulators a wave, no memory traffic), with zero or
//     with random operands (the matrix cores draw more power on random data);
//   - the same MFMAs fed from LDS at the fused GEMMs' wave tile (a wave reads
//     four A and two B fragments, 16 bytes a lane each, per eight MFMAs),
//     without the dequantization, global loads or barriers around them;
//   - a streaming read of a large buffer (16-byte loads, eight in flight a
//     lane), the HBM read bandwidth a weight stream can hope for;
//   - LDS reads (16-byte ds_read a lane, eight in flight, conflict-free
//     addresses), the local-memory bandwidth that feeds the matrix cores;
//   - an empty kernel, the launch floor of a short kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlprobe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// a bf16 in [-1, 1) from a 32-bit hash (never NaN or Inf)
__device__ __forceinline__ uint16_t rnd_bf16(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  const float f = (float)(int32_t)x * 0x1p-31f;
  return (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
}

template <bool ZERO>
__global__ __launch_bounds__(256) void k_probe_mfma(float* out, int iters) {
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = ZERO ? (__bf16)0.0f : __builtin_bit_cast(__bf16, rnd_bf16(gid * 16u + (uint32_t)i));
    b[i] = ZERO ? (__bf16)0.0f : __builtin_bit_cast(__bf16, rnd_bf16(gid * 16u + 8u + (uint32_t)i));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[gid] = s;
}

// 512 threads, 64 KiB of LDS filled with random bf16 (or zeros); per
// iteration a wave does four substeps of {4 A + 2 B fragment reads, 8 MFMAs}
// into 4 x 2 accumulators, the fused GEMMs' 128 x 64 wave tile over k = 64
template <bool ZERO>
__global__ __launch_bounds__(512) void k_probe_mfma_lds(float* out, int iters) {
  __shared__ bf16x8_t buf[4096];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4096; i += 512) {
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = ZERO ? (__bf16)0.0f : __builtin_bit_cast(__bf16, rnd_bf16(8u * (uint32_t)i + (uint32_t)e));
    buf[i] = v;
  }
  __syncthreads();
  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = (f32x16_t){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int base = 384 * (4 * it + ks) + 64 * wave + lane;
      bf16x8_t fa[4], fb[2];
#pragma unroll
      for (int a = 0; a < 4; ++a) fa[a] = buf[(base + 512 * a) & 4095];
#pragma unroll
      for (int b = 0; b < 2; ++b) fb[b] = buf[(base + 2048 + 512 * b) & 4095];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += acc[a][b][i];
  out[blockIdx.x * 512 + tid] = s;
}

// each thread reads 16-byte pieces gid, gid + T, ... (T threads in the grid),
// eight loads in flight, and folds them into one word
__global__ __launch_bounds__(256) void k_probe_read(const u32x4v* src, uint64_t n16, uint32_t* sink) {
  const uint64_t T = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * T < n16; i += 8 * T) {
    u32x4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + (uint64_t)u * T);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += T) {
    const u32x4v v = src[i];
    acc ^= v.x ^ v.w;
  }
  sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// LDS read bandwidth: 512 threads, a 32 KiB buffer; a wave's 64 lanes read
// 64 consecutive 16-byte chunks (no bank conflicts), eight reads in flight.
// cyc receives each workgroup's shader-clock cycles over the read loop.
__global__ __launch_bounds__(512) void k_probe_lds(uint32_t* sink, uint64_t* cyc, int iters) {
  __shared__ u32x4v buf[2048];
  const int tid = threadIdx.x;
  for (int i = tid; i < 2048; i += 512)
    buf[i] = (u32x4v){(uint32_t)i, 3u * i, 5u * i, 7u * i};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint32_t a0 = 0, a1 = 0;
  for (int it = 0; it < iters; ++it) {
    u32x4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = buf[(tid + 256 * u + 64 * it) & 2047];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // three-input XORs: two VALU a read
      a0 = __builtin_amdgcn_bitop3_b32(a0, v[u].x, v[u].y, 0x96);
      a1 = __builtin_amdgcn_bitop3_b32(a1, v[u].z, v[u].w, 0x96);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  sink[blockIdx.x * 512 + tid] = a0 ^ a1;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

__global__ void k_probe_empty() {}

}  // namespace qlprobe

using namespace qlprobe;

extern "C" {

// MFMA loop: grid workgroups of 256 threads, iters x 4 MFMAs a wave; out
// receives grid * 256 floats.  Flops = grid * 4 waves * iters * 4 * 32768.
int qlora_probe_mfma(float* out, int iters, int zero, int grid, void* stream) {
  if (!out || iters < 1 || grid < 1) return -1;
  if (zero)
    hipLaunchKernelGGL(k_probe_mfma<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(k_probe_mfma<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// LDS-fed MFMAs: grid workgroups of 512 threads, iters x 32 MFMAs a wave;
// out receives grid * 512 floats.  Flops = grid * 8 waves * iters * 32 * 32768.
int qlora_probe_mfma_lds(float* out, int iters, int zero, int grid, void* stream) {
  if (!out || iters < 1 || grid < 1) return -1;
  if (zero)
    hipLaunchKernelGGL(k_probe_mfma_lds<true>, dim3(grid), dim3(512), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(k_probe_mfma_lds<false>, dim3(grid), dim3(512), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) with grid
// workgroups of 256 threads; sink receives grid * 256 words.
int qlora_probe_read(const void* src, uint64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || bytes % 16 || ((uintptr_t)src & 15) || grid < 1) return -1;
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4v*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// LDS reads: grid workgroups of 512 threads, iters x 8 x 16 bytes a thread;
// sink receives grid * 512 words, cyc grid cycle counts.
int qlora_probe_lds(uint32_t* sink, uint64_t* cyc, int iters, int grid, void* stream) {
  if (!sink || !cyc || iters < 1 || grid < 1) return -1;
  hipLaunchKernelGGL(k_probe_lds, dim3(grid), dim3(512), 0, (hipStream_t)stream, sink, cyc, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int qlora_probe_empty(void* stream) {
  hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
