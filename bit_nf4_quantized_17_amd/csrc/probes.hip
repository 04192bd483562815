// probes.hip -- context kernels for the benchmark, in their own library
// (libqlora_probes.so); nothing in the QLoRA path uses them.  They measure
// what the chip itself delivers, for comparison with the path's kernels:
//   - a dense bf16 MFMA loop (v_mfma_f32_32x32x16_bf16 on register operands,
//     four independent accumulators a wave, no memory traffic), with zero or
//     with random operands (the matrix cores draw more power on random data);
//   - a streaming read of a large buffer (16-byte loads, eight in flight a
//     lane), the HBM read bandwidth a weight stream can hope for;
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

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) with grid
// workgroups of 256 threads; sink receives grid * 256 words.
int qlora_probe_read(const void* src, uint64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || bytes % 16 || ((uintptr_t)src & 15) || grid < 1) return -1;
  hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4v*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int qlora_probe_empty(void* stream) {
  hipLaunchKernelGGL(k_probe_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
