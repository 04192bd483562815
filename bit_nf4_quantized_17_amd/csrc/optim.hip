// optim.hip -- the adapters' optimizer step: AdamW over a list of tensors in
// one launch.
//
// Ultralytics glossary "QLoRA", "How QLoRA works" (paged-optimizer bullet) and
// vnread "Grokking QLoRA", "Paged Optimizers": only the adapters train, and
// their optimizer keeps a momentum and a variance per parameter -- the state
// that QLoRA keeps in paged memory.  The pages do not write the update out;
// it is Adam with bias-corrected moments and decoupled weight decay (AdamW):
//
//   theta <- theta (1 - lr wd)
//   m     <- b1 m + (1 - b1) g,      v <- b2 v + (1 - b2) g^2
//   theta <- theta - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
//
// in fp32.  The parameter is bf16 (the adapters' storage type); with an fp32
// master copy theta is read from and written to the master and the bf16
// parameter receives its rounding, otherwise theta is the bf16 parameter.
//
// The step is a pure stream (22 bytes per parameter, 30 with a master copy),
// bound by HBM.  One workgroup handles a chunk of 2048 elements of one tensor;
// a launch covers up to MAXT tensors, the chunk table in the kernel arguments.
// Each thread takes 8 consecutive elements with 16-byte loads and stores.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "device.h"

namespace qln {
namespace opt {

constexpr int MAXT = 24;
constexpr int NTHREADS = 256;
constexpr int EPT = 8;
constexpr int64_t CHUNK = NTHREADS * EPT;

struct Tensor {
  u16* p; const u16* g; float* m; float* v; float* w; int64_t n;
};

struct Args {
  Tensor t[MAXT];
  int64_t chunk0[MAXT + 1];   // first chunk of each tensor; chunk0[count] = total
  int count;
  float b1, c1, b2, c2;       // c1 = 1 - b1, c2 = 1 - b2
  float decay;                // 1 - lr wd
  float step_size;            // lr / (1 - b1^t)
  float inv_sqrt_bc2;         // 1 / sqrt(1 - b2^t)
  float eps;
};

__device__ __forceinline__ float update(const Args& a, float theta, float g, float& m, float& v) {
  theta *= a.decay;
  m = a.b1 * m + a.c1 * g;
  v = a.b2 * v + a.c2 * (g * g);
  const float denom = __builtin_sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  return theta - a.step_size * (m / denom);
}

template <bool MASTER>
__global__ __launch_bounds__(NTHREADS) void k_adamw(Args a) {
  const int64_t c = blockIdx.x;
  int ti = 0;   // the chunk's tensor (uniform: a scalar loop over the table)
  while (ti + 1 < a.count && c >= a.chunk0[ti + 1]) ++ti;
  const Tensor& T = a.t[ti];
  const int64_t e0 = (c - a.chunk0[ti]) * CHUNK + (int64_t)threadIdx.x * EPT;
  if (e0 >= T.n) return;
  if (e0 + EPT <= T.n) {
    const uint4 pv = *reinterpret_cast<const uint4*>(T.p + e0);
    const uint4 gv = *reinterpret_cast<const uint4*>(T.g + e0);
    f32x4_t m4[2], v4[2], w4[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      m4[h] = *reinterpret_cast<const f32x4_t*>(T.m + e0 + 4 * h);
      v4[h] = *reinterpret_cast<const f32x4_t*>(T.v + e0 + 4 * h);
      if constexpr (MASTER) w4[h] = *reinterpret_cast<const f32x4_t*>(T.w + e0 + 4 * h);
    }
    const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float th[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int e = 2 * i + k, h = e >> 2, l = e & 3;
        const float th0 = MASTER ? w4[h][l] : __uint_as_float(k ? (pw[i] & 0xFFFF0000u) : (pw[i] << 16));
        const float g = __uint_as_float(k ? (gw[i] & 0xFFFF0000u) : (gw[i] << 16));
        float m = m4[h][l], v = v4[h][l];
        th[k] = update(a, th0, g, m, v);
        m4[h][l] = m;
        v4[h][l] = v;
        if constexpr (MASTER) w4[h][l] = th[k];
      }
      out[i] = pack_bf16x2(th[0], th[1]);
    }
    *reinterpret_cast<uint4*>(T.p + e0) = make_uint4(out[0], out[1], out[2], out[3]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<f32x4_t*>(T.m + e0 + 4 * h) = m4[h];
      *reinterpret_cast<f32x4_t*>(T.v + e0 + 4 * h) = v4[h];
      if constexpr (MASTER) *reinterpret_cast<f32x4_t*>(T.w + e0 + 4 * h) = w4[h];
    }
  } else {  // the tensor's ragged end
    for (int64_t e = e0; e < T.n; ++e) {
      const float th0 = MASTER ? T.w[e] : bf16_to_f32(T.p[e]);
      float m = T.m[e], v = T.v[e];
      const float th = update(a, th0, bf16_to_f32(T.g[e]), m, v);
      T.m[e] = m;
      T.v[e] = v;
      if constexpr (MASTER) T.w[e] = th;
      T.p[e] = f32_to_bf16(th);
    }
  }
}

}  // namespace opt

// Tensors with and without a master copy go to separate launches; each launch
// takes up to MAXT tensors.
hipError_t launch_adamw(const AdamwTensor* ts, int count, float lr, float b1, float b2, float eps,
                        float wd, int step, hipStream_t st) {
  opt::Args a{};
  a.b1 = b1; a.c1 = 1.0f - b1; a.b2 = b2; a.c2 = 1.0f - b2;
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  const double bc1 = 1.0 - std::pow((double)b1, (double)step);
  const double bc2 = 1.0 - std::pow((double)b2, (double)step);
  a.step_size = (float)((double)lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  a.eps = eps;
  for (int master = 0; master < 2; ++master) {
    a.count = 0;
    int64_t chunks = 0;
    auto flush = [&]() -> hipError_t {
      if (a.count == 0) return hipSuccess;
      a.chunk0[a.count] = chunks;
      if (master)
        hipLaunchKernelGGL(opt::k_adamw<true>, dim3((unsigned)chunks), dim3(opt::NTHREADS), 0, st, a);
      else
        hipLaunchKernelGGL(opt::k_adamw<false>, dim3((unsigned)chunks), dim3(opt::NTHREADS), 0, st, a);
      a.count = 0;
      chunks = 0;
      return hipGetLastError();
    };
    for (int i = 0; i < count; ++i) {
      const AdamwTensor& t = ts[i];
      if (t.n <= 0 || (t.master != nullptr) != (master == 1)) continue;
      const int64_t nc = (t.n + opt::CHUNK - 1) / opt::CHUNK;
      if (a.count == opt::MAXT || chunks + nc > 0x7fffffffLL) {
        const hipError_t e = flush();
        if (e != hipSuccess) return e;
      }
      a.t[a.count] = opt::Tensor{t.param, t.grad, t.exp_avg, t.exp_avg_sq, t.master, t.n};
      a.chunk0[a.count] = chunks;
      ++a.count;
      chunks += nc;
    }
    const hipError_t e = flush();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qln
