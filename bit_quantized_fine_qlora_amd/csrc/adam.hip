// Adapter optimizer step: Adam with decoupled weight decay, fused over many
// tensors (for example A and B of every adapted layer) in one launch.
// "QLoRA: Efficient Fine-Tuning", memory-layout figure (Adam moments kept for
// the adapters only, paged to CPU memory when the GPU runs out) and "What is
// QLoRA?", Worked example (fp32 parameter, gradient and both moments: 16
// bytes per trainable parameter); paging from "QLoRA & 4-bit Fine-Tuning",
// Innovation 3.
//
// Per element, in fp32 (host-side constants from the step number in double):
//   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
//   p <- p - (lr / (1 - b1^t)) m / (sqrt(v / (1 - b2^t)) + eps)
// g is the bf16 gradient the backward writes; the fp32 master p, m and v are
// updated in place and, when asked, the bf16 copy of p that the forward and
// backward read.  Bound by memory: 28 bytes per element (p, m, v read and
// written, g read, the bf16 copy written).  The state may live in host
// memory the GPU can address (pinned host allocations): the same kernel then
// streams it over the host link, which is how paged-out state is updated.
#include <cmath>

#include "qlora_common.h"

namespace qlora {

constexpr int kAdamMaxTensors = 64;  // per launch; the table travels in the kernel arguments (< 4 KB)

struct AdamTensorDev {
  int64_t count;
  float* p;
  uint16_t* p16;        // may be null
  const uint16_t* g;
  float* m;
  float* v;
};

struct AdamArgs {
  AdamTensorDev t[kAdamMaxTensors];
  int wg_begin[kAdamMaxTensors + 1];  // first workgroup of each tensor (prefix sums)
  int count;
  float decay;      // 1 - lr wd
  float b1, c1;     // beta1, 1 - beta1
  float b2, c2;     // beta2, 1 - beta2
  float step_size;  // lr / (1 - beta1^t)
  float inv_bc2;    // 1 / (1 - beta2^t)
  float eps;
};

__device__ __forceinline__ float adam_one(const AdamArgs& a, float& p, float& m, float& v, float g) {
  p *= a.decay;
  m = __builtin_fmaf(a.b1, m, a.c1 * g);
  v = __builtin_fmaf(a.b2, v, a.c2 * g * g);
  const float denom = __builtin_sqrtf(v * a.inv_bc2) + a.eps;
  p -= a.step_size * (m / denom);
  return p;
}

// One thread per 8 consecutive elements; every workgroup belongs to one
// tensor (found by a search over the workgroup prefix sums, the same for the
// whole workgroup).
__global__ __launch_bounds__(256) void adam_step_kernel(AdamArgs a) {
  const int wg = (int)blockIdx.x;
  int lo = 0, hi = a.count;  // wg_begin[lo] <= wg < wg_begin[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.wg_begin[mid] <= wg) lo = mid; else hi = mid;
  }
  const AdamTensorDev& T = a.t[lo];
  const int64_t e0 = ((int64_t)(wg - a.wg_begin[lo]) * 256 + threadIdx.x) * 8;
  if (e0 >= T.count) return;
  if (e0 + 8 <= T.count) {
    const f32x4 p0 = *reinterpret_cast<const f32x4*>(T.p + e0), p1 = *reinterpret_cast<const f32x4*>(T.p + e0 + 4);
    const f32x4 m0 = *reinterpret_cast<const f32x4*>(T.m + e0), m1 = *reinterpret_cast<const f32x4*>(T.m + e0 + 4);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(T.v + e0), v1 = *reinterpret_cast<const f32x4*>(T.v + e0 + 4);
    const u32x4 gw = *reinterpret_cast<const u32x4*>(T.g + e0);
    float pp[8], mm[8], vv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pp[j] = p0[j]; pp[j + 4] = p1[j];
      mm[j] = m0[j]; mm[j + 4] = m1[j];
      vv[j] = v0[j]; vv[j + 4] = v1[j];
    }
    uint32_t out16[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = adam_one(a, pp[2 * j], mm[2 * j], vv[2 * j], bf16_lo_to_f32(gw[j]));
      const float a1 = adam_one(a, pp[2 * j + 1], mm[2 * j + 1], vv[2 * j + 1], bf16_hi_to_f32(gw[j]));
      out16[j] = pack_bf16x2(a0, a1);
    }
    *reinterpret_cast<f32x4*>(T.p + e0) = f32x4{pp[0], pp[1], pp[2], pp[3]};
    *reinterpret_cast<f32x4*>(T.p + e0 + 4) = f32x4{pp[4], pp[5], pp[6], pp[7]};
    *reinterpret_cast<f32x4*>(T.m + e0) = f32x4{mm[0], mm[1], mm[2], mm[3]};
    *reinterpret_cast<f32x4*>(T.m + e0 + 4) = f32x4{mm[4], mm[5], mm[6], mm[7]};
    *reinterpret_cast<f32x4*>(T.v + e0) = f32x4{vv[0], vv[1], vv[2], vv[3]};
    *reinterpret_cast<f32x4*>(T.v + e0 + 4) = f32x4{vv[4], vv[5], vv[6], vv[7]};
    if (T.p16) *reinterpret_cast<u32x4*>(T.p16 + e0) = u32x4{out16[0], out16[1], out16[2], out16[3]};
  } else {
    for (int64_t e = e0; e < T.count; ++e) {
      float p = T.p[e], m = T.m[e], v = T.v[e];
      const float g = __uint_as_float((uint32_t)T.g[e] << 16);
      adam_one(a, p, m, v, g);
      T.p[e] = p;
      T.m[e] = m;
      T.v[e] = v;
      if (T.p16) T.p16[e] = (uint16_t)(pack_bf16x2(p, 0.0f) & 0xFFFFu);
    }
  }
}

struct AdamTensorHost {
  int64_t count;
  float* p;
  uint16_t* p16;
  const uint16_t* g;
  float* m;
  float* v;
};

// Up to kAdamMaxTensors tensors per launch; the caller splits longer lists.
void launch_adam_step(const AdamTensorHost* ts, int count, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int64_t step, hipStream_t stream) {
  AdamArgs a{};
  a.count = count;
  a.wg_begin[0] = 0;
  for (int i = 0; i < count; ++i) {
    a.t[i] = AdamTensorDev{ts[i].count, ts[i].p, ts[i].p16, ts[i].g, ts[i].m, ts[i].v};
    a.wg_begin[i + 1] = a.wg_begin[i] + (int)((ts[i].count + 8 * 256 - 1) / (8 * 256));
  }
  for (int i = count; i < kAdamMaxTensors; ++i) a.wg_begin[i + 1] = a.wg_begin[count];
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  a.b1 = beta1;
  a.c1 = (float)(1.0 - (double)beta1);
  a.b2 = beta2;
  a.c2 = (float)(1.0 - (double)beta2);
  a.step_size = (float)((double)lr / bc1);
  a.inv_bc2 = (float)(1.0 / bc2);
  a.eps = eps;
  hipLaunchKernelGGL(adam_step_kernel, dim3((unsigned)a.wg_begin[count]), dim3(256), 0, stream, a);
}

}  // namespace qlora
