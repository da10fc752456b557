// Blockwise NF4 quantizer with double quantization, and the bf16 dequantizer.
//
// Method: "QLoRA: Efficient Fine-Tuning", Step 1 (Eq. 1 normalization by the
// block absmax, Eq. 2 normal-quantile levels, snap to the nearest level) and
// Step 2 (double quantization of the absmax constants to an 8-bit float in
// blocks of 256); block size 64 from "What is QLoRA?" ("The three pieces")
// and "QLoRA & 4-bit Fine-Tuning" (Innovation 2).
#include "qlora_common.h"

namespace qlora {

// fl32(w / c) for |w| <= c, c in [2^-100, 2^100], |w| >= 2^-100, with y the
// correctly rounded 1/c.  q0 = RN(w y) is within one ulp of w / c, the
// remainder w - c q0 is exact (one fused multiply-add), and one more fused
// step RN(q0 + r y) is the correctly rounded quotient (Markstein's theorem
// for reciprocal-based division).
__device__ __forceinline__ float div_by_block_absmax(float w, float c, float y) {
  const float q0 = w * y;
  const float r0 = __builtin_fmaf(-c, q0, w);
  return __builtin_fmaf(r0, y, q0);
}

// Stored code of the level nearest to v: the level index is the number of
// thresholds strictly below v.  With the symmetric table this is computed on
// |v| against the 7 positive thresholds, as integers (bit patterns of
// non-negative floats order like the floats):
//   v > 0 : level 8 + #{T_j < v}        -> code #{T_j < |v|}
//   v <= 0: level 7 - #{T_j <= |v|}     -> code 8 + #{T_j < succ(|v|)}
// (succ(|v|) is |v|'s bit pattern + 1).  v <= 0 is read off the sign bit, so
// a zero quotient must arrive as -0 (both zeros take level 7, like any v <= 0
// with |v| below the first positive threshold).
//
// The count uses a 1024-entry table over the bit patterns of |v| in [0, 1]:
// entry i covers the patterns [i * 2^20, (i + 1) * 2^20) (an eighth of a
// binade) and holds the number of thresholds below its start and the one
// threshold inside it, if any (no interval holds two, and none lies below
// 2^-4; the host-side table build checks both).  The index is bits 20..29 of
// v (|v| = 1 is entry 1016), so the lookup needs no clamp.  The key succ(|v|)
// may fall in the next interval, but only at its very first pattern, which
// no threshold of the current entry can reach, so base + [key > thr] is
// still the count.
constexpr int kCodeLutSize = 1024;

__device__ __forceinline__ uint32_t nf4_code(float v, const uint2* lut) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t neg = bits >> 31;
  const uint32_t key = (bits & 0x7FFFFFFFu) + neg;
  const uint2 e = lut[(bits >> 20) & (kCodeLutSize - 1)];
  return (e.x + (key > e.y ? 1u : 0u)) | (neg << 3);
}

// One workgroup per double-quant group (256 blocks of 64 weights).  In each
// of four passes a quad of lanes covers one block, 16 consecutive weights per
// lane (four 16-byte loads), so a wave reads 4 KB of contiguous weights.
__global__ __launch_bounds__(256) void quantize_nf4_dq_kernel(const float* __restrict__ W, int64_t nblk,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ absmax8,
                                                               float* __restrict__ c2out, Nf4Table tab) {
  __shared__ float s_c1[kGroupBlocks];
  __shared__ float s_red[4];
  __shared__ uint2 s_lut[kCodeLutSize];
  const int tid = threadIdx.x;
  const int64_t blk0 = (int64_t)blockIdx.x * kGroupBlocks;
  const int nb = (int)((nblk - blk0) < kGroupBlocks ? (nblk - blk0) : kGroupBlocks);
  for (int i = tid; i < kCodeLutSize; i += 256) {
    const uint32_t lo = (uint32_t)i << 20;
    const uint32_t hi = lo + (1u << 20);
    uint32_t below = 0, inside = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const uint32_t t = __float_as_uint(tab.t[8 + j]);
      below += t < lo ? 1u : 0u;
      if (t >= lo && t < hi) inside = t;
    }
    s_lut[i] = make_uint2(below, inside);
  }
  __syncthreads();

  // The next pass's 64 bytes per lane are loaded before this pass's
  // arithmetic, so each lane keeps two passes of loads in flight.
  float4 wq[2][4];
  auto load_pass = [&](int pass, float4 (&dst)[4]) {
    const int lb = pass * 64 + (tid >> 2);
    if (lb < nb) {
      const float4* src = reinterpret_cast<const float4*>(W + (blk0 + lb) * kBlock + (tid & 3) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_pass(0, wq[0]);
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int lb = pass * 64 + (tid >> 2);
    const int quarter = tid & 3;
    const bool valid = lb < nb;
    if (pass + 1 < 4) load_pass(pass + 1, wq[(pass + 1) & 1]);
    float w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 t = wq[pass & 1][i];
      w[4 * i + 0] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(w[i]));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    const float c1 = a;
    if (valid && quarter == 0) s_c1[lb] = c1;

    // Fast path needs every quotient away from underflow (the division's
    // residual is exact for |w| >= 2^-100 and c1 in [2^-100, 2^100], and
    // |w| >= c1 2^-125 keeps w / c1 a normal number, never 0); anything else
    // (zeros, tiny weights, tiny or huge constants) takes the IEEE division,
    // and a zero quotient there is passed on as -0 (see nf4_code).
    float amin = fabsf(w[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) amin = fminf(amin, fabsf(w[i]));
    const bool slow = !(c1 >= 0x1p-100f && c1 <= 0x1p100f) || !(amin >= 0x1p-100f) || !(amin >= c1 * 0x1p-125f);
    float q[16];
    if (!slow) {
      const float y = 1.0f / c1;
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = div_by_block_absmax(w[i], c1, y);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = (c1 > 0.0f) ? w[i] / c1 : 0.0f;
        q[i] = v == 0.0f ? -0.0f : v;
      }
    }
    // pack: per 8 weights, byte j = code(w_j) | code(w_{j+4}) << 4
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= (nf4_code(q[j], s_lut) | (nf4_code(q[j + 4], s_lut) << 4)) << (8 * j);
      hi |= (nf4_code(q[8 + j], s_lut) | (nf4_code(q[12 + j], s_lut) << 4)) << (8 * j);
    }
    if (valid) {
      u32x2 pk = {lo, hi};
      *reinterpret_cast<u32x2*>(codes + (blk0 + lb) * (kBlock / 2) + quarter * 8) = pk;
    }
  }
  __syncthreads();

  // c2 = max of the group's c1; then each block's constant as E4M3(c1 / c2).
  float c1 = tid < nb ? s_c1[tid] : 0.0f;
  float m = c1;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) s_red[tid >> 6] = m;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  if (tid < nb) {
    const uint32_t code = c2 > 0.0f ? e4m3_encode_unit(c1 / c2) : 0u;
    absmax8[blk0 + tid] = (uint8_t)code;
  }
  if (tid == 0) c2out[blockIdx.x] = c2;
}

// W' = bf16(fl32(Q[code] * s_b)) for 8 consecutive weights per thread.
__global__ __launch_bounds__(256) void dequant_nf4_dq_kernel(const uint32_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ absmax8,
                                                              const float* __restrict__ c2, int64_t nwords,
                                                              u32x4* __restrict__ out, Nf4Table tab) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int64_t blk = i >> 3;  // 8 words of codes per 64-weight block
  const MagLut L = make_mag_lut(tab, block_scale(absmax8, c2, blk));
  uint32_t o[4];
  mag_dequant8(L, codes[i], o);
  out[i] = u32x4{o[0], o[1], o[2], o[3]};
}

void launch_quantize(const float* W, int64_t numel, uint8_t* codes, uint8_t* absmax8, float* c2,
                     const Nf4Table& tab, hipStream_t stream) {
  const int64_t nblk = numel / kBlock;
  const int64_t ngrp = (nblk + kGroupBlocks - 1) / kGroupBlocks;
  hipLaunchKernelGGL(quantize_nf4_dq_kernel, dim3((unsigned)ngrp), dim3(256), 0, stream, W, nblk, codes, absmax8,
                     c2, tab);
}

void launch_dequant(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t numel, uint16_t* out,
                    const Nf4Table& tab, hipStream_t stream) {
  const int64_t nwords = numel / 8;
  const int64_t grid = (nwords + 255) / 256;
  hipLaunchKernelGGL(dequant_nf4_dq_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint32_t*>(codes), absmax8, c2, nwords, reinterpret_cast<u32x4*>(out),
                     tab);
}

}  // namespace qlora
