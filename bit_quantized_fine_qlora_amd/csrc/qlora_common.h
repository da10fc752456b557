// Shared device-side definitions for the QLoRA HIP kernels (gfx950 only).
//
// Data layout (row-major everywhere):
//   W0      m x n fp32 (out x in); quantized in 64-element blocks that run
//           along n, 256 blocks (16384 elements) per double-quant group.
//   codes   m*n/2 bytes: sign-magnitude 4-bit codes (see MagLut), per 8
//           weights byte j = weight j (low nibble) | weight j+4 (high nibble).
//   absmax8 m*n/64 bytes, E4M3FN code of c1_b / c2_g.
//   c2      ceil(m*n/16384) fp32.
//   x M x n, g M x m, A r x n, B m x r, h M x m, grad_x M x n: bf16 bits.
//   u = x A^T and v = g B: M x r fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Host: compute units of the current device (cached per device).
int device_cus();

constexpr int kBlock = 64;        // weights per absmax block
constexpr int kGroupBlocks = 256; // blocks per double-quant group
constexpr int kMaxRank = 128;

// NF4 levels (16, ascending, spanning [-1, 1]) and the 15 midpoints between
// them, passed by value in kernel arguments.
struct Nf4Table {
  float q[16];
  float t[15];
};

// E4M3FN (bias 7, 3 mantissa bits) to fp32.  Only non-negative finite codes
// occur on this path; the value is exact in fp32.  gfx950's fp8 convert reads
// the OCP E4M3FN format; on codes 0x00 .. 0x7e (subnormals included) it gives
// the same bits as the field-by-field decode (normal: 2^(e-7) (1 + m/8),
// subnormal: m 2^-9), checked exhaustively on the device.
__device__ __forceinline__ float e4m3_decode(uint32_t a) {
  return __builtin_amdgcn_cvt_f32_fp8((int)a, 0);
}

// Round-to-nearest-even E4M3FN code of v in [0, 1] (no saturation needed).
__device__ __forceinline__ uint32_t e4m3_encode_unit(float v) {
  if (!(v > 0.0f)) return 0u;
  const uint32_t b = __float_as_uint(v);
  int e = (int)(b >> 23) - 127;
  if (e < -6) {  // subnormal codes are multiples of 2^-9; 8 carries into 0x08
    return (uint32_t)__builtin_rintf(v * 512.0f);
  }
  const uint32_t mant = b & 0x7FFFFFu;
  uint32_t top = mant >> 20;
  const uint32_t rest = mant & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (top & 1u))) {
    ++top;
    if (top == 8u) { top = 0u; ++e; }
  }
  return ((uint32_t)(e + 7) << 3) | top;
}

// Per-block scale s_b = fl32(dec(a_b) * c2_g).
__device__ __forceinline__ float block_scale(const uint8_t* absmax8, const float* c2, int64_t blk) {
  return e4m3_decode(absmax8[blk]) * c2[blk >> 8];
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even (v_cvt_pk_bf16_f32)
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Stored 4-bit code of an NF4 level L (0..15): bit 3 = sign (set for the 8
// negative levels), bits 0-2 = rank of |level| among the 8 positive levels
// (code = L - 8 for L >= 8, 15 - L for L < 8; the levels are symmetric).  In
// each 32-bit word of codes (8 consecutive weights), byte j holds weight j
// in its low nibble and weight j + 4 in its high nibble.
//
// Magnitude table of one block: entry k (0..7) is bf16(fl32(Q[8+k] * s)).
// Since Q[15-k'] = -Q[k'] exactly and both roundings are sign-symmetric, a
// weight dequantizes to its entry with the code's sign bit copied into the
// bf16 sign (which also gives -0.0 for a zero scale, as bf16(fl32(Q * 0))
// does for a negative level).  lo[i] / hi[i] hold the low / high bytes of
// entries 4i..4i+3.
struct MagLut {
  uint32_t lo[2];
  uint32_t hi[2];
};

__device__ __forceinline__ MagLut make_mag_lut(const Nf4Table& tab, float s) {
  uint32_t pr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pr[k] = pack_bf16x2(tab.q[8 + 2 * k] * s, tab.q[9 + 2 * k] * s);
  MagLut L;
  L.lo[0] = __builtin_amdgcn_perm(pr[1], pr[0], 0x06040200u);
  L.hi[0] = __builtin_amdgcn_perm(pr[1], pr[0], 0x07050301u);
  L.lo[1] = __builtin_amdgcn_perm(pr[3], pr[2], 0x06040200u);
  L.hi[1] = __builtin_amdgcn_perm(pr[3], pr[2], 0x07050301u);
  return L;
}

// Dequantize one 32-bit word of codes (8 weights) into 4 words of bf16
// pairs in weight order (w0,w1) (w2,w3) (w4,w5) (w6,w7): 14 VALU ops.
__device__ __forceinline__ void mag_dequant8(const MagLut& L, uint32_t w, uint32_t out[4]) {
  const uint32_t s03 = w & 0x07070707u;          // ranks of weights 0..3 (low nibbles)
  const uint32_t s47 = (w >> 4) & 0x07070707u;   // ranks of weights 4..7 (high nibbles)
  const uint32_t L03 = __builtin_amdgcn_perm(L.lo[1], L.lo[0], s03);
  const uint32_t L47 = __builtin_amdgcn_perm(L.lo[1], L.lo[0], s47);
  const uint32_t H03 = __builtin_amdgcn_perm(L.hi[1], L.hi[0], s03) | ((w << 4) & 0x80808080u);
  const uint32_t H47 = __builtin_amdgcn_perm(L.hi[1], L.hi[0], s47) | (w & 0x80808080u);
  out[0] = __builtin_amdgcn_perm(H03, L03, 0x05010400u);
  out[1] = __builtin_amdgcn_perm(H03, L03, 0x07030602u);
  out[2] = __builtin_amdgcn_perm(H47, L47, 0x05010400u);
  out[3] = __builtin_amdgcn_perm(H47, L47, 0x07030602u);
}


// LoRA dropout on the adapter input ("QLoRA: Efficient Fine-Tuning", the
// LoraConfig snippet's lora_dropout).  Element e of a row-major tensor takes
// word e % 4 of Philox4x32-10 at the 64-bit counter e / 4 + offset (upper two
// counter words zero) under the key (seed low, seed high), and is kept when
// that word is at least thr = round(p 2^32).  Philox4x32-10 as defined by
// Salmon, Moraes, Dror and Shaw (SC 2011): per round the counter words 0 and
// 2 are multiplied by two constants and the halves mixed with the key, which
// takes two Weyl increments between rounds.
struct DropoutDev {
  uint32_t thr;       // 0: keep everything
  uint32_t k0, k1;    // key (seed)
  uint64_t offset;    // counter offset
  int on;             // apply the mask at all
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
  }
  return u32x4{c0, c1, c2, c3};
}

// 8 consecutive bf16 elements e0 .. e0 + 7 (e0 % 4 == 0, two bf16 per word,
// element order) with the dropped ones set to zero.
__device__ __forceinline__ u32x4 dropout8(const DropoutDev& d, uint64_t e0, u32x4 w) {
  const uint64_t c = (e0 >> 2) + d.offset;
  const u32x4 r0 = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), d.k0, d.k1);
  const uint64_t c1 = c + 1;
  const u32x4 r1 = philox4x32_10((uint32_t)c1, (uint32_t)(c1 >> 32), d.k0, d.k1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = (j < 2 ? r0[2 * j] : r1[2 * j - 4]) >= d.thr ? 0x0000FFFFu : 0u;
    const uint32_t hi = (j < 2 ? r0[2 * j + 1] : r1[2 * j - 3]) >= d.thr ? 0xFFFF0000u : 0u;
    w[j] &= lo | hi;
  }
  return w;
}

// Raw buffer access with a byte range: lanes whose offset is past `bytes`
// read 0 instead of touching memory.  All offsets go in the per-lane VGPR
// offset (the range check covers it).
typedef __amdgpu_buffer_rsrc_t brsrc_t;

__device__ __forceinline__ brsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(brsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bload32(brsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(brsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Split an fp32 value into bf16 hi + lo with hi + lo equal to v to ~2^-16.
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  const float h = (float)(__bf16)v;
  hi = h;
  lo = v - h;
}

// Words a GEMM's K-split hand-off needs at zero when it starts (its arrival
// counts, ready flags and give-up word), cleared by the kernel that runs just
// before the GEMM in the same call, so the GEMM needs no clearing launch.
struct SyncZero {
  uint32_t* p = nullptr;
  int n = 0;
};

}  // namespace qlora
