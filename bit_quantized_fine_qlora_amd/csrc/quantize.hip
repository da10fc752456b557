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
//   v <= 0: level 7 - #{T_j <= |v|}     -> code 8 + #{T_j <= |v|}
// v <= 0 is read off the sign bit, so a zero quotient must arrive as -0
// (both zeros take level 7, like any v <= 0 with |v| below the first
// positive threshold).
//
// The count uses a table over the bit patterns of v in [-1, 1], in two
// halves by the sign bit.  Entry i of a half covers the |v| patterns
// [i * 2^20, (i + 1) * 2^20) (an eighth of a binade) and holds the code of
// the interval's start and the one threshold inside it, if any (no interval
// holds two, and none lies below 2^-4; the host-side table build checks
// both), as the full bit pattern above which v takes the next code: T for
// v > 0, and sign | (T - 1) for v <= 0, so that one unsigned compare of v's
// own bits gives T < |v| or T <= |v| respectively.  The byte offset of the
// entry is bits 17..29 and 31 of v masked to 8-byte steps: bit 31 selects
// the half (16 KB apart), and bit 30 is 0 for |v| <= 1 (|v| = 1 is entry
// 1016), so the lookup needs no clamp.
constexpr int kCodeLutSize = 1024;              // entries per sign
constexpr int kCodeLutFirst = 0x3D800000 >> 20; // the entry of 2^-4
constexpr uint32_t kCodeLutMask = 0x5FF8u;      // (bits >> 17) & mask = byte offset
constexpr int kCodeLutNegBase = 2048;           // first entry of the v <= 0 half

__device__ __forceinline__ uint32_t nf4_code(float v, const uint2* lut) {
  const uint32_t bits = __float_as_uint(v);
  const uint2 e = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(lut) + ((bits >> 17) & kCodeLutMask));
  return e.x + (bits > e.y ? 1u : 0u);
}

// Maximum over the 8 lanes 8k .. 8k + 7 by three DPP butterfly steps
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror).
__device__ __forceinline__ float oct_max(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xF, 0xF, false)));
  return a;
}

// v | (the same value of the neighbouring lane, lane ^ 1).
__device__ __forceinline__ uint32_t or_lane_pair(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// q = fl32(w / c1) for 8 weights of one block.  The fast path needs every
// quotient away from underflow (the division's residual is exact for
// |w| >= 2^-100 and c1 in [2^-100, 2^100], and |w| >= c1 2^-125 keeps w / c1
// a normal number, never 0); anything else (zeros, tiny weights, tiny or huge
// constants) takes the IEEE division, and a zero quotient there is passed on
// as -0 (see nf4_code).  The choice is per lane: both paths give the same
// quotients where both apply.
__device__ __forceinline__ void block_quotients(const float* w, float c1, float* q) {
  float amin = fabsf(w[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) amin = fminf(amin, fabsf(w[i]));
  const bool slow = !(c1 >= 0x1p-100f && c1 <= 0x1p100f) || !(amin >= 0x1p-100f) || !(amin >= c1 * 0x1p-125f);
  if (!slow) {
    const float y = 1.0f / c1;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_by_block_absmax(w[i], c1, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = (c1 > 0.0f) ? w[i] / c1 : 0.0f;
      q[i] = v == 0.0f ? -0.0f : v;
    }
  }
}

constexpr int kAuxNonTemporal = 2;  // buffer access cache policy: nt

// One workgroup per double-quant group (256 blocks of 64 weights), in four
// passes of 64 blocks.  Per pass each wave takes 16 consecutive blocks (4 KB),
// 8 lanes to a pair of blocks: lane t of lane octet g reads the 16 bytes at
// t * 16 of each 128-byte half of blocks 2g and 2g + 1, so every 16-byte load
// of the wave covers eight whole 128-byte lines, and each lane holds 8
// weights of each of its two blocks (weights 4t .. 4t + 3 and 32 + 4t ..
// 32 + 4t + 3).  The loads are non-temporal (the weight is read once) and
// go through buffer resources with the group's byte range, so the partial
// last group reads zeros and drops its stores past the end.  Block maxima come
// from DPP steps over the octet; the 4 codes of a lane's 4 consecutive
// weights fill one nibble of each byte of a code word and the neighbouring
// lane the other (weights 8p .. 8p + 3 low, 8p + 4 .. 8p + 7 high), merged
// by one DPP exchange; even lanes store the first block's words, odd lanes
// the second's.
//
// One launch serves up to kMaxQuantWeights weights: workgroup b takes group
// b - grp_end[i - 1] of the weight i with grp_end[i - 1] <= b < grp_end[i]
// (grp_end[-1] = 0), so weights too small to fill the chip alone share it.
constexpr int kMaxQuantWeights = 8;
struct QuantArgs {
  const float* W[kMaxQuantWeights];
  uint8_t* codes[kMaxQuantWeights];
  uint8_t* absmax8[kMaxQuantWeights];
  float* c2[kMaxQuantWeights];
  int64_t nblk[kMaxQuantWeights];
  int32_t grp_end[kMaxQuantWeights];  // groups of weights 0 .. i together
  int32_t count;
};

__global__ __launch_bounds__(256) void quantize_nf4_dq_kernel(QuantArgs qa, Nf4Table tab) {
  // code table (both halves) with the block constants and the group
  // maximum in the gap between the halves
  __shared__ uint2 s_lut[kCodeLutNegBase + kCodeLutSize];
  float* s_c1 = reinterpret_cast<float*>(s_lut + kCodeLutSize);
  float* s_red = s_c1 + kGroupBlocks;
  const int tid = threadIdx.x;
  const int bid = (int)blockIdx.x;
  int wi = 0;
#pragma unroll
  for (int i = 0; i + 1 < kMaxQuantWeights; ++i) wi += (i + 1 < qa.count && bid >= qa.grp_end[i]) ? 1 : 0;
  const float* __restrict__ W = qa.W[wi];
  uint8_t* __restrict__ codes = qa.codes[wi];
  uint8_t* __restrict__ absmax8 = qa.absmax8[wi];
  const int64_t nblk = qa.nblk[wi];
  const int grp = bid - (wi ? qa.grp_end[wi - 1] : 0);
  const int64_t blk0 = (int64_t)grp * kGroupBlocks;
  const int nb = (int)((nblk - blk0) < kGroupBlocks ? (nblk - blk0) : kGroupBlocks);
  const int lane = tid & 63, wave = tid >> 6;
  const int oct = lane >> 3, t = lane & 7;
  const brsrc_t wr = make_rsrc(W + blk0 * kBlock, (uint32_t)nb * kBlock * 4u);
  const brsrc_t cr = make_rsrc(codes + blk0 * (kBlock / 2), (uint32_t)nb * (kBlock / 2));
  auto load_pass = [&](int pass, u32x4 (&dst)[4]) {
    const uint32_t base = (uint32_t)(pass * 64 + wave * 16 + oct * 2) * kBlock * 4u + (uint32_t)t * 16u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dst[k] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, (int)(base + (uint32_t)k * 128u), 0, kAuxNonTemporal));
  };
  // the first pass's loads are in flight while the table is built; the
  // next pass's are issued before each pass's arithmetic
  u32x4 wq[2][4];
  load_pass(0, wq[0]);
  for (int i = tid; i < kCodeLutSize; i += 256) {
    uint32_t below = 0, inside = 0xFFFFFFFFu;
    if (i >= kCodeLutFirst) {  // below 2^-4: no threshold below or inside
      const uint32_t lo = (uint32_t)i << 20;
      const uint32_t hi = lo + (1u << 20);
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const uint32_t th = __float_as_uint(tab.t[8 + j]);
        below += th < lo ? 1u : 0u;
        if (th >= lo && th < hi) inside = th;
      }
    }
    s_lut[i] = make_uint2(below, inside);
    s_lut[kCodeLutNegBase + i] = make_uint2(8u + below, inside == 0xFFFFFFFFu ? inside : (0x80000000u | (inside - 1u)));
  }
  __syncthreads();

#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (pass + 1 < 4) load_pass(pass + 1, wq[(pass + 1) & 1]);
    const int lb = pass * 64 + wave * 16 + oct * 2;  // first of the octet's two blocks
    // w[0..7]: block lb, w[8..15]: block lb + 1
    float w[16];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * k + e] = __uint_as_float(wq[pass & 1][k][e]);
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a0 = fmaxf(a0, fabsf(w[i]));
      a1 = fmaxf(a1, fabsf(w[8 + i]));
    }
    a0 = oct_max(a0);
    a1 = oct_max(a1);
    if (t == 0 && lb < nb) s_c1[lb] = a0;
    if (t == 1 && lb + 1 < nb) s_c1[lb + 1] = a1;
    float q[16];
    block_quotients(w, a0, q);
    block_quotients(w + 8, a1, q + 8);
    // p[k]: the codes of the 4 weights of load k in the bytes of one word
    uint32_t p[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[k] |= nf4_code(q[4 * k + j], s_lut) << (8 * j);
    const uint32_t nib = (uint32_t)(t & 1) * 4u;
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = or_lane_pair(p[k] << nib);
    // p[0], p[1]: words t/2 and 4 + t/2 of block lb; p[2], p[3]: of lb + 1
    const bool odd = (t & 1) != 0;
    const uint32_t off = (uint32_t)(lb + (odd ? 1 : 0)) * (kBlock / 2) + (uint32_t)(t >> 1) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(odd ? p[2] : p[0], cr, (int)off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(odd ? p[3] : p[1], cr, (int)(off + 16u), 0, 0);
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
  if (tid == 0) qa.c2[wi][grp] = c2;
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

// Weights 0 .. count - 1 (count 1 .. kMaxQuantWeights), each of numel
// elements (a multiple of 64), in one launch.
struct QuantWeight {
  const float* W;
  int64_t numel;
  uint8_t* codes;
  uint8_t* absmax8;
  float* c2;
};

int max_quant_weights() { return kMaxQuantWeights; }

// Groups of a weight of numel elements.
int64_t quant_groups(int64_t numel) { return (numel / kBlock + kGroupBlocks - 1) / kGroupBlocks; }

void launch_quantize_grouped(const QuantWeight* w, int count, const Nf4Table& tab, hipStream_t stream) {
  QuantArgs qa{};
  int64_t total = 0;
  for (int i = 0; i < count; ++i) {
    qa.W[i] = w[i].W;
    qa.codes[i] = w[i].codes;
    qa.absmax8[i] = w[i].absmax8;
    qa.c2[i] = w[i].c2;
    qa.nblk[i] = w[i].numel / kBlock;
    total += quant_groups(w[i].numel);
    qa.grp_end[i] = (int32_t)total;
  }
  qa.count = count;
  hipLaunchKernelGGL(quantize_nf4_dq_kernel, dim3((unsigned)total), dim3(256), 0, stream, qa, tab);
}

void launch_quantize(const float* W, int64_t numel, uint8_t* codes, uint8_t* absmax8, float* c2,
                     const Nf4Table& tab, hipStream_t stream) {
  const QuantWeight w{W, numel, codes, absmax8, c2};
  launch_quantize_grouped(&w, 1, tab, stream);
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
