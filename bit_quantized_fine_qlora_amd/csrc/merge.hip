// Adapter merge: the trained adapter folded into the dequantized weight,
//   W_merged = bf16(W' + s B A)      (m x n, W' = dequant(W0) in bf16)
// "QLoRA: Efficient Fine-Tuning", Real-World Impact (adapters merged back
// into the base weight, W_merged = W0 + B A, for inference without adapter
// cost) and "QLoRA & 4-bit Fine-Tuning", Followups to expect (dequantize the
// 4-bit weight to BF16, add the adapter, keep a 16-bit model); the adapter
// carries the alpha/r scale of the LoraConfig snippet, as in the forward.
//
// Bound by HBM: 0.516 B of packed weight read and 2 B of bf16 written per
// element.  Workgroup tile: 64 rows x 128 columns, 16 rows per wave.
//   1. The rank-r product of the tile runs on MFMA 16x16x16 (bf16, fp32
//      accumulation) transposed: D[k][f] = sum_q A[q][k] B[f][q], so a lane
//      ends with 4 consecutive columns of one row; the A tile is staged in
//      LDS as [q][k] and read transposed, B comes straight from memory.
//      D goes to LDS as [f][k] fp32.
//   2. Lane (row f = lane / 4, columns 32 (lane % 4) .. + 31) dequantizes
//      its 32 weights (4 words of codes, one 16-byte load) exactly as the
//      other kernels do, adds s D with one fused multiply-add in fp32 and
//      rounds to bf16; the results are staged in the wave's LDS rows and
//      stored 4 whole rows (256 bytes each) per instruction.
// Every global load (codes, block constants, the A tile, B) is issued at the
// start, so a workgroup waits for memory once; LDS is sized to the rank.
#include "qlora_common.h"

namespace qlora {

namespace mg {
constexpr int RT = 64;    // rows per workgroup
constexpr int CT = 128;   // columns per workgroup
}  // namespace mg

typedef short s16x4v __attribute__((ext_vector_type(4)));

// Workgroup id -> (column tile, row tile).  A 128-column tile uses half of
// every 128-byte line of codes; the two tiles of a 256-column pair are given
// ids 8 apart, so they run on the same XCD (ids go round-robin over the 8
// XCDs) close in time and the second finds the line in that XCD's L2.  Needs
// an even number of column tiles and a pair count that is a multiple of 8;
// otherwise ids map in plain order.
__device__ __forceinline__ void merge_tile(int L, int gx, int gy, int& bx, int& by) {
  const int npairs = gx * gy / 2;
  if ((gx & 1) || (npairs & 7)) {
    bx = L % gx;
    by = L / gx;
    return;
  }
  const int P = (L >> 4) * 8 + (L & 7);
  const int h = (L >> 3) & 1;
  bx = 2 * (P % (gx / 2)) + h;
  by = P / (gx / 2);
}

template <int RB>   // rank blocks of 16: r <= 16 RB
__global__ __launch_bounds__(256) void merge_adapter_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ absmax8,
                                                             const float* __restrict__ c2, int64_t m, int64_t n,
                                                             int r, float s, const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, uint16_t* __restrict__ out,
                                                             Nf4Table tab) {
  constexpr int AP = 16 * RB * (mg::CT / 8);  // 16-byte pieces of the A tile
  __shared__ __align__(16) uint16_t sA[16 * RB * mg::CT];    // [q][k]
  __shared__ __align__(16) float sD[4][16][mg::CT + 4];      // per wave [f][k], rows padded by 16 bytes
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int bx, by;
  merge_tile(blockIdx.x, (int)((n + mg::CT - 1) / mg::CT), (int)((m + mg::RT - 1) / mg::RT), bx, by);
  const int64_t f0 = (int64_t)by * mg::RT;
  const int64_t k0 = (int64_t)bx * mg::CT;
  const int li = lane & 15;
  const int lg = lane >> 4;

  // ---- every global load first, so that they overlap ----
  // this lane's 32 weights (phase 2): row f, columns kc .. kc + 31
  const int rowl = lane >> 2;
  const int64_t f = f0 + 16 * wave + rowl;
  const int64_t kc = k0 + 32 * (lane & 3);
  const bool mine = f < m && kc < n;  // else the lane computes zeros that are never stored
  const uint32_t cbytes = (uint32_t)(m * n / 2);
  const brsrc_t rc = make_rsrc(codes, cbytes);
  const int64_t e0 = f * n + kc;  // a multiple of 32: one 64-weight block, one aligned 16-byte load
  const u32x4 cw = bload128(rc, mine ? (uint32_t)(e0 / 2) : cbytes);
  const int64_t blk = mine ? e0 / kBlock : 0;
  const uint8_t a8 = absmax8[blk];
  const float cg = c2[blk / kGroupBlocks];
  // A tile [q][k0 .. k0 + 127] (zeros past r or n)
  const uint32_t abytes = (uint32_t)((int64_t)r * n * 2);
  const brsrc_t ra = make_rsrc(A, abytes);
  u32x4 at[(AP + 255) / 256];
#pragma unroll
  for (int i = 0; i < (AP + 255) / 256; ++i) {
    const int p = 256 * i + tid;
    const int q = p / (mg::CT / 8);
    const int64_t k = k0 + 8 * (p % (mg::CT / 8));
    at[i] = bload128(ra, (p < AP && q < r && k < n) ? (uint32_t)(((int64_t)q * n + k) * 2) : abytes);
  }
  // B operand of every rank block: B[f0 + 16 wave + li][16 qb + 4 lg .. + 3]
  const int64_t fb = f0 + 16 * wave + li;
  s16x4v y[RB];
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
    const int q0 = 16 * qb + 4 * lg;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[qb][e] = (fb < m && q0 + e < r) ? (short)B[fb * r + q0 + e] : (short)0;
  }
#pragma unroll
  for (int i = 0; i < (AP + 255) / 256; ++i) {
    const int p = 256 * i + tid;
    if (p < AP) *reinterpret_cast<u32x4*>(sA + 8 * p) = at[i];
  }
  __syncthreads();

  // ---- D[k][f] = sum_q A[q][k] B[f][q] for this wave's 16 rows ----
  // MFMA operands (16x16x16): lane (i = lane % 16, group g = lane / 16)
  //   X[i][4g .. 4g + 3] = A[16 qb + 4g + e][k0 + 16 t + i]   (transposed read of sA)
  //   Y[4g .. 4g + 3][j] = B[f0 + 16 wave + j][16 qb + 4g + e] (y above)
  // result: lane holds D[k = 16 t + 4 g + e][f = 16 wave + lane % 16].
  f32x4 acc[mg::CT / 16];
#pragma unroll
  for (int t = 0; t < mg::CT / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int qb = 0; qb < RB; ++qb) {
#pragma unroll
    for (int t = 0; t < mg::CT / 16; ++t) {
      // lanes 4 a + c of each 16-lane group address row 16 qb + 4 g + a, columns
      // 16 t + 4 c .. + 3: the transposed read gives lane i the four values
      // A[16 qb + 4 g .. + 3][16 t + i]
      const uint16_t* src = sA + (16 * qb + 4 * lg + (li >> 2)) * mg::CT + 16 * t + 4 * (li & 3);
      const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4v, x), y[qb], acc[t], 0, 0, 0);
    }
  }
#pragma unroll
  for (int t = 0; t < mg::CT / 16; ++t)
    *reinterpret_cast<f32x4*>(&sD[wave][li][16 * t + 4 * lg]) = acc[t];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's D is in LDS
  __builtin_amdgcn_wave_barrier();

  // ---- dequantize + add + round: lane owns row f, 32 columns ----
  // All of the lane's D is read before the results go back to the same LDS
  // rows (a wave's LDS accesses run in program order), as bf16 row-major
  // [16 rows][128 columns] at the start of each row's storage.
  const float* drow = &sD[wave][rowl][32 * (lane & 3)];
  f32x4 d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) d[i] = *reinterpret_cast<const f32x4*>(drow + 4 * i);
  const MagLut L = make_mag_lut(tab, e4m3_decode(a8) * cg);
  uint8_t* orow = reinterpret_cast<uint8_t*>(&sD[wave][rowl][0]) + 64 * (lane & 3);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t o[4];
    mag_dequant8(L, cw[w], o);
    uint32_t res[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dlo = d[2 * w + (e >> 1)][2 * (e & 1)];
      const float dhi = d[2 * w + (e >> 1)][2 * (e & 1) + 1];
      const float vlo = __builtin_fmaf(s, dlo, bf16_lo_to_f32(o[e]));
      const float vhi = __builtin_fmaf(s, dhi, bf16_hi_to_f32(o[e]));
      res[e] = pack_bf16x2(vlo, vhi);
    }
    *reinterpret_cast<u32x4*>(orow + 16 * w) = u32x4{res[0], res[1], res[2], res[3]};
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the staged rows are complete
  __builtin_amdgcn_wave_barrier();
  // ---- store: each instruction writes 4 whole 256-byte row segments ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int chunk = lane & 15;
    const int64_t fr = f0 + 16 * wave + row;
    const int64_t kk = k0 + 8 * chunk;
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(&sD[wave][row][0]) + 16 * chunk);
    if (fr < m && kk < n) *reinterpret_cast<u32x4*>(out + fr * n + kk) = v;
  }
}

void launch_merge_adapter(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m, int64_t n, int r,
                          float s, const uint16_t* A, const uint16_t* B, uint16_t* out, const Nf4Table& tab,
                          hipStream_t stream) {
  const dim3 grid((unsigned)(((n + mg::CT - 1) / mg::CT) * ((m + mg::RT - 1) / mg::RT)));
  const int rb = (r + 15) / 16;
  if (rb <= 1)
    hipLaunchKernelGGL(merge_adapter_kernel<1>, grid, dim3(256), 0, stream, codes, absmax8, c2, m, n, r, s, A, B, out, tab);
  else if (rb <= 2)
    hipLaunchKernelGGL(merge_adapter_kernel<2>, grid, dim3(256), 0, stream, codes, absmax8, c2, m, n, r, s, A, B, out, tab);
  else if (rb <= 4)
    hipLaunchKernelGGL(merge_adapter_kernel<4>, grid, dim3(256), 0, stream, codes, absmax8, c2, m, n, r, s, A, B, out, tab);
  else
    hipLaunchKernelGGL(merge_adapter_kernel<8>, grid, dim3(256), 0, stream, codes, absmax8, c2, m, n, r, s, A, B, out, tab);
}

}  // namespace qlora
