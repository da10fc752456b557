// Input gradient of the adapted linear layer through the frozen 4-bit weight:
//   grad_x = g W' + s v A,  v = g B  (v comes in precomputed, fp32)
// "QLoRA: Efficient Fine-Tuning", Step 4: gradients flow through the frozen
// quantized W0 (dequantized to BF16) while W0 itself gets none; the s v A
// term is the chain rule of the scaled adapter branch of Eq. 3.
//
// The contraction runs over the out-features f, which is the strided index
// of W' (rows are contiguous along the in-features j).  The W' tile is
// dequantized into LDS in its natural [f][j] layout, exactly as in the
// forward kernel, and read transposed into the MFMA operand with gfx950's
// ds_read_b64_tr_b16 (a 4 x 16 block of 16-bit values per 16 lanes).
//
// Tiling: 256 in-features (MFMA rows) x 256 tokens (MFMA columns) per
// workgroup, K step 64 out-features, 4 waves in 2x2 with 128x128 each.
// LDS stage: W' tile 64 x 256 (rows padded to 544 B) + g tile 256 x 64.
#include "qlora_common.h"

namespace qlora {

namespace dgr {
constexpr int BJ = 256;                  // in-features per tile
constexpr int BT = 256;                  // tokens per tile
constexpr int BK = 64;                   // out-features per K step
constexpr int WROWB = BJ * 2 + 32;       // padded bytes per W' row
constexpr int WTILEB = BK * WROWB;       // 34816
constexpr int GROWB = BK * 2;            // 128 B per g row
constexpr int GTILEB = BT * GROWB;       // 32768
constexpr int STAGEB = WTILEB + GTILEB;  // 67584
constexpr int LDSB = 2 * STAGEB;         // 135168
}  // namespace dgr

__device__ __forceinline__ uint32_t gswz(int row, int c) {
  return (uint32_t)(row * dgr::GROWB + ((c ^ (row & 7)) << 4));
}

__device__ __forceinline__ int xcd_remap_d(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

struct DgradArgs {
  const uint16_t* g;       // M x m
  const uint8_t* codes;
  const uint8_t* absmax8;
  const float* c2;
  const uint16_t* At;      // n x r (A transposed)
  const float* v;          // M x r
  uint16_t* gx;            // M x n
  int64_t M, n, m;
  int r;
  float s;
  int tiles_j;
  int tiles_t;
};

__global__ __launch_bounds__(256) void dgrad_gemm_kernel(DgradArgs p, Nf4Table tab) {
  __shared__ __align__(16) uint8_t smem[dgr::LDSB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bid = xcd_remap_d(blockIdx.x, gridDim.x);
  const int tile_j = bid % p.tiles_j;
  const int tile_t = bid / p.tiles_j;
  const int64_t j0 = (int64_t)tile_j * dgr::BJ;
  const int64_t t0 = (int64_t)tile_t * dgr::BT;
  const int64_t n = p.n, m = p.m;
  const int nk = (int)((m + dgr::BK - 1) / dgr::BK);

  // dequant assignment: W' row (t/4) of the K step, 64-column block (t%4)
  const int wr = tid >> 2;
  const int wjb = tid & 3;
  const int64_t wj = j0 + 64 * wjb;
  const bool wj_ok = wj < n;
  // g chunks: 8 per thread, row = i*32 + tid/8, chunk tid%8
  const int gr_base = tid >> 3;
  const int gc = tid & 7;
  const bool m_vec = (m & 7) == 0;

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 greg[8];
  u32x4 creg[2];
  uint32_t areg;
  float c2reg;
  bool wrow_ok;

  auto gload = [&](int ks) {
    const int64_t k0 = (int64_t)ks * dgr::BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + gr_base;
      const int64_t t = t0 + row;
      const int64_t f = k0 + gc * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (t < p.M) {
        const uint16_t* src = p.g + t * m + f;
        if (m_vec && f + 8 <= m) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 8; ++e)
            if (f + e < m) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      greg[i] = v;
    }
    const int64_t f = k0 + wr;
    wrow_ok = (f < m) && wj_ok;
    const int64_t fc = f < m ? f : (m - 1);
    const int64_t jc = wj_ok ? wj : 0;
    const int64_t e0 = fc * n + jc;
    const u32x4* cp = reinterpret_cast<const u32x4*>(p.codes + e0 / 2);
    creg[0] = cp[0];
    creg[1] = cp[1];
    const int64_t blk = e0 / kBlock;
    areg = p.absmax8[blk];
    c2reg = p.c2[blk >> 8];
  };

  auto lstore = [&](int stage) {
    uint8_t* sW = smem + stage * dgr::STAGEB;
    uint8_t* sG = sW + dgr::WTILEB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + gr_base;
      *reinterpret_cast<u32x4*>(sG + gswz(row, gc)) = greg[i];
    }
    const float sc = wrow_ok ? e4m3_decode(areg) * c2reg : 0.0f;
    const BlockLut L = make_block_lut(tab, sc);
    uint8_t* dst = sW + wr * dgr::WROWB + wjb * 128;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w = creg[d >> 2][d & 3];
      uint32_t o[4];
      lut_dequant8(L, w, o);
      *reinterpret_cast<u32x4*>(dst + 16 * d) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  const int wjo = (wave & 1) * 128;  // in-feature offset of this wave
  const int wto = (wave >> 1) * 128; // token offset
  const int lr = lane & 15;
  const int lk = lane >> 4;
  // transposed-read source address inside a 16-lane group: row (lane%16)/4,
  // columns 4*(lane%4) .. +3 of the 16-column block
  const int tr_row = lr >> 2;
  const int tr_col = 4 * (lr & 3);

  gload(0);
  lstore(0);
  __syncthreads();

#pragma unroll 1
  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    uint8_t* sW = smem + stage * dgr::STAGEB;
    const uint8_t* sG = sW + dgr::WTILEB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int frow = 32 * kk + 8 * lk + tr_row;
        const int jcol = wjo + 16 * i + tr_col;
        uint8_t* base = sW + frow * dgr::WROWB + jcol * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * dgr::WROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a[i] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
      const int c = kk * 4 + lk;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = *reinterpret_cast<const u32x4*>(sG + gswz(wto + 16 * j + lr, c));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
    if (ks + 1 < nk) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: + s * v A, as extra K=32 MFMA steps (v split hi + lo) ----
  const int r = p.r;
  for (int q0 = 0; q0 < r; q0 += 32) {
    u32x4 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t j = j0 + wjo + 16 * i + lr;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      const int qb = q0 + 8 * lk;
      if (j < n) {
        const uint16_t* src = p.At + j * r + qb;
        if (qb + 8 <= r && (r & 7) == 0) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(src);
          w[0] = t[0]; w[1] = t[1]; w[2] = t[2]; w[3] = t[3];
        } else {
          for (int e = 0; e < 8; ++e)
            if (qb + e < r) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
        }
      }
      a[i] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int64_t t = t0 + wto + 16 * jj + lr;
      float vv[8];
      const int qb = q0 + 8 * lk;
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = (t < p.M && qb + e < r) ? p.v[t * r + qb + e] * p.s : 0.0f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, l0, h1, l1;
        split_bf16(vv[2 * e], h0, l0);
        split_bf16(vv[2 * e + 1], h1, l1);
        hi[e] = pack_bf16x2(h0, h1);
        lo[e] = pack_bf16x2(l0, l1);
      }
      const u32x4 bh = u32x4{hi[0], hi[1], hi[2], hi[3]};
      const u32x4 bl = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][jj] = mfma16x16x32(a[i], bh, acc[i][jj]);
        acc[i][jj] = mfma16x16x32(a[i], bl, acc[i][jj]);
      }
    }
  }

  // ---- store grad_x (bf16): lane holds 4 consecutive in-features of a token ----
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t j = j0 + wjo + 16 * i + 4 * lk;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int64_t t = t0 + wto + 16 * jj + lr;
      if (t >= p.M || j >= n) continue;
      const f32x4 v = acc[i][jj];
      // n is a multiple of 64, so the 4 features are in range and 8-byte aligned
      *reinterpret_cast<u32x2*>(p.gx + t * n + j) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

void launch_dgrad_gemm(const uint16_t* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                       const uint16_t* At, const float* v, uint16_t* gx, int64_t M, int64_t n, int64_t m, int r,
                       float s, const Nf4Table& tab, hipStream_t stream) {
  DgradArgs p;
  p.g = g; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.At = At; p.v = v; p.gx = gx;
  p.M = M; p.n = n; p.m = m; p.r = r; p.s = s;
  p.tiles_j = (int)((n + dgr::BJ - 1) / dgr::BJ);
  p.tiles_t = (int)((M + dgr::BT - 1) / dgr::BT);
  const int grid = p.tiles_j * p.tiles_t;
  hipLaunchKernelGGL(dgrad_gemm_kernel, dim3(grid), dim3(256), 0, stream, p, tab);
}

}  // namespace qlora
