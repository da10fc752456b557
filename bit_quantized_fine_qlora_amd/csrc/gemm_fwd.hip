// Forward of the adapted linear layer for many tokens:
//   h = x W'^T + s u B^T,  u = x A^T  (u comes in precomputed, fp32)
// with W' = dequant(W0) formed tile by tile in LDS as bf16 and never written
// to HBM.  "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3: frozen term plus
// the low-rank term, both computed in BF16; scale alpha/r from the LoraConfig
// snippet) and the memory-layout figure (NF4 storage, dequant to BF16).
//
// Tiling (gfx950, 64-wide waves, MFMA 16x16x32 bf16 -> fp32):
//   workgroup tile 256 out-features x 256 tokens, K step 64 (= one absmax
//   block per feature row), 4 waves in 2x2, 128x128 per wave.
//   LDS: two stages of {W' tile 256x64, x tile 256x64} bf16 = 128 KB.
//   Each thread dequantizes one 64-weight block per K step (one row of the
//   W' tile) through a per-block 16-entry bf16 table.
#include "qlora_common.h"

namespace qlora {

namespace fwd {
constexpr int BM = 256;  // out features per tile (MFMA rows)
constexpr int BN = 256;  // tokens per tile (MFMA columns)
constexpr int BK = 64;
constexpr int ROWB = BK * 2;               // bytes per LDS row (64 bf16)
constexpr int TILEB = 256 * ROWB;          // bytes per 256-row tile
constexpr int STAGEB = 2 * TILEB;          // W' tile + x tile
constexpr int LDSB = 2 * STAGEB;           // two stages
}  // namespace fwd

// Byte offset of the 16-byte chunk (row, c) in a 64-wide bf16 tile; the chunk
// index is XOR-swizzled with the row so 8 consecutive rows hit 8 different
// bank groups.
__device__ __forceinline__ uint32_t swz64(int row, int c) {
  return (uint32_t)(row * fwd::ROWB + ((c ^ (row & 7)) << 4));
}

// Map a linear workgroup id to a tile so that the 8 XCDs (which receive
// workgroups round-robin) each work through a contiguous range of tiles.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

struct FwdArgs {
  const uint16_t* x;       // M x n
  const uint8_t* codes;    // m*n/2
  const uint8_t* absmax8;  // m*n/64
  const float* c2;
  const uint16_t* B;       // m x r
  const float* u;          // M x r
  uint16_t* h;             // M x m
  int64_t M, n, m;
  int r;
  float s;
  int tiles_f;             // ceil(m / 256)
  int tiles_t;             // ceil(M / 256)
};

__global__ __launch_bounds__(256) void fwd_gemm_kernel(FwdArgs p, Nf4Table tab) {
  __shared__ __align__(16) uint8_t smem[fwd::LDSB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile_f = bid % p.tiles_f;
  const int tile_t = bid / p.tiles_f;
  const int64_t f0 = (int64_t)tile_f * fwd::BM;
  const int64_t t0 = (int64_t)tile_t * fwd::BN;
  const int64_t n = p.n;
  const int nk = (int)(n / fwd::BK);

  // ---- per-thread load assignments ----
  // W' row owned by this thread (one 64-weight block per K step)
  const int64_t wrow = f0 + tid;
  const bool wrow_ok = wrow < p.m;
  const int64_t wrow_c = wrow_ok ? wrow : (p.m - 1);  // clamp: valid address, result discarded
  const uint8_t* code_ptr = p.codes + (wrow_c * n) / 2;
  const int64_t blk_base = (wrow_c * n) / kBlock;
  // x chunks: 8 per thread, chunk id = i*256 + tid -> row id/8, chunk id%8
  const int xr_base = tid >> 3;
  const int xc = tid & 7;

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xreg[8];
  u32x4 creg[2];
  uint32_t areg;
  float c2reg;

  auto gload = [&](int ks) {
    const int64_t k0 = (int64_t)ks * fwd::BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + xr_base;
      const int64_t t = t0 + row;
      if (t < p.M) {
        xreg[i] = *reinterpret_cast<const u32x4*>(p.x + t * n + k0 + xc * 8);
      } else {
        xreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    const u32x4* cp = reinterpret_cast<const u32x4*>(code_ptr + k0 / 2);
    creg[0] = cp[0];
    creg[1] = cp[1];
    const int64_t blk = blk_base + ks;
    areg = p.absmax8[blk];
    c2reg = p.c2[blk >> 8];
  };

  auto lstore = [&](int stage) {
    uint8_t* sW = smem + stage * fwd::STAGEB;
    uint8_t* sX = sW + fwd::TILEB;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + xr_base;
      *reinterpret_cast<u32x4*>(sX + swz64(row, xc)) = xreg[i];
    }
    const float sc = wrow_ok ? e4m3_decode(areg) * c2reg : 0.0f;
    const BlockLut L = make_block_lut(tab, sc);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t w = creg[d >> 2][d & 3];
      uint32_t o[4];
      lut_dequant8(L, w, o);
      *reinterpret_cast<u32x4*>(sW + swz64(tid, d)) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  const int wf = (wave & 1) * 128;   // feature offset of this wave in the tile
  const int wt = (wave >> 1) * 128;  // token offset
  const int lr = lane & 15;
  const int lk = lane >> 4;

  gload(0);
  lstore(0);
  __syncthreads();

#pragma unroll 1
  for (int ks = 0; ks < nk; ++ks) {
    const int stage = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    const uint8_t* sW = smem + stage * fwd::STAGEB;
    const uint8_t* sX = sW + fwd::TILEB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[8], b[8];
      const int c = kk * 4 + lk;
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const u32x4*>(sW + swz64(wf + 16 * i + lr, c));
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = *reinterpret_cast<const u32x4*>(sX + swz64(wt + 16 * j + lr, c));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
    if (ks + 1 < nk) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: + s * u B^T, as extra K=32 MFMA steps (u split hi + lo) ----
  const int r = p.r;
  for (int q0 = 0; q0 < r; q0 += 32) {
    u32x4 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t f = f0 + wf + 16 * i + lr;
      uint32_t v[4] = {0u, 0u, 0u, 0u};
      const int qb = q0 + 8 * lk;
      if (f < p.m) {
        const uint16_t* src = p.B + f * r + qb;
        if (qb + 8 <= r && (r & 7) == 0) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(src);
          v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
        } else {
          for (int e = 0; e < 8; ++e)
            if (qb + e < r) v[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
        }
      }
      a[i] = u32x4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = t0 + wt + 16 * j + lr;
      float uv[8];
      const int qb = q0 + 8 * lk;
#pragma unroll
      for (int e = 0; e < 8; ++e) uv[e] = (t < p.M && qb + e < r) ? p.u[t * r + qb + e] * p.s : 0.0f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, l0, h1, l1;
        split_bf16(uv[2 * e], h0, l0);
        split_bf16(uv[2 * e + 1], h1, l1);
        hi[e] = pack_bf16x2(h0, h1);
        lo[e] = pack_bf16x2(l0, l1);
      }
      const u32x4 bh = u32x4{hi[0], hi[1], hi[2], hi[3]};
      const u32x4 bl = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][j] = mfma16x16x32(a[i], bh, acc[i][j]);
        acc[i][j] = mfma16x16x32(a[i], bl, acc[i][j]);
      }
    }
  }

  // ---- store h (bf16): lane holds 4 consecutive features of one token ----
  const bool vec_ok = (p.m & 3) == 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t f = f0 + wf + 16 * i + 4 * lk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = t0 + wt + 16 * j + lr;
      if (t >= p.M) continue;
      const f32x4 v = acc[i][j];
      uint16_t* dst = p.h + t * p.m + f;
      if (vec_ok && f + 3 < p.m) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
        for (int e = 0; e < 4; ++e)
          if (f + e < p.m) dst[e] = (uint16_t)(pack_bf16x2(v[e], 0.0f) & 0xFFFFu);
      }
    }
  }
}

void launch_fwd_gemm(const uint16_t* x, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                     const uint16_t* B, const float* u, uint16_t* h, int64_t M, int64_t n, int64_t m, int r,
                     float s, const Nf4Table& tab, hipStream_t stream) {
  FwdArgs p;
  p.x = x; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.B = B; p.u = u; p.h = h;
  p.M = M; p.n = n; p.m = m; p.r = r; p.s = s;
  p.tiles_f = (int)((m + fwd::BM - 1) / fwd::BM);
  p.tiles_t = (int)((M + fwd::BN - 1) / fwd::BN);
  const int grid = p.tiles_f * p.tiles_t;
  hipLaunchKernelGGL(fwd_gemm_kernel, dim3(grid), dim3(256), 0, stream, p, tab);
}

}  // namespace qlora
