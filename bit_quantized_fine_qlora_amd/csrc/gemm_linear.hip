// The two large-token GEMMs of the adapted linear layer, sharing one kernel:
//   forward   h      = x W'^T + s u B^T   (K = n, output features = rows of W0)
//   backward  grad_x = g W'   + s v A     (K = m, output features = columns of W0)
// with W' = dequant(W0) formed tile by tile in LDS as bf16 and never written
// to HBM.  "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3, both terms in BF16,
// scale alpha/r from the LoraConfig snippet) and Step 4 (gradients flow
// through the frozen, dequantized W0; the s v A term is the chain rule of the
// scaled adapter branch).
//
// gfx950 design, from measurements on the device:
//   - the matrix pipe stays busy while a SIMD issues at most ~2 VALU ops per
//     16x16x32 MFMA; dequantization costs ~3 VALU ops per weight, so each
//     dequantized weight must feed >= 256 tokens;
//   - activation rows must be read as whole 128-byte lines (scattered 16-byte
//     fragment loads reach only ~15 B/clk/CU from L2, line-coalesced loads
//     ~45 B/clk/CU);
//   - LDS reads reach ~210 B/clk/CU with two waves per SIMD.
// So a workgroup of 8 waves (2 per SIMD) covers 256 output features x 256
// tokens.  Per K step (64): the activation tile (256 x 64) is loaded with
// line-coalesced 16-byte loads and stored to LDS; waves 0-3 dequantize the
// 256 x 64 W' tile (one 64-weight block per thread, one magnitude table per
// block) into LDS, so each SIMD pairs a dequantizing wave with an MFMA-only
// wave; every wave then runs 64 MFMAs on its 128 x 64 output tile from LDS
// fragments.  The forward reads W' with ds_read_b128; the backward contracts
// over W0's rows, so it reads the natural-layout tile transposed with
// ds_read_b64_tr_b16.  LDS layouts are XOR-swizzled to avoid bank conflicts.
// Two LDS stages of {W' 32 KB, activations 32 KB}: 128 KB.
#include "qlora_common.h"

namespace qlora {

namespace lg2 {
constexpr int BF = 256;              // output features per tile
constexpr int BT = 256;              // tokens per tile
constexpr int BK = 64;               // K per step
constexpr int WTILEB = BF * BK * 2;  // 32 KB
constexpr int ATILEB = BT * BK * 2;  // 32 KB
constexpr int STAGEB = WTILEB + ATILEB;
constexpr int LDSB = 2 * STAGEB;     // 128 KB
}  // namespace lg2

struct GemmArgs {
  const uint16_t* act;     // M x K activations (x for the forward, g for the backward)
  const uint8_t* codes;    // quantized W0, m x n
  const uint8_t* absmax8;
  const float* c2;
  const uint16_t* lora_a;  // N x r: B (forward) or A^T (backward)
  const float* lora_b;     // M x r: u (forward) or v (backward)
  uint16_t* out;           // M x N
  int64_t M, K, N;         // tokens, contraction, output features
  int64_t wn;              // columns of W0 (n)
  int64_t wm;              // rows of W0 (m)
  int r;
  float s;
  int tiles_f;
  int tiles_t;
};

__device__ __forceinline__ int xcd_remap_l(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// [rows][64] bf16 tile (activations; forward W'): 16-byte chunk c of row r at
// chunk position c ^ (r & 7).
__device__ __forceinline__ uint32_t sw64(int row, int chunk) {
  return (uint32_t)(row * 128 + ((chunk ^ (row & 7)) << 4));
}
// Backward W' tile [64 K-rows][256 features] bf16: 32-byte chunk c (16
// features) of row r at chunk position c ^ sw(r), sw(r) = (r & 3) |
// ((r >> 3) & 1) << 2, which spreads the 16 rows of one transposed read
// (8q + 4h + 0..3 for the four lane groups q) over all bank groups.
__device__ __forceinline__ uint32_t swbwd(int row, int col) {
  const int sw = (row & 3) | (((row >> 3) & 1) << 2);
  return (uint32_t)(row * 512 + ((((col >> 4) ^ sw)) << 5) + ((col & 15) << 1));
}

template <bool kBwd>
__global__ __launch_bounds__(512) void linear_gemm_kernel(GemmArgs p, Nf4Table tab) {
  __shared__ __align__(16) uint8_t smem[lg2::LDSB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int bid = xcd_remap_l(blockIdx.x, gridDim.x);
  const int tile_f = bid % p.tiles_f;
  const int tile_t = bid / p.tiles_f;
  const int64_t f0 = (int64_t)tile_f * lg2::BF;
  const int64_t t0 = (int64_t)tile_t * lg2::BT;
  const int64_t K = p.K;
  const int nk = (int)((K + lg2::BK - 1) / lg2::BK);
  const int64_t wn = p.wn;
  const int64_t wnumel = p.wm * wn;
  const int wf = (wave & 1) * 128;  // this wave's 128 output features in the tile
  const int wt = (wave >> 1) * 64;  // this wave's 64 tokens

  // Buffer resources: reads past a tensor's end return 0.  Rows past M (or
  // past m / n of W0) read zeros or other rows of the same tensor; they only
  // feed outputs that are never stored.  In the backward's last K step the
  // W0 rows past m read zero codes and a zero 8-bit constant, i.e. zero
  // weights, so the finite activations there add nothing.
  const brsrc_t r_act = make_rsrc(p.act, (uint32_t)(p.M * K * 2));
  const brsrc_t r_codes = make_rsrc(p.codes, (uint32_t)(wnumel / 2));
  const brsrc_t r_amax = make_rsrc(p.absmax8, (uint32_t)(wnumel / kBlock));
  const brsrc_t r_c2 = make_rsrc(p.c2, (uint32_t)(((wnumel / kBlock + kGroupBlocks - 1) / kGroupBlocks) * 4));

  // ---- dequant assignment (threads 0..255): one 64-weight block per K step ----
  // forward : LDS row tid = out feature f0 + tid, block (f0 + tid, ks)
  // backward: LDS row tid/4 = W0 row 64*ks + tid/4, features f0 + 64*(tid%4) .. +63
  const int dt = tid & 255;
  uint32_t c_off, c_step, b_off, b_step;  // byte offsets of codes and absmax8 at step 0, per-step increments
  if (!kBwd) {
    const int64_t e0 = (f0 + dt) * wn;
    c_off = (uint32_t)(e0 / 2);  c_step = lg2::BK / 2;
    b_off = (uint32_t)(e0 / kBlock);  b_step = 1;
  } else {
    const int64_t e0 = (int64_t)(dt >> 2) * wn + f0 + 64 * (dt & 3);
    c_off = (uint32_t)(e0 / 2);  c_step = (uint32_t)(lg2::BK * wn / 2);
    b_off = (uint32_t)(e0 / kBlock);  b_step = (uint32_t)(lg2::BK * wn / kBlock);
  }

  // ---- activation tile loads: chunk id = i*512 + tid -> row id/8, chunk id%8 ----
  const int a_row0 = tid >> 3;  // + 64*i
  const int a_c = tid & 7;
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_off[i] = (uint32_t)(((t0 + 64 * i + a_row0) * K + 8 * a_c) * 2);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 areg[4];        // activation chunks of the next K step
  u32x4 creg[2];        // 64 codes of the next dequant step
  uint32_t aa = 0;      // absmax8 byte
  float sa = 0.f;       // c2 of the group

  auto load_act = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      areg[i] = bload128(r_act, a_off[i]);
      a_off[i] += lg2::BK * 2;
    }
  };
  auto store_act = [&](int stage) {
    uint8_t* dA = smem + stage * lg2::STAGEB + lg2::WTILEB;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dA + sw64(64 * i + a_row0, a_c)) = areg[i];
  };
  auto load_w = [&]() {
    creg[0] = bload128(r_codes, c_off);
    creg[1] = bload128(r_codes, c_off + 16);
    aa = bload8(r_amax, b_off);
    sa = __uint_as_float(bload32(r_c2, (b_off >> 8) << 2));
    c_off += c_step;
    b_off += b_step;
  };
  auto dequant_store = [&](int stage) {
    uint8_t* dW = smem + stage * lg2::STAGEB;
    const MagLut L = make_mag_lut(tab, e4m3_decode(aa) * sa);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t o[4];
      mag_dequant8(L, creg[d >> 2][d & 3], o);
      const uint32_t off = kBwd ? swbwd(dt >> 2, 64 * (dt & 3) + 8 * d) : sw64(dt, d);
      *reinterpret_cast<u32x4*>(dW + off) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  auto mfma_step = [&](int stage, int kk) {
    const uint8_t* sW = smem + stage * lg2::STAGEB;
    const uint8_t* sA = sW + lg2::WTILEB;
    u32x4 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const u32x4*>(sA + sw64(wt + 16 * j + lr, 4 * kk + lq));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 a;
      if (!kBwd) {
        a = *reinterpret_cast<const u32x4*>(sW + sw64(wf + 16 * i + lr, 4 * kk + lq));
      } else {
        // K rows 32*kk + 8*lq + 4*h + lr/4, feature columns wf + 16*i + 4*(lr%4) .. +3
        const int row = 32 * kk + 8 * lq + (lr >> 2);
        const int col = wf + 16 * i + 4 * (lr & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sW + swbwd(row, col)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sW + swbwd(row + 4, col)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a, b[j], acc[i][j]);
    }
  };
  // One K step on LDS stage `stage`: the registers holding step ks+1 go to
  // the other stage (activations stored, W' dequantized by waves 0-3) while
  // the MFMAs run, and the loads of step ks+2 are issued.
  auto step_dq = [&](int stage) {
    store_act(stage ^ 1);
    load_act();
    mfma_step(stage, 0);
    dequant_store(stage ^ 1);
    load_w();
    mfma_step(stage, 1);
    __syncthreads();
  };
  auto step_mm = [&](int stage) {
    store_act(stage ^ 1);
    load_act();
    mfma_step(stage, 0);
    mfma_step(stage, 1);
    __syncthreads();
  };

  // prologue: stage 0 <- step 0; registers <- step 1
  const bool dq_wave = wave < 4;
  load_act();
  if (dq_wave) load_w();
  store_act(0);
  if (dq_wave) {
    dequant_store(0);
    load_w();
  }
  load_act();
  __syncthreads();

  if (dq_wave) {
#pragma unroll 1
    for (int ks = 0; ks < nk; ++ks) step_dq(ks & 1);
  } else {
#pragma unroll 1
    for (int ks = 0; ks < nk; ++ks) step_mm(ks & 1);
  }

  // ---- epilogue: + s * lora_b lora_a^T as extra K=32 MFMA steps (fp32 factor split hi + lo) ----
  const int r = p.r;
  for (int q0 = 0; q0 < r; q0 += 32) {
    u32x4 la[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t f = f0 + wf + 16 * i + lr;
      uint32_t v[4] = {0u, 0u, 0u, 0u};
      const int qb = q0 + 8 * lq;
      if (f < p.N) {
        const uint16_t* src = p.lora_a + f * r + qb;
        if (qb + 8 <= r && (r & 7) == 0) {
          const u32x4 t = *reinterpret_cast<const u32x4*>(src);
          v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
        } else {
          for (int e = 0; e < 8; ++e)
            if (qb + e < r) v[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
        }
      }
      la[i] = u32x4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wt + 16 * j + lr;
      float bv[8];
      const int qb = q0 + 8 * lq;
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = (t < p.M && qb + e < r) ? p.lora_b[t * r + qb + e] * p.s : 0.0f;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, l0, h1, l1;
        split_bf16(bv[2 * e], h0, l0);
        split_bf16(bv[2 * e + 1], h1, l1);
        hi[e] = pack_bf16x2(h0, h1);
        lo[e] = pack_bf16x2(l0, l1);
      }
      const u32x4 bh = u32x4{hi[0], hi[1], hi[2], hi[3]};
      const u32x4 bl = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][j] = mfma16x16x32(la[i], bh, acc[i][j]);
        acc[i][j] = mfma16x16x32(la[i], bl, acc[i][j]);
      }
    }
  }

  // ---- store (bf16): lane holds 4 consecutive output features of one token ----
  const bool vec_ok = (p.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t f = f0 + wf + 16 * i + 4 * lq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wt + 16 * j + lr;
      if (t >= p.M) continue;
      const f32x4 v = acc[i][j];
      uint16_t* dst = p.out + t * p.N + f;
      if (vec_ok && f + 3 < p.N) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
        for (int e = 0; e < 4; ++e)
          if (f + e < p.N) dst[e] = (uint16_t)(pack_bf16x2(v[e], 0.0f) & 0xFFFFu);
      }
    }
  }
}

static void launch_linear_gemm(bool bwd, const GemmArgs& a, const Nf4Table& tab, hipStream_t stream) {
  GemmArgs p = a;
  p.tiles_f = (int)((p.N + lg2::BF - 1) / lg2::BF);
  p.tiles_t = (int)((p.M + lg2::BT - 1) / lg2::BT);
  const int grid = p.tiles_f * p.tiles_t;
  if (bwd)
    hipLaunchKernelGGL(linear_gemm_kernel<true>, dim3(grid), dim3(512), 0, stream, p, tab);
  else
    hipLaunchKernelGGL(linear_gemm_kernel<false>, dim3(grid), dim3(512), 0, stream, p, tab);
}

void launch_fwd_gemm(const uint16_t* x, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                     const uint16_t* B, const float* u, uint16_t* h, int64_t M, int64_t n, int64_t m, int r,
                     float s, const Nf4Table& tab, hipStream_t stream) {
  GemmArgs p{};
  p.act = x; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.lora_a = B; p.lora_b = u; p.out = h;
  p.M = M; p.K = n; p.N = m; p.wn = n; p.wm = m; p.r = r; p.s = s;
  launch_linear_gemm(false, p, tab, stream);
}

// g is M x m_pad (m_pad = m, or m rounded up to 64 with zero columns when
// m % 8 != 0, so every 16-byte chunk of the tensor is whole).
void launch_dgrad_gemm(const uint16_t* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                       const uint16_t* At, const float* v, uint16_t* gx, int64_t M, int64_t n, int64_t m,
                       int64_t m_pad, int r, float s, const Nf4Table& tab, hipStream_t stream) {
  GemmArgs p{};
  p.act = g; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.lora_a = At; p.lora_b = v; p.out = gx;
  p.M = M; p.K = m_pad; p.N = n; p.wn = n; p.wm = m; p.r = r; p.s = s;
  launch_linear_gemm(true, p, tab, stream);
}

}  // namespace qlora
