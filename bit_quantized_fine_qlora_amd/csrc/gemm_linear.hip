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
//   - a wave that mixes VALU work with its own MFMAs serializes the two, but
//     VALU work of another wave on the same SIMD runs under that SIMD's
//     MFMAs; so dequantization and the activation copy go to waves of their
//     own, and the MFMA waves only read LDS fragments and issue MFMAs;
//   - dequantization costs ~3 VALU ops per weight, so each dequantized weight
//     must feed >= 256 tokens;
//   - activation rows are read as whole 128-byte lines (scattered 16-byte
//     fragment loads reach only a third of the rate from L2).
// A workgroup of 12 waves covers 256 output features x 256 tokens: 8 MFMA
// waves (2 per SIMD, each a 128 x 64 output tile) and 4 producer waves (one
// per SIMD).  Per K step (64) the producers store the dequantized W' tile
// (256 x 64, one 64-weight block per thread, one magnitude table per block)
// of the next step into the other LDS stage and issue the code loads of the
// step after, while the MFMA waves run 64 MFMAs each on the current stage;
// the MFMA waves also start the copy of the next activation tile (256 x 64)
// with buffer loads that write LDS directly (no registers, 4 per wave).  The forward reads W' with
// ds_read_b128; the backward contracts over W0's rows, so it reads the
// natural-layout tile transposed with ds_read_b64_tr_b16.  The LDS layouts
// below keep every store and the forward's fragment reads free of bank
// conflicts, and every fragment address is one per-lane base plus an
// immediate offset.  Two LDS stages of {W', activations}: 128 KB forward,
// 134 KB backward.  The
// LoRA term runs as extra K steps whose tiles the producers fill from the
// adapter factors.
#include "qlora_common.h"

namespace qlora {

namespace lg2 {
constexpr int BF = 256;              // output features per tile
constexpr int BT = 256;              // tokens per tile
constexpr int BK = 64;               // K per step
// LDS layouts, checked with the bank-conflict counter on loops of each
// access stream (LDS: 256 bytes per cycle).
//   activations [256 rows][64 K] bf16: pitch 128, written 1 KB (8 rows) at a
//     time by the direct-to-LDS loads, so the 16-byte chunk c of row r sits
//     at position c ^ (r & 7) instead (the loads pick their sources to match).
//   forward W' [256 rows][64 K] bf16: the same layout as the activations
//     (its fragment reads have the same shape).  A pitch of 144 bytes, which
//     puts 16 consecutive rows on distinct 16-byte slots, measured 2-way
//     conflicted on these reads (the bank-conflict counter and the time of
//     a read-only loop both doubled), while the XOR layout reads free.
//   backward W' [64 K rows][256 features]: pitch 560 = 35 x 16; dequant
//     stores are conflict-free.  A ds_read_b64_tr_b16 serves 32 lanes (8 rows
//     x 32 bytes) per cycle, and rows r and r + 8 of one cycle overlap here,
//     so the transposed reads take 1.5x their conflict-free LDS cycles.  A
//     pitch-512 layout with a row-dependent chunk XOR removes that, but its
//     per-read address XORs in the MFMA waves cost as much as it saved (the
//     grad_x GEMM time did not change), so this layout stays.
constexpr int WPB = 560;
constexpr int ATILEB = BT * 128;     // 32 KB
template <bool kBwd> struct Tile {
  static constexpr int W = kBwd ? BK * WPB : BF * 128;  // 35 / 32 KB
};
// The four LDS tiles are separate arrays (136 KB in all): the compiler then
// knows that reading one stage does not alias the direct-to-LDS copy into
// the other, and does not make the reads wait for that copy.  Stage indices
// are compile-time constants (the K loops are unrolled by two).
struct Lds {
  uint8_t* w[2];
  uint8_t* a[2];
};
constexpr int kMfmaWaves = 8;
constexpr int kThreads = 64 * (kMfmaWaves + 4);
}  // namespace lg2

struct GemmArgs {
  const uint16_t* act;     // M x K activations (x for the forward, g for the backward)
  const uint8_t* codes;    // quantized W0, m x n
  const uint8_t* absmax8;
  const float* c2;
  const uint16_t* lora_a;  // B (m x r, forward) or A (r x n, backward)
  const float* lora_b;     // M x r: u (forward) or v (backward)
  uint16_t* out;           // M x N
  int64_t M, K, N;         // tokens, contraction, output features
  int64_t wn;              // columns of W0 (n)
  int64_t wm;              // rows of W0 (m)
  int r;
  float s;
  int tiles_f;
  int tiles_t;
  // Last partial round of tiles split in K (see launch_linear_gemm): work
  // items full_tiles .. full_tiles + 2 nsplit - 1 are the two K halves of
  // tiles full_tiles .. full_tiles + nsplit - 1.
  int full_tiles;
  int nsplit;
  float* partial;         // nsplit x 256 x 256 fp32, the first finisher's sum
  uint32_t* split_sync;   // nsplit x {arrivals, partial ready}, then the
                          // give-up word; all zero at launch
  const float* add;       // M x N fp32 added before the rounding, or null
  // Few tiles (see gemm_pieces): pieces > 1 runs every tile as that many K
  // pieces, work item b being piece b % pieces of tile b / pieces; each piece
  // writes its fp32 sums to slot b of piece_out (256 x 256 floats a slot, in
  // the split hand-off's fragment layout) and reduce_pieces_kernel finishes
  // the output.
  int pieces;
  float* piece_out;
};

// The two halves of a split tile meet at the end: the first to finish
// (by an atomic arrival count) stores its fp32 accumulators and raises the
// ready flag; the second waits for the flag, adds the stored sum to its own
// and writes the tile.  fp32 addition of two terms is commutative, so the
// result does not depend on which half finishes first.  The halves may run
// on different XCDs (separate L2s): every access of the hand-off (sum, count,
// flag) is device-scope (sc1), which keeps it coherent without acquire /
// release fences, whose L2 writeback / invalidate would slow every other
// workgroup on the XCD.
constexpr uint32_t kSplitSpinLimit = 1u << 22;
constexpr int kAuxDevice = 16;  // buffer access cache policy: sc1 (device scope)

__device__ __forceinline__ int xcd_remap_l(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

// Producer waves (256 threads, pt = 0..255): activation tile copy, W' tile
// dequantization, and the LoRA epilogue operands.
template <bool kBwd>
__device__ __forceinline__ void gemm_producer(const GemmArgs& p, const Nf4Table& tab, const lg2::Lds& lds, int pt,
                                              int64_t f0, int64_t t0, int k0, int nk, bool lora, int split,
                                              uint32_t* lds_word) {
  const int64_t K = p.K;
  const int64_t wn = p.wn;
  const int64_t wnumel = p.wm * wn;
  // Buffer resources: reads past a tensor's end return 0.  Rows past M (or
  // past m / n of W0) read zeros or other rows of the same tensor; they only
  // feed outputs that are never stored.  In the backward's last K step the
  // W0 rows past m read zero codes and a zero 8-bit constant, i.e. zero
  // weights, so the finite activations there add nothing.
  const brsrc_t r_codes = make_rsrc(p.codes, (uint32_t)(wnumel / 2));
  const brsrc_t r_amax = make_rsrc(p.absmax8, (uint32_t)(wnumel / kBlock));
  const brsrc_t r_c2 = make_rsrc(p.c2, (uint32_t)(((wnumel / kBlock + kGroupBlocks - 1) / kGroupBlocks) * 4));

  // dequant assignment: one 64-weight block per thread and K step
  // forward : LDS row pt = out feature f0 + pt, block (f0 + pt, ks)
  // backward: LDS row pt%64 = W0 row 64*ks + pt%64, features f0 + 64*(pt/64) .. +63
  uint32_t c_off, c_step, b_off, b_step;
  if (!kBwd) {
    const int64_t e0 = (f0 + pt) * wn;
    c_off = (uint32_t)(e0 / 2);  c_step = lg2::BK / 2;
    b_off = (uint32_t)(e0 / kBlock);  b_step = 1;
  } else {
    const int64_t e0 = (int64_t)(pt & 63) * wn + f0 + 64 * (pt >> 6);
    c_off = (uint32_t)(e0 / 2);  c_step = (uint32_t)(lg2::BK * wn / 2);
    b_off = (uint32_t)(e0 / kBlock);  b_step = (uint32_t)(lg2::BK * wn / kBlock);
  }
  c_off += (uint32_t)k0 * c_step;  // first K step of this work item
  b_off += (uint32_t)k0 * b_step;
  // Two register sets, so the code loads of step ks + 2 are issued a whole
  // K step before their data is dequantized.
  struct Regs {
    u32x4 code[2];  // 64 codes
    uint8_t aa;     // absmax8 byte (kept 8-bit so its zero-extension is
                    // placed at the use, not right after the load)
    float sa;       // c2 of the group
  };
  using T = lg2::Tile<kBwd>;
  const uint32_t w_st = kBwd ? (uint32_t)((pt & 63) * lg2::WPB + 128 * (pt >> 6)) : (uint32_t)(pt * 128);
  // Address of 16-byte chunk d of this thread's W' piece.  Forward: row pt
  // in the XOR layout, i.e. w_row ^ 16 d with w_row = 128 pt + 16 (pt % 8)
  // (d flips only address bits 4-6); the base is made opaque at each store
  // so the eight addresses cost one XOR each instead of eight registers.
  const uint32_t w_row = kBwd ? w_st : (uint32_t)(pt * 128 + ((pt & 7) << 4));
  auto wbase = [&]() -> uint32_t {
    uint32_t b = w_row;
    if (!kBwd) asm volatile("" : "+v"(b));
    return b;
  };
  auto wchunk = [&](uint32_t b, int d) -> uint32_t { return kBwd ? b + (uint32_t)(16 * d) : b ^ (uint32_t)(16 * d); };
  auto load = [&](Regs& R) {
    R.code[0] = bload128(r_codes, c_off);
    R.code[1] = bload128(r_codes, c_off + 16);
    R.aa = __builtin_amdgcn_raw_buffer_load_b8(r_amax, (int)b_off, 0, 0);
    R.sa = __uint_as_float(bload32(r_c2, (b_off >> 8) << 2));
    c_off += c_step;
    b_off += b_step;
  };
  auto store = [&](const Regs& R, uint8_t* tile) {
    const uint32_t wb = wbase();
    const MagLut L = make_mag_lut(tab, e4m3_decode((uint32_t)R.aa) * R.sa);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      uint32_t o[4];
      mag_dequant8(L, R.code[d >> 2][d & 3], o);
      *reinterpret_cast<u32x4*>(tile + wchunk(wb, d)) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  // K step ks: `cur` holds step ks + 1, `nxt` receives step ks + 2.  The
  // loads are unconditional (past the end they read other rows or zeros and
  // are never stored), which keeps the compiler's wait counts exact: a
  // conditional load makes it wait for the prefetch just issued.
  auto step = [&](Regs& cur, Regs& nxt, uint8_t* next_tile) {
    load(nxt);
    store(cur, next_tile);
    __syncthreads();
  };
  (void)K;

  // The LoRA term s * lora_b lora_a^T runs as nq = ceil(r / 32) extra K
  // steps of 64 that the producers fill: step q pairs ranks 32q .. 32q + 31
  // twice, once with the bf16 hi part of s * lora_b and once with its lo part
  // (the fp32 factor as hi + lo; lora_a is bf16 already).  In the forward,
  // for r <= 16 the pairs fit the first K half (ranks 0 .. 15 with hi at
  // k 0 .. 15 and with lo at k 16 .. 31), and the MFMA waves run only that
  // half of the step (forward 424 -> 418 us; the same change in the
  // backward measured 12 us slower, so the backward keeps the full step).
  //   forward : W' row f (feature), k: B[f][32q + k % 32]
  //   backward: W' row k, feature f:   A[32q + k % 32][f]
  //   activations row t, k < 32: hi(s u[t][32q + k]), k >= 32: lo(s u[t][32q + k - 32])
  //   (v instead of u in the backward)
  // Out-of-range rows, features and ranks are zero.  The operands of q = 0
  // are loaded in the prologue and stay in registers through the K loop.
  const int r = p.r;
  const int nq = lora ? (r + 31) / 32 : 0;
  const bool lora16 = !kBwd && r <= 16;
  struct LoraRegs {
    u32x4 f[kBwd ? 8 : 4];
    float t[32];
  };
  LoraRegs LR;
  auto lora_load = [&](int q) {
    const int q0 = 32 * q;
    if (!kBwd) {
      const int64_t f = f0 + pt;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int qb = q0 + 8 * c;
        if (f < p.N && (r & 7) == 0 && qb + 8 <= r) {
          LR.f[c] = *reinterpret_cast<const u32x4*>(p.lora_a + f * r + qb);
        } else {
          uint32_t v[4] = {0u, 0u, 0u, 0u};
          if (f < p.N)
            for (int e = 0; e < 8; ++e)
              if (qb + e < r) v[e >> 1] |= (uint32_t)p.lora_a[f * r + qb + e] << (16 * (e & 1));
          LR.f[c] = u32x4{v[0], v[1], v[2], v[3]};
        }
      }
    } else {
      const int rank = q0 + (lora16 ? (pt & 15) : (pt & 31));
      const int64_t fb = f0 + 64 * (pt >> 6);  // n % 64 == 0: all 64 features in range or none
      const bool ok = rank < r && fb < p.N;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        LR.f[c] = ok ? *reinterpret_cast<const u32x4*>(p.lora_a + (int64_t)rank * p.N + fb + 8 * c)
                     : u32x4{0u, 0u, 0u, 0u};
    }
    const int64_t t = t0 + pt;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int qb = q0 + 4 * c;
      if (t < p.M && (r & 3) == 0 && qb + 4 <= r) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p.lora_b + t * r + qb);
        LR.t[4 * c] = v[0]; LR.t[4 * c + 1] = v[1]; LR.t[4 * c + 2] = v[2]; LR.t[4 * c + 3] = v[3];
      } else {
        for (int e = 0; e < 4; ++e) LR.t[4 * c + e] = (t < p.M && qb + e < r) ? p.lora_b[t * r + qb + e] : 0.0f;
      }
    }
  };
  auto lora_store = [&](uint8_t* wtile, uint8_t* atile) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const u32x4 v = kBwd ? LR.f[d] : LR.f[lora16 ? (d & 1) : (d & 3)];
      *reinterpret_cast<u32x4*>(wtile + wchunk(wbase(), d)) = v;
    }
    // activation row pt: chunk c at position c ^ (pt % 8)
    uint8_t* arow = atile + pt * 128;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (lora16 && c >= 2) break;  // ranks 16 .. 31 are zero
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float h0, l0, h1, l1;
        split_bf16(p.s * LR.t[8 * c + 2 * e], h0, l0);
        split_bf16(p.s * LR.t[8 * c + 2 * e + 1], h1, l1);
        hi[e] = pack_bf16x2(h0, h1);
        lo[e] = pack_bf16x2(l0, l1);
      }
      *reinterpret_cast<u32x4*>(arow + ((c ^ (pt & 7)) << 4)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<u32x4*>(arow + (((c + (lora16 ? 2 : 4)) ^ (pt & 7)) << 4)) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
  };

  Regs R0, R1;
  // prologue: stage 0 <- step 0, R1 <- step 1, LoRA operands of q = 0
  load(R0);
  load(R1);
  if (nq > 0) lora_load(0);
  store(R0, lds.w[0]);
  __syncthreads();
  // K step ks stores step ks + 1 into stage (ks + 1) % 2: regular steps 1 .. nk - 1
#pragma unroll 1
  for (int ks = 0; ks < nk - 1; ks += 2) {
    step(R1, R0, lds.w[1]);
    if (ks + 1 < nk - 1) step(R0, R1, lds.w[0]);
  }
  // LoRA steps nk .. nk + nq - 1, then the last step's barrier
  for (int q = 0; q < nq; ++q) {
    const int j = nk + q;
    lora_store((j & 1) ? lds.w[1] : lds.w[0], (j & 1) ? lds.a[1] : lds.a[0]);
    if (q + 1 < nq) lora_load(q + 1);
    __syncthreads();
  }
  __syncthreads();
  if (split) {  // the barriers of the split-tile hand-off (see gemm_consumer)
    __syncthreads();
    if (*lds_word == 0u) __syncthreads();
  }
}

// MFMA waves (512 threads): each owns a WF-feature x WT-token output tile,
// 128 x 64 in the forward and 64 x 128 in the backward, where the W'
// fragments come from half-rate transposed reads and the activation
// fragments from full-rate ones (the 64 x 128 shape halves the former).
template <bool kBwd, bool kPieces, bool kSkip>
__device__ __forceinline__ void gemm_consumer(const GemmArgs& p, const lg2::Lds& lds, int tid, int64_t f0,
                                              int64_t t0, int k0, int nk, bool lora, int split, uint32_t* lds_word) {
  constexpr int WF = kBwd ? 64 : 128;
  constexpr int WT = 128 * 64 / WF;
  constexpr int NI = WF / 16;  // 16-feature fragments
  constexpr int NJ = WT / 16;  // 16-token fragments
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps tile offsets scalar
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int wf = (wave % (lg2::BF / WF)) * WF;
  const int wt = (wave / (lg2::BF / WF)) * WT;
  // A wave whose tokens all lie past M (a ragged last token tile, few-token
  // GEMMs) only reads zero rows: it skips its MFMAs and its piece store
  // (the accumulators stay zero, and no output row past M is written), so
  // for M <= 128 the remaining waves' MFMAs share the SIMDs.  Only launches
  // with M % 256 != 0 test it (kSkip): the branch in the K loop costs the
  // whole-tile GEMMs 2-3 %.
  const bool active = !kSkip || t0 + wt < p.M;

  f32x4 acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  using T = lg2::Tile<kBwd>;
  // Activation tile copy: this wave fills rows 32 w .. 32 w + 31 of the tile,
  // 8 rows (1 KB) per load; lane l lands at byte 16 l of its block, i.e. row
  // l / 8, chunk position l % 8, which holds chunk (l % 8) ^ (l / 8).  Rows
  // past M are out of the buffer's range and read 0.
  const brsrc_t r_act = make_rsrc(p.act, (uint32_t)(p.M * p.K * 2));
  uint32_t act_off = (uint32_t)(((t0 + 32 * wave + (lane >> 3)) * p.K + 8 * ((lane & 7) ^ (lane >> 3)) +
                                  (int64_t)k0 * lg2::BK) * 2);
  const uint32_t act_blk = (uint32_t)(8 * p.K * 2);
  auto copy_act = [&](uint8_t* tile) {
    uint8_t* dst = tile + 32 * 128 * wave;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_act, (__attribute__((address_space(3))) void*)(dst + 1024 * b), 16,
                                               act_off + act_blk * b, 0, 0, 0);
    act_off += lg2::BK * 2;
  };

  // Fragment addresses: one per-lane base plus immediate offsets.
  //   activations: row wt + 16 j + lr, chunk 4 kk + lq at position (4 kk + lq) ^ (lr % 8)
  //   forward W' : row wf + 16 i + lr, chunk 4 kk + lq
  //   backward W': K rows 32 kk + 8 lq + 4 h + lr/4, features wf + 16 i + 4 (lr % 4) .. +3
  const uint32_t a_base0 = (uint32_t)((wt + lr) * 128 + ((lq ^ (lr & 7)) << 4));
  const uint32_t a_base1 = a_base0 ^ 64u;
  const uint32_t w_base = kBwd ? (uint32_t)((8 * lq + (lr >> 2)) * lg2::WPB + 2 * (wf + 4 * (lr & 3)))
                               : (uint32_t)((wf + lr) * 128 + ((lq ^ (lr & 7)) << 4));
  // A fragment i of step kk
  auto load_a = [&](const uint8_t* sW, int kk, int i) -> u32x4 {
    if (!kBwd) {
      // chunk 4 kk + lq of row wf + 16 i + lr: position (4 kk + lq) ^ (lr % 8)
      return *reinterpret_cast<const u32x4*>(sW + (kk ? (w_base ^ 64u) : w_base) + 2048 * i);
    } else {
      const uint8_t* src = sW + w_base + 32 * lg2::WPB * kk + 32 * i;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 4 * lg2::WPB));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
  };
  auto load_b = [&](const uint8_t* sA, int kk, int j) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(sA + (kk ? a_base1 : a_base0) + 2048 * j);
  };
  // 32 MFMAs of one K = 32 half step.  The smaller fragment set is held, the
  // larger one software-pipelined one ahead; the scheduling barriers keep the
  // compiler from hoisting all of it (the accumulators leave room for two).
  auto mfma_step = [&](const uint8_t* sW, const uint8_t* sA, int kk) {
    if constexpr (NI >= NJ) {
      u32x4 b[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = load_b(sA, kk, j);
      u32x4 a_cur = load_a(sW, kk, 0);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        u32x4 a_nxt;
        if (i + 1 < NI) a_nxt = load_a(sW, kk, i + 1);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(a_cur, b[j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < NI) a_cur = a_nxt;
      }
    } else {
      u32x4 a[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = load_a(sW, kk, i);
      u32x4 b_cur = load_b(sA, kk, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        u32x4 b_nxt;
        if (j + 1 < NJ) b_nxt = load_b(sA, kk, j + 1);
#pragma unroll
        for (int i = 0; i < NI; ++i) acc[i][j] = mfma16x16x32(a[i], b_cur, acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < NJ) b_cur = b_nxt;
      }
    }
  };

  // s_waitcnt vmcnt(0): the direct-to-LDS loads of this wave have landed
  constexpr int kWaitVm0 = 0x0F70;
  // K step ks on stage (w, a) while the next activation tile goes to a_next
  const bool lora16 = !kBwd && p.r <= 16;  // a LoRA step then fills only its first K half
  auto step = [&](int ks, const uint8_t* w, const uint8_t* a, uint8_t* a_next) {
    if (ks + 1 < nk) copy_act(a_next);
    if (active) {
      mfma_step(w, a, 0);
      if (!(lora16 && ks >= nk)) mfma_step(w, a, 1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  // nk steps of W' and activations, then the LoRA steps (filled by the producers)
  const int nsteps = nk + (lora ? (p.r + 31) / 32 : 0);
  copy_act(lds.a[0]);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();  // stage 0 ready
#pragma unroll 1
  for (int ks = 0; ks < nsteps; ks += 2) {
    step(ks, lds.w[0], lds.a[0], lds.a[1]);
    if (ks + 1 < nsteps) step(ks + 1, lds.w[1], lds.a[1], lds.a[0]);
  }

  // Split tile: arrival order decides who stores its sum and who finishes.
  // The finisher adds the stored sum through a buffer resource that is empty
  // (every load reads 0) for whole tiles, so all paths run the same in-place
  // adds and the accumulators are not copied.
  uint32_t part_bytes = 0;
  const int sidx = split ? split - 1 : 0;
  float* part_base = p.partial ? p.partial + (size_t)sidx * (lg2::BF * lg2::BT) : nullptr;
  const uint32_t poff = (uint32_t)(wave * (NI * NJ * 1024) + 16 * lane);  // [wave][i][j][lane] f32x4
  if (kPieces) {
    // one K piece (few-tile mode): its fp32 sums, in the layout below, in
    // slot tile * pieces + piece (the work item's index) of piece_out
    // (reduce_pieces_kernel reads no row past M)
    if (!active) return;
    const brsrc_t r_pl = make_rsrc(p.piece_out + (size_t)blockIdx.x * (lg2::BF * lg2::BT), lg2::BF * lg2::BT * 4);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), r_pl,
                                               (int)(poff + (i * NJ + j) * 1024), 0, 0);
    return;
  }
  if (split) {
    uint32_t* sync = p.split_sync + 2 * sidx;
    if (tid == 0) *lds_word = __hip_atomic_fetch_add(sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*lds_word == 0u) {
      const brsrc_t r_out = make_rsrc(part_base, lg2::BF * lg2::BT * 4);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), r_out,
                                                 (int)(poff + (i * NJ + j) * 1024), 0, kAuxDevice);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are done
      __syncthreads();
      if (tid == 0) __hip_atomic_store(sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    bool ready = false;
    for (uint32_t it = 0; it < kSplitSpinLimit; ++it) {
      if (__hip_atomic_load(sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        ready = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    // A wait that runs out leaves the tile without the other half's sum:
    // the give-up word after the hand-off words records it for the host
    // (qlora_linear_check), instead of the tile being wrong silently.
    if (!ready && tid == 0)
      __hip_atomic_store(p.split_sync + 2 * p.nsplit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    part_bytes = lg2::BF * lg2::BT * 4;
  }
  {
    const brsrc_t r_part = make_rsrc(part_base, part_bytes);
    // one row of fragments in flight at a time; the empty asm pins each sum
    // in its accumulator registers (otherwise the adds sink to the stores
    // below and the loaded values are spilled)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[i][j] += __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(r_part, (int)(poff + (i * NJ + j) * 1024), 0, kAuxDevice));
        asm volatile("" : "+v"(acc[i][j]));
      }
    }
  }
  if (p.add) {
    // an fp32 term of the output computed elsewhere, added once per tile
    // before the single rounding (M N 4 < 2^32 bytes; rows past M read 0)
    const uint32_t add_bytes = (uint32_t)(p.M * p.N * 4);
    const brsrc_t r_add = make_rsrc(p.add, add_bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t t = t0 + wt + 16 * j + lr;
        const int64_t f = f0 + wf + 16 * i + 4 * lq;
        const bool ok = t < p.M && f < p.N;
        acc[i][j] += __builtin_bit_cast(f32x4, bload128(r_add, ok ? (uint32_t)((t * p.N + f) * 4) : add_bytes));
        asm volatile("" : "+v"(acc[i][j]));
      }
    }
  }

  // ---- store (bf16) through LDS, so that global writes are whole rows ----
  // The K loop's last barrier has freed all tiles.  Each wave stages its
  // WT x WF tile as [WT rows][2 WF bytes] in 16 KB of its own (waves 2w',
  // 2w' + 1 share one 32 KB tile array).  The 16-byte chunk c of row t sits at
  // position c ^ (t % 16) for 256-byte rows and c ^ ((t / 2) % 8) for 128-byte
  // rows, so the 8-byte writes (16 rows x 4 lanes) and the 16-byte row reads
  // are free of bank conflicts.
  constexpr int CPR = WF / 8;  // 16-byte chunks per staged row
  auto spos = [](int row, int c) { return CPR == 16 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7)); };
  uint8_t* stg = ((wave >> 1) == 0 ? lds.a[0] : (wave >> 1) == 1 ? lds.a[1] : (wave >> 1) == 2 ? lds.w[0] : lds.w[1]) +
                 16384 * (wave & 1);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = 16 * j + lr;
      const int col = 16 * i + 4 * lq;  // 4 features: chunk col / 8, half (col / 4) % 2
      const f32x4 v = acc[i][j];
      *reinterpret_cast<u32x2*>(stg + row * (2 * WF) + (spos(row, col >> 3) << 4) + ((col & 4) << 1)) =
          u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's writes are done
  __builtin_amdgcn_wave_barrier();
  const bool vec_ok = (p.N & 7) == 0;
  // Whole-row stores carry the non-temporal hint (and sc0): the output is
  // not read again by this kernel, and streaming it past the caches keeps
  // the last-level cache for the next kernel's input (the g pass after the
  // forward ran 46 -> 41 us, the step 1.7 % faster).  M N 2 < 2^31 bytes.
  const brsrc_t r_out = make_rsrc(p.out, (uint32_t)(p.M * p.N * 2));
  constexpr int kAuxStream = 3;  // buffer cache policy: sc0 | nt
  const int c = lane % CPR;
  const int64_t f = f0 + wf + 8 * c;
#pragma unroll
  for (int k = 0; k < WT * CPR / 64; ++k) {
    const int row = (64 / CPR) * k + lane / CPR;
    const int64_t t = t0 + wt + row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * (2 * WF) + (spos(row, c) << 4));
    if (t >= p.M || f >= p.N) continue;
    uint16_t* dst = p.out + t * p.N + f;
    if (vec_ok && f + 8 <= p.N) {
      __builtin_amdgcn_raw_buffer_store_b128(v, r_out, (int)((t * p.N + f) * 2), 0, kAuxStream);
    } else {
      for (int e = 0; e < 8; ++e)
        if (f + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// kPieces: few-tile mode (every tile as p.pieces K pieces), a separate
// instantiation so that the other kernels' register allocation is untouched.
template <bool kBwd, bool kPieces, bool kSkip>
__global__ __launch_bounds__(lg2::kThreads) void linear_gemm_kernel(GemmArgs p, Nf4Table tab) {
  using T = lg2::Tile<kBwd>;
  __shared__ __align__(16) uint8_t sw0[T::W];
  __shared__ __align__(16) uint8_t sw1[T::W];
  __shared__ __align__(16) uint8_t sa0[lg2::ATILEB];
  __shared__ __align__(16) uint8_t sa1[lg2::ATILEB];
  __shared__ uint32_t lds_word;
  const lg2::Lds lds{{sw0, sw1}, {sa0, sa1}};
  const int tid = threadIdx.x;
  const int nk = (int)((p.K + lg2::BK - 1) / lg2::BK);
  // work item -> tile and K range: full tiles first (XCD-aware order), then
  // the K halves of the split tiles, which run in the last round
  int tile, k0 = 0, ks = nk, split = 0;
  bool lora = true;
  if (kPieces) {
    const int piece = (int)blockIdx.x % p.pieces;
    tile = (int)blockIdx.x / p.pieces;
    k0 = piece * nk / p.pieces;
    ks = (piece + 1) * nk / p.pieces - k0;
    lora = piece == p.pieces - 1;
  } else if ((int)blockIdx.x < p.full_tiles) {
    tile = xcd_remap_l(blockIdx.x, p.full_tiles);
  } else {
    const int w = (int)blockIdx.x - p.full_tiles;
    const int half = w & 1;
    tile = p.full_tiles + (w >> 1);
    split = (w >> 1) + 1;
    k0 = half ? nk / 2 : 0;
    ks = half ? nk - nk / 2 : nk / 2;
    lora = half != 0;
  }
  const int tile_f = tile % p.tiles_f;
  const int tile_t = tile / p.tiles_f;
  const int64_t f0 = (int64_t)tile_f * lg2::BF;
  const int64_t t0 = (int64_t)tile_t * lg2::BT;
  // wave-uniform role split; both roles pass the same number of barriers
  if (tid >= 64 * lg2::kMfmaWaves)
    gemm_producer<kBwd>(p, tab, lds, tid - 64 * lg2::kMfmaWaves, f0, t0, k0, ks, lora, split, &lds_word);
  else
    gemm_consumer<kBwd, kPieces, kSkip>(p, lds, tid, f0, t0, k0, ks, lora, split, &lds_word);
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Compute units of the current device (256 when no device answers).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

// Few tiles (at most half the CUs, e.g. 33..256 tokens at 4096 - 14336
// features): every tile runs as P K pieces, P = min(CUs / tiles, 16) with
// at least 8 K steps per piece, so up to all CUs stream the weight.  With
// P >= 3 the P fp32 tile sums (tiles P 2^18 <= CUs 2^18 bytes) are added in
// piece order by a separate pass, so the result does not depend on which
// piece ends first.  With P = 2 the two halves meet through the K-split
// hand-off instead (commutative, so also order-free): no second pass, and
// half the fp32 traffic (the 70B block's k and v forwards: 128 tiles).
constexpr int kMaxPieces = 16;
static int64_t tiles_of(int64_t M, int64_t N) { return ((N + lg2::BF - 1) / lg2::BF) * ((M + lg2::BT - 1) / lg2::BT); }
static int few_tile_pieces(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = tiles_of(M, N);
  const int cus = device_cus();
  const int64_t nk = (K + lg2::BK - 1) / lg2::BK;
  if (tiles * 2 > cus) return 1;
  int64_t pc = cus / tiles;
  if (pc > kMaxPieces) pc = kMaxPieces;
  while (pc > 1 && nk / pc < 8) --pc;
  return (int)pc;
}
int gemm_pieces(int64_t M, int64_t N, int64_t K) {
  const int pc = few_tile_pieces(M, N, K);
  return pc == 2 ? 1 : pc;
}

// Tiles split in two K halves that meet through the hand-off: every tile
// when the few-tile mode would use two pieces; otherwise, when the tile
// count leaves at most half a round for the last pass, those last tiles:
// with T tiles on C CUs (one workgroup per CU), the last T mod C <= C/2
// tiles become 2 (T mod C) half-length work items, so the last round fills
// the chip for half the time instead of half the chip for the full time.
// Either way the two halves of a tile run in the same round.
int gemm_split_tiles(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = tiles_of(M, N);
  const int cus = device_cus();
  const int64_t rem = tiles % cus;
  const int64_t nk = (K + lg2::BK - 1) / lg2::BK;
  if (nk < 8) return 0;
  if (tiles * 2 <= cus) return few_tile_pieces(M, N, K) == 2 ? (int)tiles : 0;
  if (tiles < cus || rem == 0 || rem > cus / 2) return 0;
  return (int)rem;
}

// Finishes a few-tile GEMM: out = bf16(((piece 0 + piece 1) + ...) + add).
// Thread g takes fragment item g % 16384 (4 features of one token) of tile
// g / 16384 from every piece's slot, in the consumer's [wave][i][j][lane]
// order, so that the slot reads are whole 1 KB rows.
template <bool kBwd>
__global__ __launch_bounds__(256) void reduce_pieces_kernel(GemmArgs p) {
  constexpr int WF = kBwd ? 64 : 128;
  constexpr int WT = 128 * 64 / WF;
  constexpr int NI = WF / 16, NJ = WT / 16;
  constexpr int kItems = lg2::BF * lg2::BT / 4;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int tile = (int)(g / kItems);
  const int rem = (int)(g % kItems);
  const int wave = rem / (NI * NJ * 64);
  const int ij = (rem / 64) % (NI * NJ);
  const int lane = rem % 64;
  const int i = ij / NJ, j = ij % NJ;
  const int64_t t = (int64_t)(tile / p.tiles_f) * lg2::BT + (wave / (lg2::BF / WF)) * WT + 16 * j + (lane & 15);
  const int64_t f = (int64_t)(tile % p.tiles_f) * lg2::BF + (wave % (lg2::BF / WF)) * WF + 16 * i + 4 * (lane >> 4);
  if (tile >= p.tiles_f * p.tiles_t || t >= p.M || f >= p.N) return;
  const float* slot = p.piece_out + (size_t)tile * p.pieces * kItems * 4 + (size_t)rem * 4;
  f32x4 v = *reinterpret_cast<const f32x4*>(slot);
  for (int q = 1; q < p.pieces; ++q) v += *reinterpret_cast<const f32x4*>(slot + (size_t)q * kItems * 4);
  const int64_t o = t * p.N + f;
  if ((p.N & 3) == 0) {
    if (p.add) v += *reinterpret_cast<const f32x4*>(p.add + o);
    *reinterpret_cast<u32x2*>(p.out + o) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (f + e >= p.N) break;
    const float a = v[e] + (p.add ? p.add[o + e] : 0.0f);
    p.out[o + e] = (uint16_t)(pack_bf16x2(a, 0.0f) & 0xFFFFu);
  }
}

size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const int pc = gemm_pieces(M, N, K);
  if (pc > 1) return (size_t)pc * tiles_of(M, N) * lg2::BF * lg2::BT * sizeof(float);
  const size_t ns = (size_t)gemm_split_tiles(M, N, K);
  if (!ns) return 0;
  return ns * lg2::BF * lg2::BT * sizeof(float) + (((2 * ns + 1) * sizeof(uint32_t) + 255) / 256) * 256;
}

// Byte offset, inside the split workspace, of the give-up word of a GEMM
// whose last round is split in K, or -1 when the GEMM has no hand-off.
int64_t gemm_giveup_offset(int64_t M, int64_t N, int64_t K) {
  if (gemm_pieces(M, N, K) > 1) return -1;
  const int64_t ns = gemm_split_tiles(M, N, K);
  if (!ns) return -1;
  return ns * lg2::BF * lg2::BT * (int64_t)sizeof(float) + 2 * ns * (int64_t)sizeof(uint32_t);
}

// The hand-off words of a GEMM on split_ws (none without a split or with K
// pieces), for the kernel before it to clear.
SyncZero gemm_split_sync(int64_t M, int64_t N, int64_t K, void* split_ws) {
  SyncZero z;
  if (!split_ws || gemm_pieces(M, N, K) > 1) return z;
  const int64_t ns = gemm_split_tiles(M, N, K);
  if (!ns) return z;
  z.p = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(split_ws) + (size_t)ns * lg2::BF * lg2::BT * sizeof(float));
  z.n = (int)(2 * ns + 1);
  return z;
}

template <bool kPieces>
static void launch_gemm_kernel(bool bwd, bool skip, dim3 grid, const GemmArgs& p, const Nf4Table& tab,
                               hipStream_t stream) {
  const dim3 block(lg2::kThreads);
  if (bwd) {
    if (skip)
      hipLaunchKernelGGL((linear_gemm_kernel<true, kPieces, true>), grid, block, 0, stream, p, tab);
    else
      hipLaunchKernelGGL((linear_gemm_kernel<true, kPieces, false>), grid, block, 0, stream, p, tab);
  } else {
    if (skip)
      hipLaunchKernelGGL((linear_gemm_kernel<false, kPieces, true>), grid, block, 0, stream, p, tab);
    else
      hipLaunchKernelGGL((linear_gemm_kernel<false, kPieces, false>), grid, block, 0, stream, p, tab);
  }
}

// split_ws: gemm_split_ws_bytes(M, N, K) bytes (16-byte aligned), or null to
// run every tile whole.  sync_zeroed: the words of gemm_split_sync were
// cleared by an earlier kernel on the stream (else a small launch clears them).
static void launch_linear_gemm(bool bwd, const GemmArgs& a, void* split_ws, const Nf4Table& tab,
                               hipStream_t stream, bool sync_zeroed) {
  GemmArgs p = a;
  p.tiles_f = (int)((p.N + lg2::BF - 1) / lg2::BF);
  p.tiles_t = (int)((p.M + lg2::BT - 1) / lg2::BT);
  const int tiles = p.tiles_f * p.tiles_t;
  const int pc = split_ws ? gemm_pieces(p.M, p.N, p.K) : 1;
  if (pc > 1) {
    p.pieces = pc;
    p.piece_out = static_cast<float*>(split_ws);
    p.full_tiles = tiles;
    p.nsplit = 0;
    p.partial = nullptr;
    p.split_sync = nullptr;
    launch_gemm_kernel<true>(bwd, p.M % lg2::BT != 0, dim3(tiles * pc), p, tab, stream);
    const unsigned rblocks = (unsigned)tiles * (lg2::BF * lg2::BT / 4 / 256);
    if (bwd)
      hipLaunchKernelGGL(reduce_pieces_kernel<true>, dim3(rblocks), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(reduce_pieces_kernel<false>, dim3(rblocks), dim3(256), 0, stream, p);
    return;
  }
  const int ns = split_ws ? gemm_split_tiles(p.M, p.N, p.K) : 0;
  p.full_tiles = tiles - ns;
  p.nsplit = ns;
  p.partial = nullptr;
  p.split_sync = nullptr;
  if (ns) {
    p.partial = static_cast<float*>(split_ws);
    p.split_sync = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(split_ws) +
                                               (size_t)ns * lg2::BF * lg2::BT * sizeof(float));
    if (!sync_zeroed)
      hipLaunchKernelGGL(zero_u32_kernel, dim3((2 * ns + 1 + 255) / 256), dim3(256), 0, stream, p.split_sync,
                         2 * ns + 1);
  }
  const int grid = tiles + ns;
  launch_gemm_kernel<false>(bwd, p.M % lg2::BT != 0, dim3(grid), p, tab, stream);
}

void launch_fwd_gemm(const uint16_t* x, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                     const uint16_t* B, const float* u, uint16_t* h, int64_t M, int64_t n, int64_t m, int r,
                     float s, void* split_ws, const Nf4Table& tab, hipStream_t stream, bool sync_zeroed) {
  GemmArgs p{};
  p.act = x; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.lora_a = B; p.lora_b = u; p.out = h;
  p.M = M; p.K = n; p.N = m; p.wn = n; p.wm = m; p.r = r; p.s = s;
  launch_linear_gemm(false, p, split_ws, tab, stream, sync_zeroed);
}

// g is M x m_pad (m_pad = m, or m rounded up to 64 with zero columns when
// m % 8 != 0, so every 16-byte chunk of the tensor is whole).
// add: M x n fp32 added to the result before its rounding, or null; r = 0
// runs no LoRA steps.
void launch_dgrad_gemm(const uint16_t* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                       const uint16_t* A, const float* v, uint16_t* gx, int64_t M, int64_t n, int64_t m,
                       int64_t m_pad, int r, float s, void* split_ws, const Nf4Table& tab, hipStream_t stream,
                       const float* add, bool sync_zeroed) {
  GemmArgs p{};
  p.act = g; p.codes = codes; p.absmax8 = absmax8; p.c2 = c2; p.lora_a = A; p.lora_b = v; p.out = gx; p.add = add;
  p.M = M; p.K = m_pad; p.N = n; p.wn = n; p.wm = m; p.r = r; p.s = s;
  launch_linear_gemm(true, p, split_ws, tab, stream, sync_zeroed);
}

}  // namespace qlora
