// Forward of the adapted linear layer for small token counts (M <= 32):
//   h = x W'^T + s u B^T,  u = x A^T
// "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3), with W' = dequant(W0) as
// in the dequantization passage of Step 3 and "How QLoRA Works" (BF16
// compute type).  With a few tokens every packed weight is used by at most
// 32 tokens, so the pass is bound by streaming the 4-bit codes from HBM.
//
// Design (one or several layers per launch, all sharing the token count M):
//   - the (out-feature x K) plane of each layer is cut into work items of
//     up to 16 blocks of 16 features x one K chunk of 2048, sized so that a
//     launch has about two workgroups per CU;
//   - each of a workgroup's 4 waves takes a quarter of the chunk (512 k) for
//     all the item's feature blocks and stages only its own quarter of x
//     (M x 512 bf16) in LDS, with line-coalesced loads, so no wave waits for
//     another before its main loop;
//   - a wave streams the codes as MFMA A fragments: per 16-feature block and
//     256-k piece every lane loads 32 contiguous bytes (8 code words, one
//     64-weight block, so one magnitude table per 64 weights), dequantizes a
//     word straight into the 8 bf16 of one 16x16x32 MFMA A operand, and reads
//     the matching x fragment from LDS;
//   - u = x A^T runs in extra workgroups of the same launch, one per layer
//     and K chunk, next to the dequantizing ones (a launch fits in one round
//     of the chip, so they add no tail);
//   - the four waves' partial sums are reduced through LDS in a fixed order
//     and written as fp32 partials (h and u per K chunk); a second launch sums
//     the chunks in order and adds s u B^T with MFMAs.
// Within a 256-k piece, MFMA step q takes from lane group g (lanes 16g ..
// 16g + 15) the k range 64g + 8q .. 64g + 8q + 7: the sum over k is the same,
// only grouped differently, and both operands use the same grouping.
#include "qlora_common.h"

namespace qlora {

namespace sm {
constexpr int KC = 2048;     // K per chunk
constexpr int PIECE = 256;   // k per piece (32 bytes of codes per lane)
constexpr int kPW = (KC / 4) / PIECE;   // pieces per wave and feature block (2)
constexpr int kDepth = 2;    // code pieces in flight per wave (deeper queues only delay x)
constexpr int kMaxLayers = 8;
constexpr int kWGsPerCU = 2;            // workgroups per CU a launch is sized for
constexpr int XCPR = KC / 4 / 8;         // 16-byte chunks of one token row of a wave's x quarter
constexpr int XRPL = 64 / XCPR;          // token rows per 64-lane load of the x quarter
}  // namespace sm

// feature blocks (of 16) per workgroup at most: 16 for up to 16 tokens, 8 for 17..32
template <int TB>
struct SmallTile {
  static constexpr int FBMAX = 16 / TB;
};

struct SmallLayer {
  const uint16_t* x;        // M x n
  const uint8_t* codes;
  const uint8_t* absmax8;
  const float* c2;
  const uint16_t* A;        // r x n
  const uint16_t* B;        // m x r
  uint16_t* h;              // M x m
  float* u_out;             // M x r or null
  float* hpart;             // [nkc][M][m]
  float* upart;             // [nkc][M][r]
  int64_t n, m;
  int r;
  float s;
  int nkc;                  // K chunks
  int fbw;                  // 16-feature blocks per workgroup
  int ngroups;              // feature groups (fbw blocks each)
  int wg_begin;             // first workgroup of this layer in the launch
  int u_begin;              // first u workgroup of this layer (after all dequantizing ones)
  int64_t out_begin;        // first finishing workgroup of this layer
  DropoutDev drop;          // dropout on x as the adapter reads it
  float u_scale;            // u = u_scale * (masked x) A^T: 1 / (1 - p), or 1
};

struct SmallArgs {
  SmallLayer L[sm::kMaxLayers];
  int count;
  int M;
  int main_wgs;             // dequantizing workgroups; u workgroups follow
};

// which = 0: dequantizing workgroup, 1: finishing workgroup, 2: u workgroup
__device__ __forceinline__ int find_layer(const SmallArgs& a, int64_t key, int which) {
  int li = 0;
#pragma unroll
  for (int i = 1; i < sm::kMaxLayers; ++i)
    if (i < a.count &&
        (which == 1 ? a.L[i].out_begin : (int64_t)(which == 2 ? a.L[i].u_begin : a.L[i].wg_begin)) <= key)
      li = i;
  return li;
}

// A wave's x quarter in LDS: token row t holds KC / 4 bf16 (XCPR chunks of
// 16 B); chunk c of row t sits at position c ^ (t & 15), so the 16 tokens of
// one MFMA B fragment hit 16 different bank groups.
__device__ __forceinline__ uint32_t xsw(int t, int c) {
  return (uint32_t)(t * (sm::KC / 4 * 2) + ((c ^ (t & 15)) << 4));
}

// u_chunk = x_chunk A_chunk^T for one layer and K chunk: each wave stages its
// quarter of x and runs 16 MFMA steps per rank block of 16 (A fragments two
// steps ahead); the four waves' sums are reduced through LDS in a fixed order.
template <int TB>
__device__ void small_u_chunk(const SmallArgs& a, uint8_t* lds, f32x4* ured) {
  constexpr int MP = 16 * TB;
  constexpr int QK = sm::KC / 4;
  constexpr int XQB = MP * QK * 2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int g = lane >> 4;
  const int li = find_layer(a, blockIdx.x, 2);
  const SmallLayer& Ly = a.L[li];
  const int kc = (int)blockIdx.x - Ly.u_begin;
  const int M = a.M;
  const int64_t K = Ly.n;
  const int r = Ly.r;
  const int64_t k0 = (int64_t)kc * sm::KC;
  const int kq = wave * QK;
  uint8_t* xq = lds + wave * XQB;
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const brsrc_t rx = make_rsrc(Ly.x, xbytes);
#pragma unroll
  for (int i = 0; i < MP / sm::XRPL; ++i) {
    const int t = sm::XRPL * i + lane / sm::XCPR;
    const int c = lane % sm::XCPR;
    const int64_t k = k0 + kq + 8 * c;
    const bool ok = t < M && k < K;
    u32x4 w = bload128(rx, ok ? (uint32_t)(((int64_t)t * K + k) * 2) : xbytes);
    if (Ly.drop.on && ok) w = dropout8(Ly.drop, (uint64_t)((int64_t)t * K + k), w);  // element t K + k
    *reinterpret_cast<u32x4*>(xq + xsw(t, c)) = w;
  }
  const uint32_t arbytes = (uint32_t)((int64_t)r * K * 2);
  const brsrc_t ra = make_rsrc(Ly.A, arbytes);
  float* up = Ly.upart + (int64_t)kc * M * r;
  const int RBn = (r + 15) >> 4;
  for (int rb = 0; rb < RBn; ++rb) {
    constexpr int NJ = QK / 32;
    const int q = 16 * rb + lr;
    auto load_a = [&](int j) -> u32x4 {
      const int64_t k = k0 + kq + 32 * j + 8 * g;
      const bool ok = q < r && k < K;
      return bload128(ra, ok ? (uint32_t)(((int64_t)q * K + k) * 2) : arbytes);
    };
    f32x4 ua[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) ua[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 an0 = load_a(0), an1 = load_a(1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const u32x4 af = an0;
      an0 = an1;
      if (j + 2 < NJ) an1 = load_a(j + 2);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(xq + xsw(16 * tb + lr, 4 * j + g));
        ua[tb] = mfma16x16x32(af, bf, ua[tb]);
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) ured[(wave * TB + tb) * 64 + lane] = ua[tb];
    __syncthreads();
    if (tid < TB * 64) {
      const int ln = tid & 63, tb = tid >> 6;
      f32x4 v = ured[(0 * TB + tb) * 64 + ln];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += ured[(w * TB + tb) * 64 + ln];
      // rows are adapter rows 16 rb + 4 (ln / 16) + e, column token 16 tb + ln % 16
      const int t = 16 * tb + (ln & 15);
      if (t < M) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qq = 16 * rb + 4 * (ln >> 4) + e;
          if (qq < r) up[(int64_t)t * r + qq] = v[e];
        }
      }
    }
    __syncthreads();
  }
}

template <int TB>
__global__ __launch_bounds__(256) void small_fwd_kernel(SmallArgs a, Nf4Table tab) {
  constexpr int MP = 16 * TB;                 // padded token count
  constexpr int QK = sm::KC / 4;              // k per wave quarter
  constexpr int XQB = MP * QK * 2;            // one wave's x quarter: 16 KB per token block
  constexpr int FBMAX = SmallTile<TB>::FBMAX;
  __shared__ __align__(16) uint8_t lds[4 * XQB];
  __shared__ __align__(16) f32x4 ured[4 * TB * 64];   // per-wave u partials of one rank block
  if ((int)blockIdx.x >= a.main_wgs) {
    small_u_chunk<TB>(a, lds, ured);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int g = lane >> 4;

  const int li = find_layer(a, blockIdx.x, 0);
  const SmallLayer& Ly = a.L[li];
  const int local = blockIdx.x - Ly.wg_begin;
  const int kc = local % Ly.nkc;
  const int fg = local / Ly.nkc;
  const int M = a.M;
  const int64_t K = Ly.n;
  const int64_t m = Ly.m;
  const int64_t k0 = (int64_t)kc * sm::KC;
  const int kq = wave * QK;                   // this wave's quarter within the chunk
  const int64_t f_base = (int64_t)fg * Ly.fbw * 16;
  const int64_t nfb = (m + 15) / 16;
  const int nb = (int)((nfb - (int64_t)fg * Ly.fbw) < Ly.fbw ? (nfb - (int64_t)fg * Ly.fbw) : Ly.fbw);
  uint8_t* xq = lds + wave * XQB;

  // ---- this wave's x quarter: x[0:MP][k0 + kq : + QK] (zeros past M or K);
  // load i covers token rows XRPL i .. + XRPL - 1, each QK * 2 bytes contiguous ----
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const brsrc_t rx = make_rsrc(Ly.x, xbytes);
  u32x4 xr[MP / sm::XRPL];
#pragma unroll
  for (int i = 0; i < MP / sm::XRPL; ++i) {
    const int t = sm::XRPL * i + lane / sm::XCPR;
    const int64_t k = k0 + kq + 8 * (lane % sm::XCPR);
    const bool ok = t < M && k < K;
    xr[i] = bload128(rx, ok ? (uint32_t)(((int64_t)t * K + k) * 2) : xbytes);
  }

  // ---- codes of this wave: lane's 64-weight block for (feature block b, piece p)
  // is row f = f_base + 16 b + lr, k = k0 + kq + 256 p + 64 g ----
  const uint32_t cbytes = (uint32_t)(m * K / 2);
  const uint32_t abytes = (uint32_t)(m * K / kBlock);
  const uint32_t c2bytes = (uint32_t)(((m * K / kBlock + kGroupBlocks - 1) / kGroupBlocks) * 4);
  const brsrc_t rc = make_rsrc(Ly.codes, cbytes);
  const brsrc_t rab = make_rsrc(Ly.absmax8, abytes);
  const brsrc_t rc2 = make_rsrc(Ly.c2, c2bytes);
  // No per-lane bounds checks: rows past m lie past the end of the packed
  // weight (the buffer range reads them as 0); k past K within a row reads the
  // next row's codes, which meet the zero-padded x and add nothing.  Blocks
  // past nb (prefetched, never used) get an offset past the end: the choice
  // is the same for the whole wave, so it costs no vector instruction.
  const uint32_t row_step = (uint32_t)(16 * K / 2);   // bytes of codes per feature block
  const uint32_t cbase_off = (uint32_t)(((f_base + lr) * K + k0 + kq + 64 * g) / 2);
  auto load_codes = [&](int b, int p, u32x4& c0, u32x4& c1, uint32_t& ab, float& cs) {
    const uint32_t off = cbase_off + (b < nb ? (uint32_t)b * row_step + (uint32_t)p * (sm::PIECE / 2) : cbytes);
    c0 = bload128(rc, off);
    c1 = bload128(rc, off + 16);
    const uint32_t blk = off / (kBlock / 2);
    ab = bload8(rab, blk);
    cs = __uint_as_float(bload32(rc2, (blk >> 8) << 2));
  };

  // first pieces' codes in flight while x lands
  constexpr int NI = FBMAX * sm::kPW;   // (block, piece) iterations of a wave
  u32x4 cq0[sm::kDepth], cq1[sm::kDepth];
  uint32_t abq[sm::kDepth];
  float csq[sm::kDepth];
#pragma unroll
  for (int i = 0; i < sm::kDepth; ++i) load_codes(i / sm::kPW, i % sm::kPW, cq0[i], cq1[i], abq[i], csq[i]);

  // x quarter to LDS: read back only by this wave (LDS keeps a wave's
  // accesses in order), so no workgroup barrier.  Up to 16 tokens the wave
  // then reads all its MFMA B fragments once and keeps them in registers (64
  // VGPRs: fragment (p, q) of lane (lr, g) is x[lr][kq + 256 p + 64 g + 8 q ..
  // + 7], the same for every feature block).
  constexpr bool kXReg = TB == 1;
  u32x4 xf[kXReg ? sm::kPW * 8 : 1];
#pragma unroll
  for (int i = 0; i < MP / sm::XRPL; ++i)
    *reinterpret_cast<u32x4*>(xq + xsw(sm::XRPL * i + lane / sm::XCPR, lane % sm::XCPR)) = xr[i];
  if constexpr (kXReg) {
#pragma unroll
    for (int j = 0; j < sm::kPW * 8; ++j)
      xf[j] = *reinterpret_cast<const u32x4*>(xq + xsw(lr, (sm::PIECE * (j >> 3) + 64 * g) / 8 + (j & 7)));
  }

  // ---- main loop over (feature block, piece), codes kDepth iterations ahead ----
  f32x4 acc[FBMAX][TB];
#pragma unroll
  for (int b = 0; b < FBMAX; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[b][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int b = i / sm::kPW, p = i % sm::kPW, slot = i % sm::kDepth;
    if (b >= nb) break;
    const u32x4 c0 = cq0[slot], c1 = cq1[slot];
    const MagLut L = make_mag_lut(tab, e4m3_decode(abq[slot]) * csq[slot]);
    if (i + sm::kDepth < NI)
      load_codes((i + sm::kDepth) / sm::kPW, (i + sm::kDepth) % sm::kPW, cq0[slot], cq1[slot], abq[slot], csq[slot]);
    // keep the prefetch where it is: the scheduler would otherwise sink these
    // loads next to their use kDepth iterations later
    __builtin_amdgcn_sched_barrier(0);
    const int cbase = (sm::PIECE * p + 64 * g) / 8;   // 16-byte chunk of k for step 0
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t o[4];
      mag_dequant8(L, (q < 4 ? c0 : c1)[q & 3], o);
      const u32x4 af = u32x4{o[0], o[1], o[2], o[3]};
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 bf = kXReg ? xf[8 * p + q] : *reinterpret_cast<const u32x4*>(xq + xsw(16 * tb + lr, cbase + q));
        acc[b][tb] = mfma16x16x32(af, bf, acc[b][tb]);
      }
    }
  }

  // ---- reduce the four waves' partial sums through LDS (x is no longer
  // needed), FBR feature blocks per round so that the buffer fits the x
  // quarters' LDS ----
  constexpr int FBR = (4 * XQB) / (4 * TB * 64 * 16) < FBMAX ? (4 * XQB) / (4 * TB * 64 * 16) : FBMAX;
  static_assert(FBR >= 1 && FBMAX % FBR == 0, "reduction rounds");
  f32x4* red = reinterpret_cast<f32x4*>(lds);   // [wave][b - b0][tb][lane]
  float* hp = Ly.hpart + (int64_t)kc * M * m;
#pragma unroll
  for (int b0 = 0; b0 < FBMAX; b0 += FBR) {
    if (b0 >= nb) break;
    __syncthreads();
#pragma unroll
    for (int b = b0; b < b0 + FBR; ++b)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        if (b < nb) red[((wave * FBR + (b - b0)) * TB + tb) * 64 + lane] = acc[b][tb];
    __syncthreads();
    const int nbr = nb - b0 < FBR ? nb - b0 : FBR;
    for (int idx = tid; idx < nbr * TB * 64; idx += 256) {
      const int ln = idx & 63;
      const int tb = (idx >> 6) % TB;
      const int br = (idx >> 6) / TB;
      f32x4 v = red[((0 * FBR + br) * TB + tb) * 64 + ln];
#pragma unroll
      for (int w = 1; w < 4; ++w) v += red[((w * FBR + br) * TB + tb) * 64 + ln];
      // C layout: lane ln holds token 16 tb + ln % 16, features 4 (ln / 16) + e of block b
      const int t = 16 * tb + (ln & 15);
      const int64_t f = f_base + 16 * (b0 + br) + 4 * (ln >> 4);
      if (t < M) {
        if ((m & 3) == 0 && f + 4 <= m) {
          *reinterpret_cast<f32x4*>(hp + (int64_t)t * m + f) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (f + e < m) hp[(int64_t)t * m + f + e] = v[e];
        }
      }
    }
  }
}

// h[t][f] = bf16(sum_c hpart[c][t][f] + s * sum_q u[t][q] B[f][q]) with
// u[t][q] = sum over chunks (in chunk order) of upart.  One
// workgroup (4 waves) finishes 64 features of one layer for every token, in
// the MFMA C layout: wave w takes feature block w (16 features); lane (lr, g)
// holds features 4 g .. 4 g + 3 of token 16 tb + lr, which is one 16-byte
// vector of each chunk's partial.  s u B^T runs as MFMAs with the B rows as A
// operand and s u^T, split into bf16 hi + lo, as B operand.  The layer's
// first workgroup also writes u_out.
//
// With 16-byte rows (r a multiple of 8, m of 4) every lane loads what it
// needs directly, all loads independent: its 16-byte vector of each chunk's
// h partial, its B fragment, and the u partials of its 8 ranks, which it sums
// in chunk order itself (every wave of a tile repeats this small sum).
template <int TB>
__device__ void small_reduce_aligned(const SmallLayer& Ly, int tile, int M) {
  const int64_t m = Ly.m;
  const int r = Ly.r;
  const int nkc = Ly.nkc;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;
  const int64_t fa = (int64_t)tile * 64 + 16 * wave + lr;   // B row of this lane's A fragment
  const int64_t fc = (int64_t)tile * 64 + 16 * wave + 4 * g;  // this lane's 4 output features
  const int QB = (r + 31) / 32;
  constexpr int kQB = kMaxRank / 32;
  constexpr int kC = 8;                                       // chunks per batch of loads
  const uint32_t bbytes = (uint32_t)(m * r * 2);
  const brsrc_t rbm = make_rsrc(Ly.B, bbytes);
  const uint32_t hbytes = (uint32_t)((int64_t)nkc * M * m * 4);
  const brsrc_t rhp = make_rsrc(Ly.hpart, hbytes);
  const uint32_t ubytes = (uint32_t)((int64_t)nkc * M * r * 4);
  const brsrc_t rup = make_rsrc(Ly.upart, ubytes);
  // B fragment of rank block qb: B[fa][32 qb + 8 g .. + 7] (zeros past m or r)
  auto load_b = [&](int qb) {
    const int q0 = 32 * qb + 8 * g;
    return bload128(rbm, (qb < QB && fa < m && q0 < r) ? (uint32_t)((fa * r + q0) * 2) : bbytes);
  };
  // B operand of one rank block: s u as bf16 hi + lo
  auto su_split = [&](const f32x4& u0, const f32x4& u1, u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = Ly.s * (e < 2 ? u0[2 * e] : u1[2 * e - 4]);
      const float v1 = Ly.s * (e < 2 ? u0[2 * e + 1] : u1[2 * e - 3]);
      float h0, l0, h1, l1;
      split_bf16(v0, h0, l0);
      split_bf16(v1, h1, l1);
      hi[e] = pack_bf16x2(h0, h1);
      lo[e] = pack_bf16x2(l0, l1);
    }
  };
  auto store_h = [&](int t, const f32x4& v) {
    uint16_t* dst = Ly.h + (int64_t)t * m + fc;
    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  };
  if (nkc <= kC && QB == 1) {
    // the common shape in one round of loads: every load is issued (zeros
    // past nkc, M or m) before the first sum
    const int q0 = 8 * g;
    const u32x4 b0 = load_b(0);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = 16 * tb + lr;
      const bool tv = t < M;
      u32x4 w[kC], w0[kC], w1[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        w[c] = bload128(rhp, (c < nkc && tv && fc < m) ? (uint32_t)((((int64_t)c * M + t) * m + fc) * 4) : hbytes);
        const bool uv = c < nkc && tv && q0 < r;
        const uint32_t off = uv ? (uint32_t)((((int64_t)c * M + t) * r + q0) * 4) : ubytes;
        w0[c] = bload128(rup, off);
        w1[c] = bload128(rup, uv ? off + 16 : ubytes);
      }
      f32x4 hs = {0.f, 0.f, 0.f, 0.f}, u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kC; ++c)
        if (c < nkc) {
          hs += __builtin_bit_cast(f32x4, w[c]);
          u0 += __builtin_bit_cast(f32x4, w0[c]);
          u1 += __builtin_bit_cast(f32x4, w1[c]);
        }
      u0 *= Ly.u_scale;
      u1 *= Ly.u_scale;
      if (Ly.u_out && tile == 0 && wave == 0 && tv && q0 < r) {
        *reinterpret_cast<f32x4*>(Ly.u_out + (int64_t)t * r + q0) = u0;
        *reinterpret_cast<f32x4*>(Ly.u_out + (int64_t)t * r + q0 + 4) = u1;
      }
      u32x4 hi, lo;
      su_split(u0, u1, hi, lo);
      f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
      acc2 = mfma16x16x32(b0, hi, acc2);
      acc2 = mfma16x16x32(b0, lo, acc2);
      if (tv && fc < m) store_h(t, hs + acc2);
    }
    return;
  }
  u32x4 bw[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) bw[qb] = load_b(qb);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = 16 * tb + lr;
    const bool tv = t < M;
    // chunk partials of h, kC at a time
    f32x4 hs = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nkc; c0 += kC) {
      u32x4 w[kC];
#pragma unroll
      for (int c = 0; c < kC; ++c)
        w[c] = bload128(rhp, (c0 + c < nkc && tv && fc < m) ? (uint32_t)((((int64_t)(c0 + c) * M + t) * m + fc) * 4) : hbytes);
#pragma unroll
      for (int c = 0; c < kC; ++c)
        if (c0 + c < nkc) hs += __builtin_bit_cast(f32x4, w[c]);
    }
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
    for (int qb = 0; qb < QB; ++qb) {
      const int q0 = 32 * qb + 8 * g;
      const bool qv = tv && q0 < r;
      // u[t][q0 .. q0 + 7], summed over the chunks in order from 0
      f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = 0; c0 < nkc; c0 += kC) {
        u32x4 w0[kC], w1[kC];
#pragma unroll
        for (int c = 0; c < kC; ++c) {
          const uint32_t off = (c0 + c < nkc && qv) ? (uint32_t)((((int64_t)(c0 + c) * M + t) * r + q0) * 4) : ubytes;
          w0[c] = bload128(rup, off);
          w1[c] = bload128(rup, off == ubytes ? ubytes : off + 16);
        }
#pragma unroll
        for (int c = 0; c < kC; ++c)
          if (c0 + c < nkc) {
            u0 += __builtin_bit_cast(f32x4, w0[c]);
            u1 += __builtin_bit_cast(f32x4, w1[c]);
          }
      }
      u0 *= Ly.u_scale;
      u1 *= Ly.u_scale;
      if (Ly.u_out && tile == 0 && wave == 0 && qv) {
        *reinterpret_cast<f32x4*>(Ly.u_out + (int64_t)t * r + q0) = u0;
        *reinterpret_cast<f32x4*>(Ly.u_out + (int64_t)t * r + q0 + 4) = u1;
      }
      u32x4 hi, lo;
      su_split(u0, u1, hi, lo);
      u32x4 aa = bw[0];
#pragma unroll
      for (int j = 1; j < kQB; ++j)
        if (qb == j) aa = bw[j];
      acc2 = mfma16x16x32(aa, hi, acc2);
      acc2 = mfma16x16x32(aa, lo, acc2);
    }
    if (tv && fc < m) store_h(t, hs + acc2);
  }
}

template <int TB>
__global__ __launch_bounds__(256) void small_reduce_kernel(SmallArgs a) {
  __shared__ float su[32 * kMaxRank];
  const int li = find_layer(a, blockIdx.x, 1);
  const SmallLayer& Ly = a.L[li];
  const int tile = (int)(blockIdx.x - Ly.out_begin);
  const int M = a.M;
  const int64_t m = Ly.m;
  const int r = Ly.r;
  if ((r & 7) == 0 && (m & 3) == 0) {
    small_reduce_aligned<TB>(Ly, tile, M);
    return;
  }
  const int nkc = Ly.nkc;
  const int nparts = nkc;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;
  // u partials are loaded 8 at a time before they are summed (in order), so
  // the loads of one thread overlap instead of forming a chain
  for (int idx = tid; idx < M * r; idx += 256) {
    float uq = 0.0f;
    for (int c0 = 0; c0 < nparts; c0 += 8) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = (c0 + c < nparts) ? Ly.upart[(int64_t)(c0 + c) * M * r + idx] : 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c0 + c < nparts) uq += v[c];
    }
    uq *= Ly.u_scale;
    su[idx] = uq;
    if (Ly.u_out && tile == 0) Ly.u_out[idx] = uq;
  }
  __syncthreads();
  const int64_t fa = (int64_t)tile * 64 + 16 * wave + lr;   // B row of this lane's A fragment
  const int64_t fc = (int64_t)tile * 64 + 16 * wave + 4 * g;  // this lane's 4 output features
  const int QB = (r + 31) / 32;
  const uint32_t bbytes = (uint32_t)(m * r * 2);
  const brsrc_t rbm = make_rsrc(Ly.B, bbytes);
  const uint32_t hbytes = (uint32_t)((int64_t)nkc * M * m * 4);
  const brsrc_t rhp = make_rsrc(Ly.hpart, hbytes);
  const bool v4 = (m & 3) == 0 && fc + 4 <= m;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int t = 16 * tb + lr;
    // chunk partials first (8 in flight), then the adapter term
    f32x4 hs = {0.f, 0.f, 0.f, 0.f};
    if (v4) {
      for (int c0 = 0; c0 < nkc; c0 += 8) {
        u32x4 w[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          w[c] = bload128(rhp, (c0 + c < nkc && t < M) ? (uint32_t)((((int64_t)(c0 + c) * M + t) * m + fc) * 4) : hbytes);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c0 + c < nkc) hs += __builtin_bit_cast(f32x4, w[c]);
      }
    } else if (t < M) {
      for (int c = 0; c < nkc; ++c)
        for (int e = 0; e < 4; ++e)
          if (fc + e < m) hs[e] += Ly.hpart[((int64_t)c * M + t) * m + fc + e];
    }
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
    for (int qb = 0; qb < QB; ++qb) {
      // A: B[fa][32 qb + 8 g .. + 7] (zeros past m or r)
      uint32_t av[4] = {0u, 0u, 0u, 0u};
      const int q0 = 32 * qb + 8 * g;
      if (fa < m) {
        if ((r & 7) == 0 && q0 + 8 <= r) {
          const u32x4 w = bload128(rbm, (uint32_t)((fa * r + q0) * 2));
          av[0] = w[0]; av[1] = w[1]; av[2] = w[2]; av[3] = w[3];
        } else {
          for (int e = 0; e < 8; ++e)
            if (q0 + e < r) av[e >> 1] |= (uint32_t)Ly.B[fa * r + q0 + e] << (16 * (e & 1));
        }
      }
      // B operand: s u[t][32 qb + 8 g .. + 7] as bf16 hi + lo (zeros past M or r)
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float uv[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int q = q0 + 2 * e + h2;
          uv[h2] = (t < M && q < r) ? Ly.s * su[t * r + q] : 0.0f;
        }
        float h0, l0, h1, l1;
        split_bf16(uv[0], h0, l0);
        split_bf16(uv[1], h1, l1);
        hi[e] = pack_bf16x2(h0, h1);
        lo[e] = pack_bf16x2(l0, l1);
      }
      const u32x4 aa = u32x4{av[0], av[1], av[2], av[3]};
      acc2 = mfma16x16x32(aa, u32x4{hi[0], hi[1], hi[2], hi[3]}, acc2);
      acc2 = mfma16x16x32(aa, u32x4{lo[0], lo[1], lo[2], lo[3]}, acc2);
    }
    if (t >= M || fc >= m) continue;
    const f32x4 v = hs + acc2;
    uint16_t* dst = Ly.h + (int64_t)t * m + fc;
    if (v4) {
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    } else {
      for (int e = 0; e < 4; ++e)
        if (fc + e < m) dst[e] = (uint16_t)(pack_bf16x2(v[e], 0.0f) & 0xFFFFu);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int small_max_tokens() { return 32; }
int small_max_layers() { return sm::kMaxLayers; }

static inline int64_t cdiv_s(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t small_nkc(int64_t n) { return cdiv_s(n, sm::KC); }

// fp32 partial workspace of one layer: h [nkc][M][m] and u [nkc][M][r]
size_t small_ws_bytes(int64_t M, int64_t n, int64_t m, int r) {
  const int64_t nkc = small_nkc(n);
  const size_t hb = (size_t)nkc * M * m * sizeof(float);
  const size_t ub = (size_t)nkc * M * r * sizeof(float);
  return ((hb + 255) & ~(size_t)255) + ((ub + 255) & ~(size_t)255);
}

struct SmallLayerHost {
  const uint16_t* x; const uint8_t* codes; const uint8_t* absmax8; const float* c2;
  const uint16_t* A; const uint16_t* B; uint16_t* h; float* u_out;
  int64_t n, m; int r; float s;
  void* ws;  // small_ws_bytes(M, n, m, r) bytes, 256-aligned
  DropoutDev drop{};     // off unless set
  float u_scale = 1.0f;  // applied to u after the chunk sum
};

void launch_small_fwd(int M, const SmallLayerHost* layers, int count, const Nf4Table& tab, hipStream_t stream) {
  SmallArgs a{};
  a.count = count;
  a.M = M;
  const int fbmax = M <= 16 ? SmallTile<1>::FBMAX : SmallTile<2>::FBMAX;
  // feature blocks per workgroup: the fewest that keep the launch (with its
  // u workgroups) within two workgroups per CU (a launch a few workgroups over
  // that would run a second, almost empty round), the same width for every layer
  auto wgs_for = [&](int fbw) {
    int64_t w = 0;
    for (int i = 0; i < count; ++i) w += small_nkc(layers[i].n) * (cdiv_s(cdiv_s(layers[i].m, 16), fbw) + 1);
    return w;
  };
  const int64_t target = (int64_t)sm::kWGsPerCU * device_cus();
  int fbw = 1;
  while (fbw < fbmax && wgs_for(fbw) > target) ++fbw;
  int wg = 0;
  int64_t outs = 0;
  for (int i = 0; i < count; ++i) {
    const SmallLayerHost& h = layers[i];
    SmallLayer& L = a.L[i];
    L.x = h.x; L.codes = h.codes; L.absmax8 = h.absmax8; L.c2 = h.c2; L.A = h.A; L.B = h.B; L.h = h.h;
    L.u_out = h.u_out; L.n = h.n; L.m = h.m; L.r = h.r; L.s = h.s;
    L.drop = h.drop; L.u_scale = h.u_scale;
    L.nkc = (int)small_nkc(h.n);
    L.fbw = fbw;
    L.ngroups = (int)cdiv_s(cdiv_s(h.m, 16), fbw);
    const size_t hb = (size_t)L.nkc * M * h.m * sizeof(float);
    L.hpart = reinterpret_cast<float*>(h.ws);
    L.upart = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(h.ws) + ((hb + 255) & ~(size_t)255));
    L.wg_begin = wg;
    L.out_begin = outs;
    wg += L.nkc * L.ngroups;
    outs += cdiv_s(h.m, 64);
  }
  a.main_wgs = wg;
  for (int i = 0; i < count; ++i) {
    a.L[i].u_begin = wg;
    wg += a.L[i].nkc;
  }
  if (M <= 16)
    hipLaunchKernelGGL(small_fwd_kernel<1>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  else
    hipLaunchKernelGGL(small_fwd_kernel<2>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  if (M <= 16)
    hipLaunchKernelGGL(small_reduce_kernel<1>, dim3((unsigned)outs), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(small_reduce_kernel<2>, dim3((unsigned)outs), dim3(256), 0, stream, a);
}

}  // namespace qlora
