// The rank-r adapter products of the adapted linear layer.
//   u = x A^T, v = g B                   (down-projections, split over K)
//   grad_A = s v^T x, grad_B = s g^T u   (reductions over tokens)
// "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3, the low-rank term B A x)
// and Step 4 (Eq. 5, the adapter gradients), with the alpha/r scale of the
// LoraConfig snippet.  All products run on bf16 MFMA with fp32 accumulation;
// fp32 operands (u, v) enter as a bf16 hi + lo pair.  Every reduction over a
// split dimension goes through fp32 partials summed in a fixed order, so
// results are deterministic.
//
// Both kernels stream one large bf16 matrix (x or g) from HBM exactly once
// and are bound by that read.  Each workgroup stages 16 KB tiles through LDS
// with line-coalesced 16-byte loads (a wave covers 4 rows x 256 B), keeps
// the next tile's loads in flight in registers while the MFMAs consume the
// current one, and reads MFMA fragments out of XOR-swizzled LDS rows.
#include "qlora_common.h"

namespace qlora {

__host__ __device__ static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Offset of 16-byte piece c (0..15) of row `row` in a tile of 256-byte rows;
// any 16 consecutive rows read at one piece index hit 16 distinct bank groups.
__device__ __forceinline__ uint32_t sw256(int row, int c) {
  return (uint32_t)(row * 256 + ((c ^ (row & 15)) << 4));
}

// ---------------------------------------------------------------------------
// part[split][t][q] = sum_{k in split} X[t][k] * Y[q][k]
// X: M x K bf16 (K a multiple of 8), Y: R x K bf16, R <= 16 * RB.
// Workgroup: 64 tokens (16 per wave) x all R columns; its K range
// [split * kc, split * kc + kc) is walked in stages of 128.
// ---------------------------------------------------------------------------
namespace dp {
constexpr int TT = 64;        // tokens per workgroup
constexpr int KCH = 128;      // k per stage
constexpr int XB = TT * 256;  // X tile bytes per stage
}  // namespace dp

template <int RB>
__global__ __launch_bounds__(256) void down_proj_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        const uint16_t* __restrict__ Y, int R,
                                                        float* __restrict__ part, int64_t kc, DropoutDev drop) {
  constexpr int YB = RB * 16 * 256;
  constexpr int STAGE = dp::XB + YB;
  __shared__ __align__(16) uint8_t lds[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lk = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * dp::TT;
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * kc;
  const int64_t kend = (kbeg + kc < K) ? kbeg + kc : K;
  const int nst = (int)cdiv(kend - kbeg, dp::KCH);

  const uint32_t xbytes = (uint32_t)(M * K * 2);
  const uint32_t ybytes = (uint32_t)((int64_t)R * K * 2);
  const brsrc_t rx = make_rsrc(X, xbytes);
  const brsrc_t ry = make_rsrc(Y, ybytes);
  // Load i of a stage covers row 16 i + prow, 16-byte piece pc (k offset 8 pc).
  const int prow = tid >> 4;
  const int pc = tid & 15;
  const int64_t kl = kbeg + 8 * pc;
  uint32_t xo[4], yo[RB];
  bool rowok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rowok[i] = t0 + 16 * i + prow < M;
    xo[i] = (uint32_t)(((t0 + 16 * i + prow) * K + kl) * 2);
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) yo[i] = (uint32_t)(((int64_t)(16 * i + prow) * K + kl) * 2);

  auto load = [&](int st, u32x4(&xr)[4], u32x4(&yr)[RB]) {
    const bool ok = kl + (int64_t)st * dp::KCH < kend;  // pieces past the split read as 0
    const uint32_t d = (uint32_t)st * (dp::KCH * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = bload128(rx, (ok && rowok[i]) ? xo[i] + d : xbytes);
#pragma unroll
    for (int i = 0; i < RB; ++i) yr[i] = bload128(ry, ok ? yo[i] + d : ybytes);
  };
  // dropout (adapter input only): X element (t, k) is e = t K + k
  auto store = [&](int buf, int st, const u32x4(&xr)[4], const u32x4(&yr)[RB]) {
    uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 w = xr[i];
      if (drop.on) w = dropout8(drop, (uint64_t)((t0 + 16 * i + prow) * K + kl + (int64_t)st * dp::KCH), w);
      *reinterpret_cast<u32x4*>(base + sw256(16 * i + prow, pc)) = w;
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) *reinterpret_cast<u32x4*>(base + dp::XB + sw256(16 * i + prow, pc)) = yr[i];
  };

  f32x4 acc[RB];
#pragma unroll
  for (int c = 0; c < RB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
    const uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(base + sw256(16 * wave + lr, 4 * s + lk));
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(base + dp::XB + sw256(16 * cb + lr, 4 * s + lk));
        acc[cb] = mfma16x16x32(a, b, acc[cb]);
      }
    }
  };

  u32x4 xa[4], ya[RB], xb[4], yb[RB];
  load(0, xa, ya);
  if (nst > 1) load(1, xb, yb);
  for (int st = 0; st < nst; st += 2) {
    store(0, st, xa, ya);
    if (st + 2 < nst) load(st + 2, xa, ya);
    __syncthreads();
    compute(0);
    if (st + 1 >= nst) break;
    store(1, st + 1, xb, yb);
    if (st + 3 < nst) load(st + 3, xb, yb);
    __syncthreads();
    compute(1);
  }

  // lane holds tokens 16*wave + 4*lk + e, column q = 16*cb + lr
  float* dst = part + (int64_t)split * M * R;
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    const int q = 16 * cb + lr;
    if (q >= R) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t t = t0 + 16 * wave + 4 * lk + e;
      if (t < M) dst[t * R + q] = acc[cb][e];
    }
  }
}

// sum_k part[k * stride + i] for k = 0 .. n - 1, added in k order from 0;
// the loads go out 8 at a time so that they overlap
__device__ __forceinline__ float sum_splits(const float* __restrict__ part, int n, int64_t stride, int64_t i) {
  float s = 0.0f;
  for (int k0 = 0; k0 < n; k0 += 8) {
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = k0 + c < n ? part[(int64_t)(k0 + c) * stride + i] : 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (k0 + c < n) s += v[c];
  }
  return s;
}

// out[i] = scale * sum_s part[s][i], summed in split order (fp32)
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int nsplit, int64_t count,
                                                            float scale, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const float v = sum_splits(part, nsplit, count, i);
  out[i] = scale == 1.0f ? v : scale * v;
}

// ---------------------------------------------------------------------------
// part[split][j][q] = sum_{t in split} X[t][j] * Y[t][q]
// X: M x J bf16 (J a multiple of 8), Y: M x R fp32, R <= 16 * RB.
// Workgroup: 128 columns j (32 per wave) x all R; its token range is walked
// in stages of 64.  The X tile keeps its natural [t][j] layout (32-byte units
// of each row XOR-swizzled) and is read transposed with ds_read_b64_tr_b16;
// the Y tile is split into bf16 hi and lo planes stored transposed [q][t].
// ---------------------------------------------------------------------------
namespace tg {
constexpr int TT = 64;        // tokens per stage
constexpr int JT = 128;       // columns per workgroup
constexpr int XB = TT * 256;  // X tile bytes per stage
}  // namespace tg

// X tile: row t, 16-byte piece c (columns 8c..8c+7).  Rows t, t+1, t+2, t+3,
// t+8, .. t+11 put a given 32-byte unit in 8 different bank groups.
__device__ __forceinline__ uint32_t swtg(int t, int c) {
  const int f = (t & 3) | (((t >> 3) & 1) << 2);
  return (uint32_t)(t * 256 + ((((c >> 1) ^ f)) << 5) + ((c & 1) << 4));
}
// Y planes: row q holds 64 tokens (128 B) in 16-byte chunks of 8 tokens.
__device__ __forceinline__ uint32_t swy(int q, int chunk) {
  return (uint32_t)(q * 128 + ((chunk ^ ((q >> 1) & 7)) << 4));
}

template <int RB>
__global__ __launch_bounds__(256) void token_grad_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t J,
                                                         const float* __restrict__ Y, int R,
                                                         float* __restrict__ part, int64_t tc, DropoutDev drop) {
  constexpr int PLANE = RB * 16 * 128;
  constexpr int STAGE = tg::XB + 2 * PLANE;
  __shared__ __align__(16) uint8_t lds[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lk = lane >> 4;
  const int64_t j0 = (int64_t)blockIdx.x * tg::JT;
  const int split = blockIdx.y;
  const int64_t tbeg = (int64_t)split * tc;
  const int64_t tend = (tbeg + tc < M) ? tbeg + tc : M;
  const int nst = (int)cdiv(tend - tbeg, tg::TT);

  const uint32_t xbytes = (uint32_t)(M * J * 2);
  const uint32_t ybytes = (uint32_t)(M * R * 4);
  const brsrc_t rx = make_rsrc(X, xbytes);
  const brsrc_t ry = make_rsrc(Y, ybytes);
  const int prow = tid >> 4;
  const int pc = tid & 15;
  const bool jok = j0 + 8 * pc < J;
  uint32_t xo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xo[i] = (uint32_t)(((tbeg + 16 * i + prow) * J + j0 + 8 * pc) * 2);
  const int ypieces = 16 * R;  // 16-byte pieces of fp32 in one 64-token Y tile

  // Planes rows q in [R, 16 RB) are never written by the stages: clear them.
  for (int id = tid; id < 2 * 2 * (16 * RB - R) * 8; id += 256) {
    const int chunk = id & 7;
    const int rest = id >> 3;
    const int q = R + rest % (16 * RB - R);
    const int pl = rest / (16 * RB - R);  // stage * 2 + plane
    *reinterpret_cast<u32x4*>(lds + (pl >> 1) * STAGE + tg::XB + (pl & 1) * PLANE + swy(q, chunk)) =
        u32x4{0u, 0u, 0u, 0u};
  }

  auto load = [&](int st, u32x4(&xr)[4], u32x4(&yr)[RB]) {
    const int64_t tb = tbeg + (int64_t)st * tg::TT;
    const uint32_t d = (uint32_t)(st * tg::TT * J * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = jok && (tb + 16 * i + prow < tend);
      xr[i] = bload128(rx, ok ? xo[i] + d : xbytes);
    }
    const uint32_t ybase = (uint32_t)(tb * R * 4);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int p = 256 * i + tid;
      yr[i] = bload128(ry, p < ypieces ? ybase + 16 * p : ybytes);
    }
  };
  auto store = [&](int buf, int st, const u32x4(&xr)[4], const u32x4(&yr)[RB]) {
    uint8_t* base = lds + buf * STAGE;
    const int64_t tb = tbeg + (int64_t)st * tg::TT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // dropout (adapter input only): X element (t, j) is e = t J + j
      u32x4 w = xr[i];
      if (drop.on) w = dropout8(drop, (uint64_t)((tb + 16 * i + prow) * J + j0 + 8 * pc), w);
      *reinterpret_cast<u32x4*>(base + swtg(16 * i + prow, pc)) = w;
    }
    const int tlim = (int)((tend - tb) < tg::TT ? (tend - tb) : tg::TT);
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int p = 256 * i + tid;
      if (p < ypieces) {
        int f = 4 * p;
        int t = f / R;
        int q = f - t * R;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = t < tlim ? __uint_as_float(yr[i][e]) : 0.0f;
          float h, l;
          split_bf16(y, h, l);
          const uint32_t off = swy(q, t >> 3) + (t & 7) * 2;
          *reinterpret_cast<uint16_t*>(base + tg::XB + off) = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
          *reinterpret_cast<uint16_t*>(base + tg::XB + PLANE + off) = (uint16_t)(pack_bf16x2(l, 0.f) & 0xFFFFu);
          if (++q == R) { q = 0; ++t; }
        }
      }
    }
  };

  f32x4 acc[2][RB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tr_row = lr >> 2;
  const int tr_c = lr & 3;
  auto compute = [&](int buf) {
    const uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        // lanes 4r+c of each 16-lane group address row r, columns 4c..4c+3
        const int t = 32 * kk + 8 * lk + tr_row;
        const int c = 2 * (2 * wave + ib) + (tr_c >> 1);
        const uint8_t* p0 = base + swtg(t, c) + (tr_c & 1) * 8;
        const uint8_t* p1 = base + swtg(t + 4, c) + (tr_c & 1) * 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a[ib] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const uint32_t off = swy(16 * cb + lr, 4 * kk + lk);
        const u32x4 bh = *reinterpret_cast<const u32x4*>(base + tg::XB + off);
        const u32x4 bl = *reinterpret_cast<const u32x4*>(base + tg::XB + PLANE + off);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          acc[ib][cb] = mfma16x16x32(a[ib], bh, acc[ib][cb]);
          acc[ib][cb] = mfma16x16x32(a[ib], bl, acc[ib][cb]);
        }
      }
    }
  };

  u32x4 xa[4], ya[RB], xb[4], yb[RB];
  load(0, xa, ya);
  if (nst > 1) load(1, xb, yb);
  for (int st = 0; st < nst; st += 2) {
    store(0, st, xa, ya);
    if (st + 2 < nst) load(st + 2, xa, ya);
    __syncthreads();
    compute(0);
    if (st + 1 >= nst) break;
    store(1, st + 1, xb, yb);
    if (st + 3 < nst) load(st + 3, xb, yb);
    __syncthreads();
    compute(1);
  }

  // lane holds columns j = 32*wave + 16*ib + 4*lk + e, q = 16*cb + lr
  float* dst = part + (int64_t)split * J * R;
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    const int q = 16 * cb + lr;
    if (q >= R) continue;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + 32 * wave + 16 * ib + 4 * lk + e;
        if (j < J) dst[j * R + q] = acc[ib][cb][e];
      }
  }
}

// ---------------------------------------------------------------------------
// One read of g for both products that need it:
//   vpart[fs][t][q]  = sum_{f in feature tile fs} g[t][f] * B[f][q]
//   gbpart[ts][f][q] = sum_{t in token tile ts}  g[t][f] * u[t][q]
// (v = sum_fs vpart, grad_B = s sum_ts gbpart).  A workgroup owns 256
// tokens x 512 features of g and walks them as 16 sub-tiles of 64 x 128
// (feature sub-tile outer).  Per sub-tile every wave adds 16 tokens' worth
// of v (A = g rows, B operand = B read transposed from its natural [f][q]
// tile) and 32 features' worth of grad_B (A = g columns read transposed, B
// operand = u as bf16 hi + lo planes [q][t]) into accumulators that live
// through the whole walk.  R a multiple of 8 and at most 16 RB.
// ---------------------------------------------------------------------------
namespace gp {
constexpr int TT = 64;        // tokens per sub-tile
constexpr int FT = 128;       // features per sub-tile
constexpr int ST = 4;         // sub-tiles along tokens per workgroup
constexpr int GB = TT * 256;  // g sub-tile bytes
}  // namespace gp

template <int RB, int SF>
__global__ __launch_bounds__(256) void gpass_kernel(const uint16_t* __restrict__ G, int64_t M, int64_t J,
                                                    const uint16_t* __restrict__ Bm, int64_t m,
                                                    const float* __restrict__ U, int R, float* __restrict__ vpart,
                                                    float* __restrict__ gbpart) {
  constexpr int BP = 32 * RB;                // B tile row pitch: 16 RB ranks
  constexpr int BTB = gp::FT * BP;           // B tile bytes
  constexpr int PLANE = RB * 16 * 128;       // u plane: 16 RB rows of 64 tokens
  constexpr int STAGE = gp::GB + BTB + 2 * PLANE;
  __shared__ __align__(16) uint8_t lds[2 * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lk = lane >> 4;
  // 1D grid (either tile count can exceed the 65535 limit of a grid's y):
  // workgroup fs + nfs ts
  const int nfs = (int)((J + gp::FT * SF - 1) / (gp::FT * SF));
  const int fs = (int)blockIdx.x % nfs;      // feature tile (v partial index)
  const int ts = (int)blockIdx.x / nfs;      // token tile (grad_B partial index)
  const int64_t f0 = (int64_t)fs * gp::FT * SF;
  const int64_t t0 = (int64_t)ts * gp::TT * gp::ST;

  // Rank slots q >= R of the B tiles and u planes are never loaded: clear them.
  if (R < 16 * RB) {
    for (int id = tid; id < 2 * gp::FT * (16 * RB - R) / 8; id += 256) {
      const int st = id / (gp::FT * (16 * RB - R) / 8);
      const int rest = id % (gp::FT * (16 * RB - R) / 8);
      const int f = rest / ((16 * RB - R) / 8);
      const int c = rest % ((16 * RB - R) / 8);
      *reinterpret_cast<u32x4*>(lds + st * STAGE + gp::GB + f * BP + 2 * R + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
    for (int id = tid; id < 2 * 2 * (16 * RB - R) * 8; id += 256) {
      const int chunk = id & 7;
      const int rest = id >> 3;
      const int q = R + rest % (16 * RB - R);
      const int pl = rest / (16 * RB - R);  // stage * 2 + plane
      *reinterpret_cast<u32x4*>(lds + (pl >> 1) * STAGE + gp::GB + BTB + (pl & 1) * PLANE + swy(q, chunk)) =
          u32x4{0u, 0u, 0u, 0u};
    }
  }

  const uint32_t gbytes = (uint32_t)(M * J * 2);
  const uint32_t bbytes = (uint32_t)(m * R * 2);
  const uint32_t ubytes = (uint32_t)(M * R * 4);
  const brsrc_t rg = make_rsrc(G, gbytes);
  const brsrc_t rb = make_rsrc(Bm, bbytes);
  const brsrc_t ru = make_rsrc(U, ubytes);
  const int prow = tid >> 4;
  const int pc = tid & 15;
  // 16-byte pieces of one B sub-tile (128 rows of R bf16), which is also the
  // count of one u sub-tile (64 rows of R fp32)
  const int npieces = gp::FT * R / 8;
  constexpr int PPT = RB;                    // pieces per thread, upper bound (R <= 16 RB)

  // sub-tile i: feature sub-tile i / ST, token sub-tile i % ST
  auto load = [&](int i, u32x4(&gr)[4], u32x4(&br)[PPT], u32x4(&ur)[PPT]) {
    const int64_t fb = f0 + (int64_t)(i / gp::ST) * gp::FT;
    const int64_t tb = t0 + (int64_t)(i % gp::ST) * gp::TT;
    const bool fok = fb + 8 * pc < J;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = tb + 16 * k + prow;
      gr[k] = bload128(rg, (fok && t < M) ? (uint32_t)((t * J + fb + 8 * pc) * 2) : gbytes);
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = 256 * k + tid;
      // B rows fb .. fb + 127 and u rows tb .. tb + 63 are contiguous ranges
      br[k] = bload128(rb, (p < npieces && fb * R * 2 + 16 * p < (int64_t)bbytes) ? (uint32_t)(fb * R * 2 + 16 * p)
                                                                                 : bbytes);
      ur[k] = bload128(ru, (p < npieces && tb * R * 4 + 16 * p < (int64_t)ubytes)
                               ? (uint32_t)(tb * R * 4 + 16 * p) : ubytes);
    }
  };
  auto store = [&](int buf, const u32x4(&gr)[4], const u32x4(&br)[PPT], const u32x4(&ur)[PPT]) {
    uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(base + swtg(16 * k + prow, pc)) = gr[k];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int p = 256 * k + tid;
      if (p < npieces) {
        const int f = (16 * p) / (2 * R);
        const int cb = (16 * p) % (2 * R);
        *reinterpret_cast<u32x4*>(base + gp::GB + f * BP + cb) = br[k];
      }
      if (p < npieces) {
        // 4 fp32 of u: token t, ranks q .. q + 3 (R % 4 == 0)
        const int t = (4 * p) / R;
        const int q = (4 * p) % R;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float h, l;
          split_bf16(__uint_as_float(ur[k][e]), h, l);
          const uint32_t off = swy(q + e, t >> 3) + (t & 7) * 2;
          *reinterpret_cast<uint16_t*>(base + gp::GB + BTB + off) = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
          *reinterpret_cast<uint16_t*>(base + gp::GB + BTB + PLANE + off) = (uint16_t)(pack_bf16x2(l, 0.f) & 0xFFFFu);
        }
      }
    }
  };

  f32x4 av[gp::ST][RB];        // v: tokens 64 ts' + 16 wave + 4 lk + e, rank 16 cb + lr
  f32x4 ab[SF][2][RB];     // grad_B: features 128 fs' + 32 wave + 16 ib + 4 lk + e, rank 16 cb + lr
#pragma unroll
  for (int i = 0; i < gp::ST; ++i)
#pragma unroll
    for (int c = 0; c < RB; ++c) av[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SF; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < RB; ++c) ab[i][j][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int tr_row = lr >> 2;
  const int tr_c = lr & 3;
  auto compute = [&](int buf, int i) {
    const uint8_t* base = lds + buf * STAGE;
    const int fsub = i / gp::ST, tsub = i % gp::ST;
    // v += g[16 wave + lr][f] B[f][q] over the 128 features
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(base + swtg(16 * wave + lr, 4 * s4 + lk));
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        // B operand: rows f = 32 s4 + 8 lk + 4 h + lr / 4, ranks 16 cb + 4 (lr % 4) .. + 3
        const uint8_t* p0 = base + gp::GB + (32 * s4 + 8 * lk + tr_row) * BP + 2 * (16 * cb + 4 * tr_c);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * BP));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        av[tsub][cb] = mfma16x16x32(a, u32x4{l2[0], l2[1], h2[0], h2[1]}, av[tsub][cb]);
      }
    }
    // grad_B += g[t][32 wave + 16 ib + lr] u[t][q] over the 64 tokens
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int t = 32 * kk + 8 * lk + tr_row;
        const int c = 2 * (2 * wave + ib) + (tr_c >> 1);
        const uint8_t* p0 = base + swtg(t, c) + (tr_c & 1) * 8;
        const uint8_t* p1 = base + swtg(t + 4, c) + (tr_c & 1) * 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a[ib] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const uint32_t off = swy(16 * cb + lr, 4 * kk + lk);
        const u32x4 bh = *reinterpret_cast<const u32x4*>(base + gp::GB + BTB + off);
        const u32x4 bl = *reinterpret_cast<const u32x4*>(base + gp::GB + BTB + PLANE + off);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          ab[fsub][ib][cb] = mfma16x16x32(a[ib], bh, ab[fsub][ib][cb]);
          ab[fsub][ib][cb] = mfma16x16x32(a[ib], bl, ab[fsub][ib][cb]);
        }
      }
    }
  };

  // D sub-tiles of loads in flight (register sets used round-robin), two LDS
  // buffers: sub-tile i is stored into buffer i % 2 once every wave has left
  // the compute of sub-tile i - 2 (the barrier of sub-tile i - 1)
  constexpr int NS = gp::ST * SF;
  constexpr int D = RB == 1 ? 4 : 2;
  u32x4 gr[D][4], br[D][PPT], ur[D][PPT];
#pragma unroll
  for (int i = 0; i < D; ++i) load(i, gr[i], br[i], ur[i]);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    store(i & 1, gr[i % D], br[i % D], ur[i % D]);
    if (i + D < NS) load(i + D, gr[i % D], br[i % D], ur[i % D]);
    __syncthreads();
    compute(i & 1, i);
  }

  float* vdst = vpart + (int64_t)fs * M * R;
#pragma unroll
  for (int i = 0; i < gp::ST; ++i)
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      const int q = 16 * cb + lr;
      if (q >= R) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = t0 + gp::TT * i + 16 * wave + 4 * lk + e;
        if (t < M) vdst[t * R + q] = av[i][cb][e];
      }
    }
  float* bdst = gbpart + (int64_t)ts * J * R;
#pragma unroll
  for (int i = 0; i < SF; ++i)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const int q = 16 * cb + lr;
        if (q >= R) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t f = f0 + gp::FT * i + 32 * wave + 16 * ib + 4 * lk + e;
          if (f < J) bdst[f * R + q] = ab[i][ib][cb][e];
        }
      }
}

// out = bf16(s * sum_s part[s]) over the first Jout rows of part ([J][R] per
// split); out is [Jout][R] or, when transpose_out, [R][Jout].
__global__ __launch_bounds__(256) void reduce_grad_kernel(const float* __restrict__ part, int nsplit, int64_t J,
                                                          int64_t Jout, int R, float s, int transpose_out,
                                                          uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Jout * R) return;
  const float acc = sum_splits(part, nsplit, J * R, i);
  const uint16_t b = (uint16_t)(pack_bf16x2(s * acc, 0.f) & 0xFFFFu);
  if (!transpose_out) {
    out[i] = b;
  } else {
    const int64_t j = i / R, q = i % R;
    out[q * Jout + j] = b;
  }
}

// out[r][0:cols] = in[r][0:cols], out[r][cols:cols_pad] = 0 (bf16 rows)
__global__ __launch_bounds__(256) void pad_cols_bf16_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                            int64_t cols, int64_t cols_pad,
                                                            uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols_pad) return;
  const int64_t r = i / cols_pad, c = i % cols_pad;
  out[i] = c < cols ? in[r * cols + c] : (uint16_t)0;
}

// out[c][r] = in[r][c] for a rows x cols bf16 matrix; out rows have length
// ld >= rows and out[c][rows:ld] = 0.  One thread per output element.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                             int64_t cols, int64_t ld, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= cols * ld) return;
  const int64_t c = i / ld, r = i % ld;
  out[i] = r < rows ? in[r * cols + c] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------
static inline int rank_blocks(int R) { return R <= 16 ? 1 : R <= 32 ? 2 : R <= 64 ? 4 : 8; }
// Workgroups wanted per launch: enough to cover every CU a few times over
// (fewer for the large-rank variants, which hold one workgroup per CU).
static inline int64_t target_wgs(int R) { return rank_blocks(R) <= 2 ? 512 : 256; }

int down_proj_splits(int64_t M, int64_t K, int R) {
  const int64_t tiles = cdiv(M, dp::TT);
  const int64_t stages = cdiv(K, dp::KCH);
  int64_t want = cdiv(target_wgs(R), tiles);
  if (want < 1) want = 1;
  if (want > stages) want = stages;
  if (want > 64) want = 64;
  return (int)cdiv(K, cdiv(cdiv(K, want), dp::KCH) * dp::KCH);
}

// drop: dropout on X (the adapter input), or null; the result is scaled by
// `scale` (1 / (1 - p) with dropout) after the fixed-order sum
void launch_down_proj(const uint16_t* X, int64_t M, int64_t K, const uint16_t* Y, int R, float* part, int splits,
                      float* out, hipStream_t stream, const DropoutDev* drop, float scale) {
  const int64_t kc = cdiv(cdiv(K, splits), dp::KCH) * dp::KCH;
  const dim3 grid((unsigned)cdiv(M, dp::TT), (unsigned)splits);
  const DropoutDev d = drop ? *drop : DropoutDev{0u, 0u, 0u, 0ull, 0};
  switch (rank_blocks(R)) {
    case 1: hipLaunchKernelGGL(down_proj_kernel<1>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
    case 2: hipLaunchKernelGGL(down_proj_kernel<2>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
    case 4: hipLaunchKernelGGL(down_proj_kernel<4>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
    default: hipLaunchKernelGGL(down_proj_kernel<8>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
  }
  const int64_t count = M * R;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, part, splits,
                     count, scale, out);
}

int token_grad_splits(int64_t M, int64_t J, int R) {
  const int64_t tiles = cdiv(J, tg::JT);
  const int64_t stages = cdiv(M, tg::TT);
  int64_t want = cdiv(target_wgs(R), tiles);
  if (want < 1) want = 1;
  if (want > stages) want = stages;
  if (want > 64) want = 64;
  return (int)cdiv(M, cdiv(cdiv(M, want), tg::TT) * tg::TT);
}

void launch_token_grad(const uint16_t* X, int64_t M, int64_t J, int64_t Jout, const float* Y, int R, float s,
                       int splits, float* part, int transpose_out, uint16_t* out, hipStream_t stream,
                       const DropoutDev* drop) {
  const int64_t tc = cdiv(cdiv(M, splits), tg::TT) * tg::TT;
  const dim3 grid((unsigned)cdiv(J, tg::JT), (unsigned)splits);
  const DropoutDev d = drop ? *drop : DropoutDev{0u, 0u, 0u, 0ull, 0};
  switch (rank_blocks(R)) {
    case 1: hipLaunchKernelGGL(token_grad_kernel<1>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
    case 2: hipLaunchKernelGGL(token_grad_kernel<2>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
    case 4: hipLaunchKernelGGL(token_grad_kernel<4>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
    default: hipLaunchKernelGGL(token_grad_kernel<8>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
  }
  const int64_t count = Jout * R;
  hipLaunchKernelGGL(reduce_grad_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, part, splits, J,
                     Jout, R, s, transpose_out, out);
}

// The adapter part of grad_x under dropout, in fp32 for the grad_x GEMM to
// add before its single bf16 rounding:
//   out[t][f] = scale * keep(t, f) * sum_q v[t][q] A[q][f],  scale = s / (1 - p)
// (the chain rule through the dropped adapter input).  Workgroup: 32 tokens x
// 128 features; v rows and the A tile are staged in LDS; a thread owns 4
// tokens x 4 consecutive features (one Philox call gives their 4 words).
// LDS is sized to the rank (RB blocks of 16), so small ranks keep many
// workgroups per CU.
template <int RB>
__global__ __launch_bounds__(256) void lora_dropout_term_kernel(const float* __restrict__ v,
                                                                const uint16_t* __restrict__ A, int64_t M,
                                                                int64_t n, int R, float scale, DropoutDev drop,
                                                                float* __restrict__ out) {
  __shared__ float sv[32][16 * RB + 1];
  __shared__ __align__(16) uint16_t sa[16 * RB][128];
  const int tid = threadIdx.x;
  // 1D grid (the token tile count can exceed the 65535 limit of a grid's y)
  const int64_t nft = (n + 127) / 128;
  const int64_t t0 = ((int64_t)blockIdx.x / nft) * 32;
  const int64_t f0 = ((int64_t)blockIdx.x % nft) * 128;
  for (int i = tid; i < 32 * R; i += 256) {
    const int t = i / R, q = i % R;
    sv[t][q] = t0 + t < M ? v[(t0 + t) * R + q] : 0.0f;
  }
  for (int i = tid; i < R * 16; i += 256) {
    const int q = i / 16, c = i % 16;
    const int64_t f = f0 + 8 * c;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (f < n) w = *reinterpret_cast<const u32x4*>(A + (int64_t)q * n + f);
    *reinterpret_cast<u32x4*>(&sa[q][8 * c]) = w;
  }
  __syncthreads();
  const int fl = 4 * (tid & 31);
  const int tl = 4 * (tid >> 5);
  float acc[4][4] = {};
  for (int q = 0; q < R; ++q) {
    const uint32_t a01 = *reinterpret_cast<const uint32_t*>(&sa[q][fl]);
    const uint32_t a23 = *reinterpret_cast<const uint32_t*>(&sa[q][fl + 2]);
    const float a[4] = {bf16_lo_to_f32(a01), bf16_hi_to_f32(a01), bf16_lo_to_f32(a23), bf16_hi_to_f32(a23)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float vv = sv[tl + e][q];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[e][c] = __builtin_fmaf(vv, a[c], acc[e][c]);
    }
  }
  const int64_t f = f0 + fl;
  if (f >= n) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t t = t0 + tl + e;
    if (t >= M) break;
    const uint64_t c = ((uint64_t)(t * n + f) >> 2) + drop.offset;
    const u32x4 r = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), drop.k0, drop.k1);
    f32x4 o;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) o[cc] = r[cc] >= drop.thr ? scale * acc[e][cc] : 0.0f;
    *reinterpret_cast<f32x4*>(out + t * n + f) = o;
  }
}

void launch_lora_dropout_term(const float* v, const uint16_t* A, int64_t M, int64_t n, int R, float scale,
                              const DropoutDev& drop, float* out, hipStream_t stream) {
  const dim3 grid((unsigned)(cdiv(n, 128) * cdiv(M, 32)));
  switch (rank_blocks(R)) {
    case 1: hipLaunchKernelGGL(lora_dropout_term_kernel<1>, grid, dim3(256), 0, stream, v, A, M, n, R, scale, drop, out); break;
    case 2: hipLaunchKernelGGL(lora_dropout_term_kernel<2>, grid, dim3(256), 0, stream, v, A, M, n, R, scale, drop, out); break;
    case 4: hipLaunchKernelGGL(lora_dropout_term_kernel<4>, grid, dim3(256), 0, stream, v, A, M, n, R, scale, drop, out); break;
    default: hipLaunchKernelGGL(lora_dropout_term_kernel<8>, grid, dim3(256), 0, stream, v, A, M, n, R, scale, drop, out); break;
  }
}

// v and grad_B from one read of g (R % 8 == 0, R <= 32): vpart holds
// gpass_splits_f(J, R) x M x R floats, gbpart gpass_splits_t(M) x J x R.
bool gpass_supported(int R) { return R % 8 == 0 && R <= 32; }
static inline int gpass_sf(int R) { return R <= 16 ? 4 : 2; }
int gpass_splits_f(int64_t J, int R) { return (int)cdiv(J, gp::FT * gpass_sf(R)); }
int gpass_splits_t(int64_t M) { return (int)cdiv(M, gp::TT * gp::ST); }

void launch_gpass(const uint16_t* G, int64_t M, int64_t J, const uint16_t* B, int64_t m, const float* U, int R,
                  float s, float* vpart, float* gbpart, float* v, uint16_t* grad_B, hipStream_t stream) {
  const int sf = gpass_splits_f(J, R), st = gpass_splits_t(M);
  const dim3 grid((unsigned)((int64_t)sf * st));
  if (R <= 16)
    hipLaunchKernelGGL((gpass_kernel<1, 4>), grid, dim3(256), 0, stream, G, M, J, B, m, U, R, vpart, gbpart);
  else
    hipLaunchKernelGGL((gpass_kernel<2, 2>), grid, dim3(256), 0, stream, G, M, J, B, m, U, R, vpart, gbpart);
  const int64_t count = M * R;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, vpart, sf, count,
                     1.0f, v);
  const int64_t gcount = m * R;
  hipLaunchKernelGGL(reduce_grad_kernel, dim3((unsigned)cdiv(gcount, 256)), dim3(256), 0, stream, gbpart, st, J, m,
                     R, s, 0, grad_B);
}

void launch_pad_cols_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t cols_pad, uint16_t* out,
                          hipStream_t stream) {
  const int64_t count = rows * cols_pad;
  hipLaunchKernelGGL(pad_cols_bf16_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, in, rows, cols,
                     cols_pad, out);
}

void launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld, uint16_t* out,
                           hipStream_t stream) {
  const int64_t count = cols * ld;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, in, rows, cols,
                     ld, out);
}

}  // namespace qlora
