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

// out[i] = scale * sum_s part[s][i], summed in split order (fp32); also
// clears the next GEMM's hand-off words z
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int nsplit, int64_t count,
                                                            float scale, float* __restrict__ out, SyncZero z) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < z.n) z.p[i] = 0u;
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
// (v = sum_fs vpart, grad_B = s sum_ts gbpart).  A workgroup owns 64 ST
// tokens x 128 SF features of g (ST = SF = 1 up to 64 tokens, ST = 2 and
// SF = 1 up to 128, otherwise ST = 4 and SF = 512 / (128 RB): few tokens
// then still give one workgroup per 128 features instead of tiles that are
// mostly past M) and walks them as ST SF sub-tiles of 64 x 128 (feature
// sub-tile outer).  Per sub-tile every wave adds 16 tokens' worth
// of v (A = g rows, B operand = B read transposed from its natural [f][q]
// tile) and 32 features' worth of grad_B (A = g columns read transposed, B
// operand = u as bf16 hi + lo planes [q][t]) into accumulators that live
// through the whole walk.  R a multiple of 8 and at most 16 RB.
// ---------------------------------------------------------------------------
namespace gp {
constexpr int TT = 64;        // tokens per sub-tile
constexpr int FT = 128;       // features per sub-tile
constexpr int GB = TT * 256;  // g sub-tile bytes
}  // namespace gp

template <int RB, int SF, int ST>
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
  const int64_t t0 = (int64_t)ts * gp::TT * ST;

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
    const int64_t fb = f0 + (int64_t)(i / ST) * gp::FT;
    const int64_t tb = t0 + (int64_t)(i % ST) * gp::TT;
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

  f32x4 av[ST][RB];        // v: tokens 64 ts' + 16 wave + 4 lk + e, rank 16 cb + lr
  f32x4 ab[SF][2][RB];     // grad_B: features 128 fs' + 32 wave + 16 ib + 4 lk + e, rank 16 cb + lr
#pragma unroll
  for (int i = 0; i < ST; ++i)
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
    const int fsub = i / ST, tsub = i % ST;
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
  constexpr int NS = ST * SF;
  constexpr int D = (RB == 1 ? 4 : 2) < NS ? (RB == 1 ? 4 : 2) : NS;
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
  for (int i = 0; i < ST; ++i)
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
__device__ __forceinline__ void reduce_grad_body(int64_t i, const float* __restrict__ part, int nsplit, int64_t J,
                                                 int64_t Jout, int R, float s, int transpose_out,
                                                 uint16_t* __restrict__ out) {
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

// The transposed case of reduce_grad_body (out [R][Jout]): thread (g, q)
// sums rows j = 8 g .. 8 g + 7 at column q, each in split order from 0 as
// sum_splits adds them, and writes the 8 results as 16 contiguous bytes of
// out's row q.  A wave's loads of one row j are R consecutive floats, and
// up to 16 loads of a thread are in flight together (one element per
// thread wrote 2 bytes at stride Jout and waited for each element's loads).
__device__ __forceinline__ void reduce_grad_t_body(int64_t i, const float* __restrict__ part, int nsplit, int64_t J,
                                                   int64_t Jout, int R, float s, uint16_t* __restrict__ out) {
  const int64_t groups = (Jout + 7) / 8;
  if (i >= groups * R) return;
  const int q = (int)(i % R);
  const int64_t j0 = (i / R) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < nsplit; k0 += 2) {
    float v[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[c][e] = (k0 + c < nsplit && j0 + e < Jout) ? part[(int64_t)(k0 + c) * J * R + (j0 + e) * R + q] : 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + c < nsplit) acc[e] += v[c][e];
  }
  uint16_t* dst = out + (int64_t)q * Jout + j0;
  if ((Jout & 7) == 0) {
    *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(s * acc[0], s * acc[1]), pack_bf16x2(s * acc[2], s * acc[3]),
                                           pack_bf16x2(s * acc[4], s * acc[5]), pack_bf16x2(s * acc[6], s * acc[7])};
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < Jout) dst[e] = (uint16_t)(pack_bf16x2(s * acc[e], 0.f) & 0xFFFFu);
  }
}

// Both adapter gradients' split sums in one launch: workgroups below nb
// finish grad_B ([Jout][R], reduce_grad_body), the rest grad_A ([R][Jout],
// reduce_grad_t_body); each sum adds the splits in order from 0.
struct GradSum {
  const float* part;
  int nsplit;
  int64_t J, Jout;
  int R;
  float s;
  uint16_t* out;
};
__global__ __launch_bounds__(256) void reduce_grads_kernel(GradSum b, GradSum a, int nb, SyncZero z) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi < z.n) z.p[gi] = 0u;  // the next GEMM's hand-off words
  if ((int)blockIdx.x < nb)
    reduce_grad_body((int64_t)blockIdx.x * 256 + threadIdx.x, b.part, b.nsplit, b.J, b.Jout, b.R, b.s, 0, b.out);
  else
    reduce_grad_t_body((int64_t)(blockIdx.x - nb) * 256 + threadIdx.x, a.part, a.nsplit, a.J, a.Jout, a.R, a.s,
                       a.out);
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
// ld >= rows and out[c][rows:ld] = 0.  One thread per output element (B^T
// of a 70B layer, 28672 x 64: 10 us; a tile transpose through LDS was no
// faster there and twice as slow on 1024 x 64, its load - barrier - store
// chain being longer than the whole launch).
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                             int64_t cols, int64_t ld, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= cols * ld) return;
  const int64_t c = i / ld, r = i % ld;
  out[i] = r < rows ? in[r * cols + c] : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// Streaming adapter products for many tokens (the masked calls of LoRA
// dropout keep the kernels above, which apply the mask between load and
// LDS store):
//   skinny_down_kernel : part[split][t][q] = sum_{k in split} X[t][k] Y[q][k]
//   skinny_token_kernel: part[split][j][q] = sum_{t in split} X[t][j] P[q][t]
// X streams through an NS-stage LDS ring filled by direct-to-LDS buffer loads
// (no registers in between, no LDS store instructions), the small operand
// rides along the same way in bf16: A or B^T for the down products; for the
// token products the fp32 factor (u or v) as bf16 hi and lo planes [q][t],
// written once per call by factor_planes_kernel.  Each stage is a separate
// LDS array and every loop over the ring is unrolled by NS, so the compiler
// sees which stage each fragment read touches and does not make it wait for
// the loads in flight into the other stages.  A wave waits only for its own
// loads of the stage it is about to read (loads complete in order), then
// one barrier publishes the stage and frees the oldest one for the next
// loads.  Rows, columns and k past the split or the tensor read as zero
// (out-of-range buffer offsets).
// ---------------------------------------------------------------------------
namespace sk {
constexpr int DT = 128;   // down: tokens per workgroup (32 per wave)
constexpr int DCH = 8;    // down: 16-byte chunks per token row and stage (8 CH k)
constexpr int TJ = 128;   // token: columns per workgroup (32 per wave)
constexpr int TS = 64;    // token: tokens per stage
}  // namespace sk

// s_waitcnt vmcnt(N) with the other counters unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// One direct-to-LDS load of 16 bytes per lane: lane l writes bytes
// 16 l .. 16 l + 15 of the 1 KB block at `blk`.
__device__ __forceinline__ void dma16(brsrc_t r, uint8_t* blk, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)blk, 16, voff, 0, 0, 0);
}

// 16-byte chunk c (0..7) of row `row` in a tile of 128-byte rows sits at
// slot c ^ (row % 8): 16x16x32 fragment reads and 1 KB block writes are free
// of bank conflicts.
__device__ __forceinline__ uint32_t sw128(int row, int c) { return (uint32_t)(row * 128 + ((c ^ (row & 7)) << 4)); }

// Workgroup barrier without __syncthreads' memory fence, which the compiler
// lowers to a wait for every load in flight (the whole ring).  The ring's
// own vmcnt wait makes this wave's loads of the stage complete, the barrier
// makes every wave's, and LDS needs no cache maintenance; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The ring: stage s lives in buffer s % NS; step s waits for stage s, issues
// stage s + NS - 1 into the buffer of stage s - 1 (free after the barrier)
// and computes stage s.  Loads are issued unconditionally: stages past the
// end read only out-of-range offsets (zeros, no memory traffic) into buffers
// nobody reads again.  So before the wait of step s exactly the stages
// s .. s + NS - 2 are in flight, and since loads retire in order, allowing
// the later stages' loads to stay outstanding leaves stage s complete (LMIN:
// the loads every wave issues per stage; waves that issue more only wait
// longer).  A conditional issue would make the compiler wait for every load
// in flight where the paths meet, so the steady-state loop runs whole rings
// and the remaining steps follow it.  The final wait keeps late loads from
// writing LDS after the workgroup has ended.
template <int NS, int LMIN, typename Issue, typename Compute>
__device__ __forceinline__ void ring_run(int nst, uint8_t* const (&buf)[NS], Issue issue, Compute compute) {
  static_assert(NS >= 3 && NS <= 4, "ring depth");
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) issue(u, buf[u]);
  auto step = [&](int s, int u) {
    wait_vmcnt<LMIN * (NS - 2)>();
    ring_barrier();
    issue(s + NS - 1, buf[(u + NS - 1) % NS]);
    compute(buf[u]);
  };
  const int full = nst - nst % NS;
  for (int s0 = 0; s0 < full; s0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) step(s0 + u, u);
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (full + u < nst) step(full + u, u);
  wait_vmcnt<0>();
}

// CH 16-byte chunks (8 CH k) per token row and stage: chunk c of row r
// sits at slot c ^ (r % CH), so 16x16x32 fragment reads are conflict-free.
template <int CH>
__device__ __forceinline__ uint32_t swch(int row, int c) {
  return (uint32_t)(row * (16 * CH) + ((c ^ (row & (CH - 1))) << 4));
}

// kYT: Y is given as [k][q] (B itself, R = 16 RB ranks, rows past yrows
// read as zero) instead of [q][k]; its stage tile keeps that layout (KS rows
// of 32 RB bytes, loaded as contiguous 1 KB blocks) and the MFMA operand is
// read transposed with ds_read_b64_tr_b16, so v = g B needs no copy of B^T.
template <int RB, int NS, int CH, bool kYT>
__global__ __launch_bounds__(256) void skinny_down_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                          const uint16_t* __restrict__ Y, int R,
                                                          float* __restrict__ part, int64_t kc, int64_t yrows) {
  static_assert(CH == 8 || CH == 16, "row chunks per stage");
  static_assert(!kYT || CH == 8, "transposed rank operand: 64 k per stage");
  constexpr int KS = 8 * CH;               // k per stage
  constexpr int RPB = 64 / CH;             // rows per 1 KB load block
  constexpr int XPW = 32 / RPB;            // X blocks per wave (its 32 token rows)
  // Rank rows: 16 RB rows of CH chunks, in 1 KB blocks, YPW per wave (every
  // wave issues the same number of loads; blocks past the rank rows read
  // zeros into the padding)
  constexpr int YBLK = (16 * RB) / RPB;
  constexpr int YPW = YBLK >= 4 ? YBLK / 4 : 1;
  constexpr int XB = sk::DT * 16 * CH;     // 128 token rows x KS k
  constexpr int YB = 4 * YPW * 1024;
  constexpr int STAGE = XB + YB;
  __shared__ __align__(16) uint8_t s0[STAGE];
  __shared__ __align__(16) uint8_t s1[STAGE];
  __shared__ __align__(16) uint8_t s2[NS > 2 ? STAGE : 16];
  __shared__ __align__(16) uint8_t s3[NS > 3 ? STAGE : 16];
  uint8_t* const buf4[4] = {s0, s1, s2, s3};
  uint8_t* buf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) buf[i] = buf4[i];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * sk::DT;
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * kc;
  const int64_t kend = (kbeg + kc < K) ? kbeg + kc : K;
  const int nst = (int)cdiv(kend - kbeg, KS);
  const uint32_t xbytes = (uint32_t)(M * K * 2);
  const uint32_t ybytes = (uint32_t)((int64_t)R * (kYT ? yrows : K) * 2);
  const brsrc_t rx = make_rsrc(X, xbytes);
  const brsrc_t ry = make_rsrc(Y, ybytes);
  // A 1 KB load block holds RPB rows: lane l lands in row l / CH of the
  // block at slot l % CH, which holds chunk (l % CH) ^ (row % CH) (swch).
  const int drow = lane / CH;
  const int dslot = lane % CH;
  constexpr int LMIN = XPW + YPW;
  auto issue = [&](int s, uint8_t* stg) {
    const int64_t kb = kbeg + (int64_t)s * KS;
#pragma unroll
    for (int b = 0; b < XPW; ++b) {  // this wave's token rows 32 w .. 32 w + 31
      const int row = 32 * wave + RPB * b + drow;
      const int64_t k = kb + 8 * (dslot ^ (row & (CH - 1)));
      const int64_t t = t0 + row;
      dma16(rx, stg + (32 * wave + RPB * b) * (16 * CH), (k < kend && t < M) ? (uint32_t)((t * K + k) * 2) : xbytes);
    }
#pragma unroll
    for (int j = 0; j < YPW; ++j) {
      const int blk = wave + 4 * j;
      if constexpr (kYT) {
        // rows kb + 1024 / (32 RB) blk .. of B, 2 RB lanes a row (KS rows in all)
        const int row = (1024 / (32 * RB)) * blk + lane / (2 * RB);
        const int64_t k = kb + row;
        const int c = lane % (2 * RB);
        dma16(ry, stg + XB + blk * 1024, (k < kend && row < KS) ? (uint32_t)((k * R + 8 * c) * 2) : ybytes);
      } else {
        const int q = RPB * blk + drow;
        const int64_t k = kb + 8 * (dslot ^ (q & (CH - 1)));
        dma16(ry, stg + XB + blk * 1024, (k < kend && q < R) ? (uint32_t)(((int64_t)q * K + k) * 2) : ybytes);
      }
    }
  };
  f32x4 acc[2][RB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint8_t* stg) {
#pragma unroll
    for (int kk = 0; kk < CH / 4; ++kk) {
      u32x4 bq[RB];
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        if constexpr (kYT) {
          // k rows 32 kk + 8 lq + 4 h + lr / 4, ranks 16 cb + 4 (lr % 4) .. + 3
          const uint8_t* src = stg + XB + (32 * kk + 8 * lq + (lr >> 2)) * (32 * RB) + 2 * (16 * cb + 4 * (lr & 3));
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 4 * (32 * RB)));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
          bq[cb] = u32x4{l2[0], l2[1], h2[0], h2[1]};
        } else {
          bq[cb] = *reinterpret_cast<const u32x4*>(stg + XB + swch<CH>(16 * cb + lr, 4 * kk + lq));
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(stg + swch<CH>(32 * wave + 16 * i + lr, 4 * kk + lq));
#pragma unroll
        for (int cb = 0; cb < RB; ++cb) acc[i][cb] = mfma16x16x32(a, bq[cb], acc[i][cb]);
      }
    }
  };
  ring_run<NS, LMIN>(nst, buf, issue, compute);

  // lane holds tokens 32 w + 16 i + 4 lq + e, rank 16 cb + lr
  float* dst = part + (int64_t)split * M * R;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int cb = 0; cb < RB; ++cb) {
      const int q = 16 * cb + lr;
      if (q >= R) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = t0 + 32 * wave + 16 * i + 4 * lq + e;
        if (t < M) dst[t * R + q] = acc[i][cb][e];
      }
    }
}

template <int RB, int NS>
__global__ __launch_bounds__(256) void skinny_token_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t J,
                                                           const uint16_t* __restrict__ P, int64_t Mp, int R,
                                                           float* __restrict__ part, int64_t tc) {
  constexpr int XB = sk::TS * 256;     // 64 token rows x 128 columns
  constexpr int PB = RB * 16 * 128;    // one plane: 16 RB rank rows x 64 tokens
  constexpr int STAGE = XB + 2 * PB;
  __shared__ __align__(16) uint8_t s0[STAGE];
  __shared__ __align__(16) uint8_t s1[STAGE];
  __shared__ __align__(16) uint8_t s2[NS > 2 ? STAGE : 16];
  __shared__ __align__(16) uint8_t s3[NS > 3 ? STAGE : 16];
  uint8_t* const buf4[4] = {s0, s1, s2, s3};
  uint8_t* buf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) buf[i] = buf4[i];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int64_t j0 = (int64_t)blockIdx.x * sk::TJ;
  const int split = blockIdx.y;
  const int64_t tbeg = (int64_t)split * tc;
  const int64_t tend = (tbeg + tc < M) ? tbeg + tc : M;
  const int nst = (int)cdiv(tend - tbeg, sk::TS);
  const uint32_t xbytes = (uint32_t)(M * J * 2);
  const uint32_t pbytes = (uint32_t)(2 * (int64_t)R * Mp * 2);
  const brsrc_t rx = make_rsrc(X, xbytes);
  const brsrc_t rp = make_rsrc(P, pbytes);
  // X: a 1 KB load block is 4 token rows of 256 B; lane l lands in row l / 16
  // at 16-byte slot l % 16, which holds piece c of the row with
  // (c / 2) ^ f(row) == slot / 2 and c % 2 == slot % 2 (swtg).
  const int xrow = lane >> 4;
  const int slot = lane & 15;
  // Planes: a 1 KB block is 8 rank rows of 128 B; lane l lands in row l / 8,
  // slot l % 8, which holds chunk (l % 8) ^ ((q / 2) % 8) (swy).
  const int prow = lane >> 3;
  constexpr int LMIN = 4 + RB;
  auto issue = [&](int s, uint8_t* stg) {
    const int64_t tb = tbeg + (int64_t)s * sk::TS;
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // rows 16 w .. 16 w + 15 of the stage
      const int blk = 4 * wave + b;
      const int row = 4 * blk + xrow;
      const int f = (row & 3) | (((row >> 3) & 1) << 2);
      const int c = ((((slot >> 1) ^ f)) << 1) | (slot & 1);
      const int64_t t = tb + row;
      const int64_t j = j0 + 8 * c;
      dma16(rx, stg + blk * 1024, (t < tend && j < J) ? (uint32_t)((t * J + j) * 2) : xbytes);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {  // blocks 4 b + w of the two planes (2 RB blocks each)
      const int id = 4 * b + wave;
      const int pl = id / (2 * RB);
      const int q = 8 * (id % (2 * RB)) + prow;
      const int c = (lane & 7) ^ ((q >> 1) & 7);
      dma16(rp, stg + XB + pl * PB + (id % (2 * RB)) * 1024,
            (q < R && tb < tend) ? (uint32_t)((((int64_t)pl * R + q) * Mp + tb + 8 * c) * 2) : pbytes);
    }
  };
  f32x4 acc[2][RB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < RB; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tr_row = lr >> 2;
  const int tr_c = lr & 3;
  auto compute = [&](const uint8_t* stg) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        // lanes 4 r + c of each 16-lane group address token row r, columns 4 c .. 4 c + 3
        const int t = 32 * kk + 8 * lq + tr_row;
        const int c = 2 * (2 * wave + ib) + (tr_c >> 1);
        const uint8_t* p0 = stg + swtg(t, c) + (tr_c & 1) * 8;
        const uint8_t* p1 = stg + swtg(t + 4, c) + (tr_c & 1) * 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a[ib] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int cb = 0; cb < RB; ++cb) {
        const uint32_t off = swy(16 * cb + lr, 4 * kk + lq);
        const u32x4 bh = *reinterpret_cast<const u32x4*>(stg + XB + off);
        const u32x4 bl = *reinterpret_cast<const u32x4*>(stg + XB + PB + off);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          acc[ib][cb] = mfma16x16x32(a[ib], bh, acc[ib][cb]);
          acc[ib][cb] = mfma16x16x32(a[ib], bl, acc[ib][cb]);
        }
      }
    }
  };
  ring_run<NS, LMIN>(nst, buf, issue, compute);

  // lane holds columns j = 32 w + 16 ib + 4 lq + e, rank q = 16 cb + lr
  float* dst = part + (int64_t)split * J * R;
#pragma unroll
  for (int cb = 0; cb < RB; ++cb) {
    const int q = 16 * cb + lr;
    if (q >= R) continue;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + 32 * wave + 16 * ib + 4 * lq + e;
        if (j < J) dst[j * R + q] = acc[ib][cb][e];
      }
  }
}

// bf16 hi / lo planes of an fp32 M x R factor, transposed:
//   P[0][q][t] = bf16(Y[t][q]),  P[1][q][t] = bf16(Y[t][q] - P[0][q][t]),
// zero for M <= t < Mp.  Grid y = 0 makes the planes of Y = sum of `nsplit`
// fp32 partials (stride M R, added in split order from 0, as
// reduce_splits_kernel adds them) and, if Yout is given, also writes that
// sum; grid y = 1 makes the planes P2 of a second factor Y2 (one part).  A
// workgroup takes 8 tokens (8 R <= 1024 elements, up to 4 per thread) and
// issues the loads of 4 splits of all its elements together, so a launch
// waits for memory about ceil(nsplit / 4) times (with 64 tokens and one
// element's splits at a time it waited 16 times: 15.8 us for the 70B
// block's v at r = 64, 8 splits).  Beyond 8 splits (the single-read g pass
// leaves one per 128 features for few tokens, 112 for the 8B gate
// projection) 16 go out together.  The sums are staged in LDS, then thread
// i < 2 R writes the 8 tokens of plane row i (16 bytes).
constexpr int kPlaneTok = 8;
template <bool kMany>  // beyond 8 splits (a separate instantiation keeps the other's registers)
__global__ __launch_bounds__(256) void factor_planes_kernel(const float* __restrict__ Y, int nsplit, int64_t M, int R,
                                                            int64_t Mp, uint16_t* __restrict__ P,
                                                            float* __restrict__ Yout, const float* __restrict__ Y2,
                                                            uint16_t* __restrict__ P2) {
  __shared__ float sy[kPlaneTok][kMaxRank + 1];
  const int64_t t0 = (int64_t)blockIdx.x * kPlaneTok;
  const bool second = blockIdx.y == 1;
  const float* src = second ? Y2 : Y;
  const int ns = second ? 1 : nsplit;
  uint16_t* dstp = second ? P2 : P;
  const int64_t lim = M * R;
  const int64_t base = t0 * R;
  const int n = kPlaneTok * R;
  constexpr int E = kPlaneTok * kMaxRank / 256;  // elements per thread at most
  bool ok[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = threadIdx.x + 256 * e;
    ok[e] = i < n && base + i < lim;
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  if (!kMany || ns <= 8) {
    // 4 splits' loads at a time, each under its guard
    for (int k0 = 0; k0 < ns; k0 += 4) {
      float v[4][E];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
          v[c][e] = (k0 + c < ns && ok[e]) ? src[(int64_t)(k0 + c) * lim + base + threadIdx.x + 256 * e] : 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (k0 + c < ns) acc[e] += v[c][e];
    }
  } else {
    // many splits (few tokens through the single-read g pass): 16 splits'
    // loads go out together, unconditionally (a load under a branch makes
    // the compiler wait for every load in flight where the paths meet):
    // split indices past the end repeat the last one and element indices
    // past the range read element 0; those values are added as +0, which
    // leaves the sum's bits unchanged (it starts at +0 and so is never -0)
    constexpr int KF = 16;
    for (int k0 = 0; k0 < ns; k0 += KF) {
      float v[KF][E];
#pragma unroll
      for (int c = 0; c < KF; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int64_t k = k0 + c < ns ? k0 + c : ns - 1;
          v[c][e] = src[k * lim + (ok[e] ? base + threadIdx.x + 256 * e : 0)];
        }
#pragma unroll
      for (int c = 0; c < KF; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += (k0 + c < ns && ok[e]) ? v[c][e] : 0.0f;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = threadIdx.x + 256 * e;
    if (i < n) {
      sy[i / R][i % R] = acc[e];
      if (!second && Yout && ok[e]) Yout[base + i] = acc[e];
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < 2 * R) {
    const int q = threadIdx.x % R;
    const int pl = threadIdx.x / R;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float h0, l0, h1, l1;
      split_bf16(sy[2 * e][q], h0, l0);
      split_bf16(sy[2 * e + 1][q], h1, l1);
      w[e] = pl ? pack_bf16x2(l0, l1) : pack_bf16x2(h0, h1);
    }
    *reinterpret_cast<u32x4*>(dstp + ((int64_t)pl * R + q) * Mp + t0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------
static inline int rank_blocks(int R) { return R <= 16 ? 1 : R <= 32 ? 2 : R <= 64 ? 4 : 8; }
// LDS ring depth of the streaming token kernel: three stages while two
// workgroups fit a CU, four when the hi / lo planes make a stage 32 KB.
static inline int token_stages(int R) { return rank_blocks(R) == 4 ? 4 : 3; }
// Workgroups that fit one CU (160 KB of LDS) for the streaming kernels.
static inline int down_wgs_per_cu(int R) { return rank_blocks(R) <= 4 ? 2 : 1; }
static inline int token_wgs_per_cu(int R) { return rank_blocks(R) <= 2 ? 2 : 1; }

// Split count s in 1 .. most for `tiles` tiles on `slots` resident
// workgroups: the stream takes about ceil(tiles s / slots) rounds of 1 / s of
// a tile's work, so the one with the fewest rounds per split wins (ties: the
// larger s).  E.g. 112 column tiles on 256 slots: 2 splits (224 workgroups,
// one round) instead of 3 (336 workgroups, a second round of 80).
static int64_t fewest_rounds_splits(int64_t tiles, int64_t slots, int64_t most) {
  int64_t best = 1;
  for (int64_t sp = 1; sp <= most; ++sp) {
    // rounds(sp) / sp <= rounds(best) / best, in integers
    if (cdiv(tiles * sp, slots) * best <= cdiv(tiles * best, slots) * sp) best = sp;
  }
  return best;
}

// K splits of a down product: enough 128-token tiles x splits to fill every
// CU with its resident workgroups, at most 64 splits, each at least 512 k
// long and a multiple of 128 (the masked kernel takes 128-k stages).
int down_proj_splits(int64_t M, int64_t K, int R) {
  const int64_t tiles = cdiv(M, sk::DT);
  const int64_t slots = (int64_t)down_wgs_per_cu(R) * device_cus();
  int64_t want = cdiv(slots, tiles);
  const int64_t most = cdiv(K, 512);
  if (want > most) want = most;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  want = fewest_rounds_splits(tiles, slots, want);
  return (int)cdiv(K, cdiv(cdiv(K, want), dp::KCH) * dp::KCH);
}

// drop: dropout on X (the adapter input), or null; the result is scaled by
// `scale` (1 / (1 - p) with dropout) after the fixed-order sum; with out
// null only the split partials are written.  Unmasked
// products stream through skinny_down_kernel; masked ones take
// down_proj_kernel, which applies the mask between its loads and LDS stores.
// z: hand-off words of the GEMM that follows, cleared by the split sum
// (only when out is given).
void launch_down_proj(const uint16_t* X, int64_t M, int64_t K, const uint16_t* Y, int R, float* part, int splits,
                      float* out, hipStream_t stream, const DropoutDev* drop, float scale, SyncZero z) {
  const int64_t kc = cdiv(cdiv(K, splits), dp::KCH) * dp::KCH;
  if (drop && drop->on) {
    const dim3 grid((unsigned)cdiv(M, dp::TT), (unsigned)splits);
    const DropoutDev d = *drop;
    switch (rank_blocks(R)) {
      case 1: hipLaunchKernelGGL(down_proj_kernel<1>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
      case 2: hipLaunchKernelGGL(down_proj_kernel<2>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
      case 4: hipLaunchKernelGGL(down_proj_kernel<4>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
      default: hipLaunchKernelGGL(down_proj_kernel<8>, grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, d); break;
    }
  } else {
    const dim3 grid((unsigned)cdiv(M, sk::DT), (unsigned)splits);
    constexpr int CH = sk::DCH;
    switch (rank_blocks(R)) {
      case 1: hipLaunchKernelGGL((skinny_down_kernel<1, 3, CH, false>), grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, K); break;
      case 2: hipLaunchKernelGGL((skinny_down_kernel<2, 3, CH, false>), grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, K); break;
      case 4: hipLaunchKernelGGL((skinny_down_kernel<4, 3, CH, false>), grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, K); break;
      default: hipLaunchKernelGGL((skinny_down_kernel<8, 3, CH, false>), grid, dim3(256), 0, stream, X, M, K, Y, R, part, kc, K); break;
    }
  }
  if (!out) return;  // the caller sums the partials (factor_planes_kernel)
  const int64_t count = M * R;
  const int64_t blocks = std::max(cdiv(count, 256), cdiv((int64_t)z.n, 256));
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, count, scale,
                     out, z);
}

// v partials straight from B (m x R, R = 64 or 128): part[split][t][q] =
// sum over the split's k of G[t][k] B[k][q], G M x K with K >= m (rows of B
// past m read as zero).  The split rule and partial layout of
// launch_down_proj.
bool down_proj_bt_supported(int R) { return R == 64 || R == 128; }
void launch_down_proj_bt(const uint16_t* G, int64_t M, int64_t K, const uint16_t* B, int64_t m, int R, float* part,
                         int splits, hipStream_t stream) {
  const int64_t kc = cdiv(cdiv(K, splits), dp::KCH) * dp::KCH;
  const dim3 grid((unsigned)cdiv(M, sk::DT), (unsigned)splits);
  if (R == 64)
    hipLaunchKernelGGL((skinny_down_kernel<4, 3, 8, true>), grid, dim3(256), 0, stream, G, M, K, B, R, part, kc, m);
  else
    hipLaunchKernelGGL((skinny_down_kernel<8, 3, 8, true>), grid, dim3(256), 0, stream, G, M, K, B, R, part, kc, m);
}

// Token splits of a reduction over tokens: enough 128-column tiles x splits
// to fill every CU, at most 64 splits of at least 512 tokens (multiples of 64).
int token_grad_splits(int64_t M, int64_t J, int R) {
  const int64_t tiles = cdiv(J, tg::JT);
  const int64_t slots = (int64_t)token_wgs_per_cu(R) * device_cus();
  int64_t want = cdiv(slots, tiles);
  const int64_t most = cdiv(M, 512);
  if (want > most) want = most;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  want = fewest_rounds_splits(tiles, slots, want);
  return (int)cdiv(M, cdiv(cdiv(M, want), tg::TT) * tg::TT);
}

// Bytes of the bf16 hi / lo planes of an M x R factor (token pitch M rounded
// up to 64).
size_t token_planes_bytes(int64_t M, int R) { return (size_t)2 * R * (size_t)(cdiv(M, 64) * 64) * 2; }

// Planes of Y = sum of nsplit partials (written to Yout when given) and, if
// Y2 is given, of Y2; token_planes_bytes each.
void launch_factor_planes(const float* Y, int nsplit, int64_t M, int R, uint16_t* P, float* Yout, const float* Y2,
                          uint16_t* P2, hipStream_t stream) {
  const int64_t Mp = cdiv(M, 64) * 64;
  const dim3 grid((unsigned)(Mp / kPlaneTok), Y2 ? 2u : 1u);
  if (nsplit > 8)
    hipLaunchKernelGGL(factor_planes_kernel<true>, grid, dim3(256), 0, stream, Y, nsplit, M, R, Mp, P, Yout, Y2, P2);
  else
    hipLaunchKernelGGL(factor_planes_kernel<false>, grid, dim3(256), 0, stream, Y, nsplit, M, R, Mp, P, Yout, Y2, P2);
}

// part[split][j][q] = sum over the split's tokens of X[t][j] Y[t][q]; the
// caller sums the splits (launch_reduce_grads).  Unmasked reductions stream
// through skinny_token_kernel from Y's bf16 hi / lo planes (`planes`,
// token_planes_bytes), made here unless planes_ready; masked ones (drop on)
// take token_grad_kernel, which reads Y itself.
void launch_token_grad(const uint16_t* X, int64_t M, int64_t J, const float* Y, int R, int splits, float* part,
                       hipStream_t stream, const DropoutDev* drop, uint16_t* planes, bool planes_ready) {
  const int64_t tc = cdiv(cdiv(M, splits), tg::TT) * tg::TT;
  const dim3 grid((unsigned)cdiv(J, tg::JT), (unsigned)splits);
  if (drop && drop->on) {
    const DropoutDev d = *drop;
    switch (rank_blocks(R)) {
      case 1: hipLaunchKernelGGL(token_grad_kernel<1>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
      case 2: hipLaunchKernelGGL(token_grad_kernel<2>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
      case 4: hipLaunchKernelGGL(token_grad_kernel<4>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
      default: hipLaunchKernelGGL(token_grad_kernel<8>, grid, dim3(256), 0, stream, X, M, J, Y, R, part, tc, d); break;
    }
  } else {
    const int64_t Mp = cdiv(M, 64) * 64;
    if (!planes_ready) launch_factor_planes(Y, 1, M, R, planes, nullptr, nullptr, nullptr, stream);
    switch (rank_blocks(R)) {
      case 1: hipLaunchKernelGGL((skinny_token_kernel<1, 3>), grid, dim3(256), 0, stream, X, M, J, planes, Mp, R, part, tc); break;
      case 2: hipLaunchKernelGGL((skinny_token_kernel<2, 3>), grid, dim3(256), 0, stream, X, M, J, planes, Mp, R, part, tc); break;
      case 4: hipLaunchKernelGGL((skinny_token_kernel<4, 4>), grid, dim3(256), 0, stream, X, M, J, planes, Mp, R, part, tc); break;
      default: hipLaunchKernelGGL((skinny_token_kernel<8, 3>), grid, dim3(256), 0, stream, X, M, J, planes, Mp, R, part, tc); break;
    }
  }
}

// grad_B = bf16(s_b sum of bpart's nb_split [Jb][R] partials) over the
// first mb rows ([mb][R]) and grad_A = bf16(s_a sum of apart's na_split
// [Ja][R] partials) over the first na rows, written transposed ([R][na]),
// in one launch.
void launch_reduce_grads(const float* bpart, int nb_split, int64_t Jb, int64_t mb, float s_b, uint16_t* grad_B,
                         const float* apart, int na_split, int64_t Ja, int64_t na, float s_a, uint16_t* grad_A, int R,
                         hipStream_t stream, SyncZero z) {
  const GradSum b{bpart, nb_split, Jb, mb, R, s_b, grad_B};
  const GradSum a{apart, na_split, Ja, na, R, s_a, grad_A};
  const int nbw = (int)cdiv(mb * R, 256);
  const int naw = (int)cdiv(cdiv(na, 8) * R, 256);
  const int64_t blocks = std::max((int64_t)(nbw + naw), cdiv((int64_t)z.n, 256));
  hipLaunchKernelGGL(reduce_grads_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, b, a, nbw, z);
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

// v and grad_B partials from one read of g (R % 8 == 0, R <= 32): vpart
// holds gpass_splits_f(M, J, R) x M x R floats (summed by
// factor_planes_kernel), gbpart gpass_splits_t(M) x J x R (summed by
// launch_reduce_grads).
bool gpass_supported(int R) { return R % 8 == 0 && R <= 32; }
static inline int gpass_st(int64_t M) { return M <= 64 ? 1 : M <= 128 ? 2 : 4; }
static inline int gpass_sf(int64_t M, int R) { return M <= 128 ? 1 : R <= 16 ? 4 : 2; }
int gpass_splits_f(int64_t M, int64_t J, int R) { return (int)cdiv(J, gp::FT * gpass_sf(M, R)); }
int gpass_splits_t(int64_t M) { return (int)cdiv(M, gp::TT * gpass_st(M)); }

void launch_gpass(const uint16_t* G, int64_t M, int64_t J, const uint16_t* B, int64_t m, const float* U, int R,
                  float* vpart, float* gbpart, hipStream_t stream) {
  const int sf = gpass_splits_f(M, J, R), st = gpass_splits_t(M);
  const dim3 grid((unsigned)((int64_t)sf * st));
  const int sub_t = gpass_st(M);
#define QLORA_GPASS(RB_, SF_, ST_) \
  hipLaunchKernelGGL((gpass_kernel<RB_, SF_, ST_>), grid, dim3(256), 0, stream, G, M, J, B, m, U, R, vpart, gbpart)
  if (R <= 16) {
    if (sub_t == 1) QLORA_GPASS(1, 1, 1);
    else if (sub_t == 2) QLORA_GPASS(1, 1, 2);
    else QLORA_GPASS(1, 4, 4);
  } else {
    if (sub_t == 1) QLORA_GPASS(2, 1, 1);
    else if (sub_t == 2) QLORA_GPASS(2, 1, 2);
    else QLORA_GPASS(2, 2, 4);
  }
#undef QLORA_GPASS
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
