// The rank-r adapter products of the adapted linear layer.
//   u = x A^T, v = g B             (down-projections, split over K)
//   grad_A = s v^T x, grad_B = s g^T u   (reductions over tokens)
// "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3, the low-rank term B A x)
// and Step 4 (Eq. 5, the adapter gradients), with the alpha/r scale of the
// LoraConfig snippet.  All products run on bf16 MFMA with fp32 accumulation;
// fp32 operands (u, v) enter as a bf16 hi + lo pair.  Every reduction over a
// split dimension goes through fp32 partials summed in a fixed order, so
// results are deterministic.
#include "qlora_common.h"

namespace qlora {

// ---------------------------------------------------------------------------
// out_part[split][t][q] = sum_{k in split} X[t][k] * Y[q][k]
// X: M x K bf16 (row stride K), Y: R x K bf16.  Workgroup: 64 tokens (16 per
// wave) x all R columns, K range [split*kc, split*kc + kc) walked in 256-wide
// chunks with the Y chunk staged in LDS (chunk index XOR-swizzled by row).
// ---------------------------------------------------------------------------
namespace sk {
constexpr int KCH = 256;                 // K per LDS chunk
constexpr int YROWB = KCH * 2;           // 512 B
}  // namespace sk

__global__ __launch_bounds__(256) void skinny_nt_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                        const uint16_t* __restrict__ Y, int R,
                                                        float* __restrict__ part, int64_t kc) {
  __shared__ __align__(16) uint8_t sY[kMaxRank * sk::YROWB];  // 64 KB
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lk = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int64_t kbeg = (int64_t)split * kc;
  const int64_t kend = (kbeg + kc < K) ? kbeg + kc : K;
  const int RB = (R + 15) >> 4;
  const int Rp = RB * 16;
  const int64_t t = t0 + 16 * wave + lr;  // token row this lane feeds to MFMA
  const bool t_ok = t < M;
  const bool kvec = (K & 7) == 0;

  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t kb = kbeg; kb < kend; kb += sk::KCH) {
    __syncthreads();
    // stage Y[0:Rp][kb : kb+256] (zero past R or K)
    for (int id = tid; id < Rp * 32; id += 256) {
      const int row = id >> 5, c = id & 31;
      const int64_t k = kb + 8 * c;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (row < R) {
        const uint16_t* src = Y + (int64_t)row * K + k;
        if (kvec && k + 8 <= kend) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 8; ++e)
            if (k + e < kend) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      *reinterpret_cast<u32x4*>(sY + row * sk::YROWB + ((c ^ (row & 7)) << 4)) = v;
    }
    __syncthreads();
#pragma unroll 2
    for (int s8 = 0; s8 < sk::KCH / 32; ++s8) {
      const int64_t k = kb + 32 * s8 + 8 * lk;
      u32x4 a = u32x4{0u, 0u, 0u, 0u};
      if (t_ok) {
        const uint16_t* src = X + t * K + k;
        if (kvec && k + 8 <= kend) {
          a = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 8; ++e)
            if (k + e < kend) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
          a = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      const int c = 4 * s8 + lk;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        if (cb < RB) {
          const int row = 16 * cb + lr;
          const u32x4 b = *reinterpret_cast<const u32x4*>(sY + row * sk::YROWB + ((c ^ (row & 7)) << 4));
          acc[cb] = mfma16x16x32(a, b, acc[cb]);
        }
      }
    }
  }
  // lane holds rows (tokens) 16*wave + 4*lk + e, column q = 16*cb + lr
  float* dst = part + (int64_t)split * M * R;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    if (cb >= RB) break;
    const int q = 16 * cb + lr;
    if (q >= R) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t tt = t0 + 16 * wave + 4 * lk + e;
      if (tt < M) dst[tt * R + q] = acc[cb][e];
    }
  }
}

// out[i] = sum_s part[s][i] in split order (fp32)
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int nsplit, int64_t count,
                                                            float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int k = 0; k < nsplit; ++k) s += part[(int64_t)k * count + i];
  out[i] = s;
}

// ---------------------------------------------------------------------------
// part[split][j][q] = sum_{t in split} X[t][j] * Y[t][q]
// X: M x J bf16, Y: M x R fp32.  Workgroup: 256 columns j (64 per wave) x all
// R, token range of the split walked 64 at a time.  The X tile [64 t][256 j]
// is staged in its natural layout and read transposed (ds_read_b64_tr_b16);
// Y is staged transposed as bf16 hi and lo planes [q][t].
// ---------------------------------------------------------------------------
namespace lg {
constexpr int TT = 64;
constexpr int XROWB = 256 * 2 + 32;   // padded row of the X tile
constexpr int XTILEB = TT * XROWB;    // 34816
constexpr int YROWB = TT * 2;         // 128 B per q row
constexpr int YPLANEB = kMaxRank * YROWB;  // 16 KB
}  // namespace lg

__global__ __launch_bounds__(256) void lora_grad_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t J,
                                                        const float* __restrict__ Y, int R,
                                                        float* __restrict__ part, int64_t tc) {
  __shared__ __align__(16) uint8_t sX[lg::XTILEB];
  __shared__ __align__(16) uint8_t sYh[lg::YPLANEB];
  __shared__ __align__(16) uint8_t sYl[lg::YPLANEB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lk = lane >> 4;
  const int64_t j0 = (int64_t)blockIdx.x * 256;
  const int split = blockIdx.y;
  const int64_t tbeg = (int64_t)split * tc;
  const int64_t tend = (tbeg + tc < M) ? tbeg + tc : M;
  const int RB = (R + 15) >> 4;
  const int Rp = RB * 16;
  const bool jvec = (J & 7) == 0;
  const int tr_row = lr >> 2;
  const int tr_col = 4 * (lr & 3);

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t tb = tbeg; tb < tend; tb += lg::TT) {
    __syncthreads();
    // X tile: 64 rows x 32 chunks of 16 B
    for (int id = tid; id < lg::TT * 32; id += 256) {
      const int row = id >> 5, c = id & 31;
      const int64_t t = tb + row;
      const int64_t j = j0 + 8 * c;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (t < tend) {
        const uint16_t* src = X + t * J + j;
        if (jvec && j + 8 <= J) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int e = 0; e < 8; ++e)
            if (j + e < J) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      *reinterpret_cast<u32x4*>(sX + row * lg::XROWB + 16 * c) = v;
    }
    // Y tile transposed into bf16 hi / lo planes; chunk of 8 tokens XOR-swizzled by q
    for (int id = tid; id < lg::TT * Rp; id += 256) {
      const int trow = id / Rp, q = id % Rp;
      const int64_t t = tb + trow;
      const float y = (t < tend && q < R) ? Y[t * R + q] : 0.0f;
      float h, l;
      split_bf16(y, h, l);
      const uint32_t off = q * lg::YROWB + ((((trow >> 3) ^ (q & 7))) << 4) + (trow & 7) * 2;
      *reinterpret_cast<uint16_t*>(sYh + off) = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
      *reinterpret_cast<uint16_t*>(sYl + off) = (uint16_t)(pack_bf16x2(l, 0.f) & 0xFFFFu);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int trow = 32 * kk + 8 * lk + tr_row;
        const int jcol = 64 * wave + 16 * i + tr_col;
        uint8_t* base = sX + trow * lg::XROWB + jcol * 2;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 4 * lg::XROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        a[i] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
      const int c = 4 * kk + lk;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        if (cb < RB) {
          const int q = 16 * cb + lr;
          const uint32_t off = q * lg::YROWB + ((c ^ (q & 7)) << 4);
          const u32x4 bh = *reinterpret_cast<const u32x4*>(sYh + off);
          const u32x4 bl = *reinterpret_cast<const u32x4*>(sYl + off);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][cb] = mfma16x16x32(a[i], bh, acc[i][cb]);
            acc[i][cb] = mfma16x16x32(a[i], bl, acc[i][cb]);
          }
        }
      }
    }
  }
  // lane holds rows j = 64*wave + 16*i + 4*lk + e, column q = 16*cb + lr
  float* dst = part + (int64_t)split * J * R;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    if (cb >= RB) break;
    const int q = 16 * cb + lr;
    if (q >= R) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + 64 * wave + 16 * i + 4 * lk + e;
        if (j < J) dst[j * R + q] = acc[i][cb][e];
      }
  }
}

// out = bf16(s * sum_s part[s]); part is [J][R]; out is [J][R] or, when
// transpose_out, [R][J].
__global__ __launch_bounds__(256) void reduce_grad_kernel(const float* __restrict__ part, int nsplit, int64_t J,
                                                          int R, float s, int transpose_out,
                                                          uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t count = J * R;
  if (i >= count) return;
  float acc = 0.0f;
  for (int k = 0; k < nsplit; ++k) acc += part[(int64_t)k * count + i];
  const uint16_t b = (uint16_t)(pack_bf16x2(s * acc, 0.f) & 0xFFFFu);
  if (!transpose_out) {
    out[i] = b;
  } else {
    const int64_t j = i / R, q = i % R;
    out[q * J + j] = b;
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

// out[c][r] = in[r][c] for a rows x cols bf16 matrix
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                             int64_t cols, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i % cols;
  out[c * rows + r] = in[i];
}

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------
static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int skinny_splits(int64_t M, int64_t K) {
  const int64_t tiles = cdiv(M, 64);
  const int64_t chunks = cdiv(K, sk::KCH);
  int64_t want = cdiv(1024, tiles);
  if (want < 1) want = 1;
  if (want > chunks) want = chunks;
  if (want > 64) want = 64;
  return (int)want;
}

int64_t skinny_kc(int64_t K, int splits) {
  return cdiv(cdiv(K, splits), sk::KCH) * sk::KCH;
}

void launch_skinny_nt(const uint16_t* X, int64_t M, int64_t K, const uint16_t* Y, int R, float* part, int splits,
                      float* out, hipStream_t stream) {
  const int64_t kc = skinny_kc(K, splits);
  const int nsplit = (int)cdiv(K, kc);
  hipLaunchKernelGGL(skinny_nt_kernel, dim3((unsigned)cdiv(M, 64), (unsigned)nsplit), dim3(256), 0, stream, X, M, K,
                     Y, R, part, kc);
  const int64_t count = M * R;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, part, nsplit,
                     count, out);
}

int grad_splits(int64_t M, int64_t J) {
  const int64_t tiles = cdiv(J, 256);
  const int64_t chunks = cdiv(M, lg::TT);
  int64_t want = cdiv(768, tiles);
  if (want < 1) want = 1;
  if (want > chunks) want = chunks;
  if (want > 64) want = 64;
  return (int)want;
}

int64_t grad_tc(int64_t M, int splits) { return cdiv(cdiv(M, splits), lg::TT) * lg::TT; }

void launch_lora_grad(const uint16_t* X, int64_t M, int64_t J, const float* Y, int R, float s, int splits,
                      float* part, int transpose_out, uint16_t* out, hipStream_t stream) {
  const int64_t tc = grad_tc(M, splits);
  const int nsplit = (int)cdiv(M, tc);
  hipLaunchKernelGGL(lora_grad_kernel, dim3((unsigned)cdiv(J, 256), (unsigned)nsplit), dim3(256), 0, stream, X, M, J,
                     Y, R, part, tc);
  const int64_t count = J * R;
  hipLaunchKernelGGL(reduce_grad_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, part, nsplit, J, R,
                     s, transpose_out, out);
}

void launch_pad_cols_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t cols_pad, uint16_t* out,
                          hipStream_t stream) {
  const int64_t count = rows * cols_pad;
  hipLaunchKernelGGL(pad_cols_bf16_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, in, rows, cols,
                     cols_pad, out);
}

void launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out, hipStream_t stream) {
  const int64_t count = rows * cols;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)cdiv(count, 256)), dim3(256), 0, stream, in, rows, cols,
                     out);
}

}  // namespace qlora
