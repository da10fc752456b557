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
//   - a workgroup (4 waves) stages its x chunk (M x 2048 bf16, 64 or 128 KB)
//     in LDS once, with line-coalesced loads, and each wave takes a quarter
//     of the chunk (512 k) for all the item's feature blocks;
//   - a wave streams the codes as MFMA A fragments: per 16-feature block and
//     256-k piece every lane loads 32 contiguous bytes (8 code words, one
//     64-weight block, so one magnitude table per 64 weights), dequantizes a
//     word straight into the 8 bf16 of one 16x16x32 MFMA A operand, and reads
//     the matching x fragment from LDS;
//   - the four waves' partial sums are reduced through LDS in a fixed order
//     and written as fp32 partials per K chunk; the last feature group of a
//     chunk also writes that chunk's u = x_chunk A_chunk^T; a second launch
//     sums the chunks in order and adds s u B^T.
// Within a 256-k piece, MFMA step q takes from lane group g (lanes 16g ..
// 16g + 15) the k range 64g + 8q .. 64g + 8q + 7: the sum over k is the same,
// only grouped differently, and both operands use the same grouping.
#include "qlora_common.h"

namespace qlora {

namespace sm {
constexpr int KC = 2048;     // K per chunk
constexpr int PIECE = 256;   // k per piece (32 bytes of codes per lane)
constexpr int kPW = (KC / 4) / PIECE;   // pieces per wave and feature block (2)
constexpr int kDepth = 6;    // code pieces in flight per wave
constexpr int kMaxLayers = 8;
constexpr int kTargetWGs = 512;         // two workgroups per CU
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
  int64_t out_begin;        // first finishing workgroup of this layer
};

struct SmallArgs {
  SmallLayer L[sm::kMaxLayers];
  int count;
  int M;
};

__device__ __forceinline__ int find_layer(const SmallArgs& a, int64_t key, bool by_out) {
  int li = 0;
#pragma unroll
  for (int i = 1; i < sm::kMaxLayers; ++i)
    if (i < a.count && (by_out ? a.L[i].out_begin : (int64_t)a.L[i].wg_begin) <= key) li = i;
  return li;
}

// x chunk in LDS: token row t holds KC bf16; 16-byte chunk c of row t sits at
// chunk position c ^ (t & 15), so the 16 tokens of one MFMA B fragment hit
// 16 different bank groups.
__device__ __forceinline__ uint32_t xsw(int t, int c) {
  return (uint32_t)(t * (sm::KC * 2) + ((c ^ (t & 15)) << 4));
}

template <int TB>
__global__ __launch_bounds__(256) void small_fwd_kernel(SmallArgs a, Nf4Table tab) {
  constexpr int MP = 16 * TB;                 // padded token count
  constexpr int XB = MP * sm::KC * 2;         // 64 KB per token block
  constexpr int FBMAX = SmallTile<TB>::FBMAX;
  __shared__ __align__(16) uint8_t lds[XB];
  __shared__ __align__(16) f32x4 ured[4 * TB * 64];   // per-wave u partials of one rank block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int g = lane >> 4;

  const int li = find_layer(a, blockIdx.x, false);
  const SmallLayer& Ly = a.L[li];
  const int local = blockIdx.x - Ly.wg_begin;
  const int kc = local % Ly.nkc;
  const int fg = local / Ly.nkc;
  const int M = a.M;
  const int64_t K = Ly.n;
  const int64_t m = Ly.m;
  const int64_t k0 = (int64_t)kc * sm::KC;
  const int kq = wave * (sm::KC / 4);        // this wave's quarter within the chunk
  const int64_t f_base = (int64_t)fg * Ly.fbw * 16;
  const int64_t nfb = (m + 15) / 16;
  const int nb = (int)((nfb - (int64_t)fg * Ly.fbw) < Ly.fbw ? (nfb - (int64_t)fg * Ly.fbw) : Ly.fbw);

  // ---- stage x[0:MP][k0 : k0 + KC] (zeros past M or K) ----
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const brsrc_t rx = make_rsrc(Ly.x, xbytes);
  constexpr int XPT = MP * (sm::KC / 8) / 256;   // 16-byte chunks per thread
  u32x4 xr[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int id = i * 256 + tid;
    const int t = id / (sm::KC / 8);
    const int c = id % (sm::KC / 8);
    const int64_t k = k0 + 8 * c;
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
  // next row's codes, which meet the zero-padded x and add nothing.
  const uint32_t row_step = (uint32_t)(16 * K / 2);   // bytes of codes per feature block
  const uint32_t cbase_off = (uint32_t)(((f_base + lr) * K + k0 + kq + 64 * g) / 2);
  auto load_codes = [&](int b, int p, u32x4& c0, u32x4& c1, uint32_t& ab, float& cs) {
    const uint32_t off = b < nb ? cbase_off + (uint32_t)b * row_step + (uint32_t)p * (sm::PIECE / 2) : cbytes;
    c0 = bload128(rc, off);
    c1 = bload128(rc, off + 16);
    const uint32_t blk = off / (kBlock / 2);
    ab = bload8(rab, b < nb ? blk : abytes);
    cs = __uint_as_float(bload32(rc2, b < nb ? ((blk >> 8) << 2) : c2bytes));
  };

  // first pieces' codes in flight while x lands
  constexpr int NI = FBMAX * sm::kPW;   // (block, piece) iterations of a wave
  u32x4 cq0[sm::kDepth], cq1[sm::kDepth];
  uint32_t abq[sm::kDepth];
  float csq[sm::kDepth];
#pragma unroll
  for (int i = 0; i < sm::kDepth; ++i) load_codes(i / sm::kPW, i % sm::kPW, cq0[i], cq1[i], abq[i], csq[i]);

#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int id = i * 256 + tid;
    *reinterpret_cast<u32x4*>(lds + xsw(id / (sm::KC / 8), id % (sm::KC / 8))) = xr[i];
  }
  __syncthreads();

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
    const int cbase = (kq + sm::PIECE * p + 64 * g) / 8;   // 16-byte chunk of k for step 0
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t o[4];
      mag_dequant8(L, (q < 4 ? c0 : c1)[q & 3], o);
      const u32x4 af = u32x4{o[0], o[1], o[2], o[3]};
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(lds + xsw(16 * tb + lr, cbase + q));
        acc[b][tb] = mfma16x16x32(af, bf, acc[b][tb]);
      }
    }
  }

  // ---- the last feature group of each chunk (usually the one with fewest
  // blocks) forms u_chunk = x_chunk A_chunk^T, each wave over its quarter,
  // one rank block of 16 at a time ----
  if (fg == Ly.ngroups - 1) {
    const int r = Ly.r;
    const int RBn = (r + 15) >> 4;
    const uint32_t arbytes = (uint32_t)((int64_t)r * K * 2);
    const brsrc_t ra = make_rsrc(Ly.A, arbytes);
    float* up = Ly.upart + (int64_t)kc * M * r;
    constexpr int NJ = (sm::KC / 4) / 32;   // 16 MFMA steps over the wave's quarter
    for (int rb = 0; rb < RBn; ++rb) {
      const int q = 16 * rb + lr;
      u32x4 af[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t k = k0 + kq + 32 * j + 8 * g;
        const bool ok = q < r && k < K;
        af[j] = bload128(ra, ok ? (uint32_t)(((int64_t)q * K + k) * 2) : arbytes);
      }
      f32x4 ua[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) ua[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int kl = kq + 32 * j + 8 * g;   // k within the chunk
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const u32x4 bf = *reinterpret_cast<const u32x4*>(lds + xsw(16 * tb + lr, kl / 8));
          ua[tb] = mfma16x16x32(af[j], bf, ua[tb]);
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

  // ---- reduce the four waves' partial sums through LDS (x is no longer needed) ----
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);   // [wave][b][tb][lane]
#pragma unroll
  for (int b = 0; b < FBMAX; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
      if (b < nb) red[((wave * FBMAX + b) * TB + tb) * 64 + lane] = acc[b][tb];
  __syncthreads();
  float* hp = Ly.hpart + (int64_t)kc * M * m;
  for (int idx = tid; idx < nb * TB * 64; idx += 256) {
    const int ln = idx & 63;
    const int tb = (idx >> 6) % TB;
    const int b = (idx >> 6) / TB;
    f32x4 v = red[((0 * FBMAX + b) * TB + tb) * 64 + ln];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[((w * FBMAX + b) * TB + tb) * 64 + ln];
    // C layout: lane ln holds token 16 tb + ln % 16, features 4 (ln / 16) + e of block b
    const int t = 16 * tb + (ln & 15);
    const int64_t f = f_base + 16 * b + 4 * (ln >> 4);
    if (t < M) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (f + e < m) hp[(int64_t)t * m + f + e] = v[e];
    }
  }
}

// h[t][f] = bf16(sum_c hpart[c][t][f] + s * sum_q u[t][q] B[f][q]) with
// u[t][q] = sum_c upart[c][t][q] (chunk order).  One workgroup finishes 128
// features of one layer for every token: the B rows of those features and u
// are staged in LDS; thread (token t, segment j) forms features
// 8j .. 8j + 7 for tokens t and t + 16.  The layer's first workgroup also
// writes u_out.
__global__ __launch_bounds__(256) void small_reduce_kernel(SmallArgs a) {
  __shared__ float su[32 * kMaxRank];
  __shared__ __align__(16) uint16_t sb[128 * kMaxRank];
  const int li = find_layer(a, blockIdx.x, true);
  const SmallLayer& Ly = a.L[li];
  const int tile = (int)(blockIdx.x - Ly.out_begin);
  const int M = a.M;
  const int64_t m = Ly.m;
  const int r = Ly.r;
  const int nkc = Ly.nkc;
  const int tid = threadIdx.x;
  const int64_t fbase = (int64_t)tile * 128;
  const int nf_tile = (int)((m - fbase) < 128 ? (m - fbase) : 128);
  // chunk partials are loaded 8 at a time before they are summed (in chunk
  // order), so the loads of one thread overlap instead of forming a chain
  for (int idx = tid; idx < M * r; idx += 256) {
    float uq = 0.0f;
    for (int c0 = 0; c0 < nkc; c0 += 8) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = (c0 + c < nkc) ? Ly.upart[(int64_t)(c0 + c) * M * r + idx] : 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c0 + c < nkc) uq += v[c];
    }
    su[idx] = uq;
    if (Ly.u_out && tile == 0) Ly.u_out[idx] = uq;
  }
  {
    // B rows fbase .. fbase + nf_tile - 1 are one contiguous run of bf16
    const uint16_t* src = Ly.B + fbase * r;
    const int cnt = nf_tile * r;
    if ((cnt & 7) == 0) {
      for (int i = tid; i < cnt / 8; i += 256)
        reinterpret_cast<u32x4*>(sb)[i] = reinterpret_cast<const u32x4*>(src)[i];
    } else {
      for (int i = tid; i < cnt; i += 256) sb[i] = src[i];
    }
  }
  __syncthreads();
  const int j = tid & 15;
  const int nf = nf_tile - 8 * j;   // features of this thread (<= 0: none)
  if (nf <= 0) return;
  const int64_t f0 = fbase + 8 * j;
  const bool vec = (m & 7) == 0;
  for (int t = tid >> 4; t < M; t += 16) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    if (vec) {
      for (int c0 = 0; c0 < nkc; c0 += 4) {
        f32x4 v[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4* hp = reinterpret_cast<const f32x4*>(Ly.hpart + ((int64_t)(c0 + c) * M + t) * m + f0);
          v[c][0] = (c0 + c < nkc) ? hp[0] : f32x4{0.f, 0.f, 0.f, 0.f};
          v[c][1] = (c0 + c < nkc) ? hp[1] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c0 + c < nkc) {
#pragma unroll
            for (int e = 0; e < 4; ++e) { acc[e] += v[c][0][e]; acc[4 + e] += v[c][1][e]; }
          }
        }
      }
    } else {
      for (int c = 0; c < nkc; ++c) {
        const float* hp = Ly.hpart + ((int64_t)c * M + t) * m + f0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < nf) acc[e] += hp[e];
      }
    }
    uint32_t outw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float lo0 = 0.0f, lo1 = 0.0f;
      const uint16_t* b0 = sb + (8 * j + e) * r;
      const uint16_t* b1 = b0 + r;
      for (int q = 0; q < r; ++q) {
        const float uq = su[t * r + q];
        lo0 += uq * bf16_lo_to_f32((uint32_t)b0[q]);
        lo1 += uq * bf16_lo_to_f32((uint32_t)b1[q]);
      }
      outw[e / 2] = pack_bf16x2(acc[e] + Ly.s * lo0, acc[e + 1] + Ly.s * lo1);
    }
    uint16_t* dst = Ly.h + (int64_t)t * m + f0;
    if (vec) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{outw[0], outw[1], outw[2], outw[3]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e < nf) dst[e] = (uint16_t)((outw[e / 2] >> (16 * (e & 1))) & 0xFFFFu);
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

// fp32 partial workspace of one layer: [nkc][M][m] + [nkc][M][r]
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
};

void launch_small_fwd(int M, const SmallLayerHost* layers, int count, const Nf4Table& tab, hipStream_t stream) {
  SmallArgs a{};
  a.count = count;
  a.M = M;
  const int fbmax = M <= 16 ? SmallTile<1>::FBMAX : SmallTile<2>::FBMAX;
  // feature blocks per workgroup: the fewest that keep the launch within two
  // workgroups per CU (a launch a few workgroups over that would run a second,
  // almost empty round), the same width for every layer
  auto wgs_for = [&](int fbw) {
    int64_t w = 0;
    for (int i = 0; i < count; ++i) w += small_nkc(layers[i].n) * cdiv_s(cdiv_s(layers[i].m, 16), fbw);
    return w;
  };
  int fbw = 1;
  while (fbw < fbmax && wgs_for(fbw) > sm::kTargetWGs) ++fbw;
  int wg = 0;
  int64_t outs = 0;
  for (int i = 0; i < count; ++i) {
    const SmallLayerHost& h = layers[i];
    SmallLayer& L = a.L[i];
    L.x = h.x; L.codes = h.codes; L.absmax8 = h.absmax8; L.c2 = h.c2; L.A = h.A; L.B = h.B; L.h = h.h;
    L.u_out = h.u_out; L.n = h.n; L.m = h.m; L.r = h.r; L.s = h.s;
    L.nkc = (int)small_nkc(h.n);
    L.fbw = fbw;
    L.ngroups = (int)cdiv_s(cdiv_s(h.m, 16), fbw);
    const size_t hb = (size_t)L.nkc * M * h.m * sizeof(float);
    L.hpart = reinterpret_cast<float*>(h.ws);
    L.upart = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(h.ws) + ((hb + 255) & ~(size_t)255));
    L.wg_begin = wg;
    L.out_begin = outs;
    wg += L.nkc * L.ngroups;
    outs += cdiv_s(h.m, 128);
  }
  if (M <= 16)
    hipLaunchKernelGGL(small_fwd_kernel<1>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  else
    hipLaunchKernelGGL(small_fwd_kernel<2>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  hipLaunchKernelGGL(small_reduce_kernel, dim3((unsigned)outs), dim3(256), 0, stream, a);
}

}  // namespace qlora
