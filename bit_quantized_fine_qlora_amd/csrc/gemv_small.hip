// Forward of the adapted linear layer for small token counts (M <= 32):
//   h = x W'^T + s u B^T,  u = x A^T
// "QLoRA: Efficient Fine-Tuning", Step 3 (Eq. 3), with W' = dequant(W0) as
// in the dequantization passage of Step 3 and "How QLoRA Works" (BF16
// compute type).  With a few tokens every packed weight is used by at most
// 32 tokens, so the pass is bound by streaming the 4-bit codes from HBM.
//
// Design (one or several layers per launch, all sharing the token count M):
//   - the (out-feature x K) plane of each layer is cut into work items of
//     8 blocks of 16 features x one K chunk of 2048;
//   - a workgroup (4 waves) stages its x chunk (M x 2048 bf16, 64 or 128 KB)
//     in LDS once, with line-coalesced loads, and each wave takes a quarter
//     of the chunk (512 k) for all 8 feature blocks;
//   - a wave streams the codes as MFMA A fragments: per 16-feature block and
//     256-k piece every lane loads 32 contiguous bytes (8 code words, one
//     64-weight block, so one magnitude table per 64 weights), dequantizes a
//     word straight into the 8 bf16 of one 16x16x32 MFMA A operand, and reads
//     the matching x fragment from LDS;
//   - the four waves' partial sums are reduced through LDS in a fixed order
//     and written as fp32 partials per K chunk; the first feature groups of a
//     chunk also write per-wave partials of u = x_chunk A_chunk^T (one 256-k
//     slice each); a second launch sums the partials in order and adds
//     s u B^T.
// Within a 256-k piece, MFMA step q takes from lane group g (lanes 16g ..
// 16g + 15) the k range 64g + 8q .. 64g + 8q + 7: the sum over k is the same,
// only grouped differently, and both operands use the same grouping.
#include "qlora_common.h"

namespace qlora {

namespace sm {
constexpr int KC = 2048;     // K per chunk (work item)
constexpr int FBW = 8;       // 16-feature blocks per work item
constexpr int PIECE = 256;   // k per piece (32 bytes of codes per lane)
constexpr int kMaxLayers = 8;
}  // namespace sm

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
  float* upart;             // [nkc][8 slices][4 waves][M][r]
  int64_t n, m;
  int r;
  float s;
  int nkc;                  // K chunks
  int ngroups;              // feature groups (8 blocks of 16 features)
  int wg_begin;             // first workgroup of this layer in the launch
  int64_t out_begin;        // first reduce thread of this layer
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
  __shared__ __align__(16) uint8_t lds[XB];
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
  const int64_t f_base = (int64_t)fg * sm::FBW * 16;

  // ---- stage x[0:MP][k0 : k0 + KC] (zeros past M or K) ----
  const uint32_t xbytes = (uint32_t)((int64_t)M * K * 2);
  const brsrc_t rx = make_rsrc(Ly.x, xbytes);
  constexpr int XCH = MP * (sm::KC / 8);      // 16-byte chunks
  constexpr int XPT = XCH / 256;              // per thread
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

  // ---- codes of this wave: row f, byte offset of piece p ----
  const uint32_t cbytes = (uint32_t)(m * K / 2);
  const uint32_t abytes = (uint32_t)(m * K / kBlock);
  const uint32_t c2bytes = (uint32_t)(((m * K / kBlock + kGroupBlocks - 1) / kGroupBlocks) * 4);
  const brsrc_t rc = make_rsrc(Ly.codes, cbytes);
  const brsrc_t rab = make_rsrc(Ly.absmax8, abytes);
  const brsrc_t rc2 = make_rsrc(Ly.c2, c2bytes);
  constexpr int kPW = (sm::KC / 4) / sm::PIECE;   // pieces per wave (2)
  constexpr int kDepth = 4;                       // code loads in flight, in pieces
  // lane's 64-weight block for (feature block b, piece p): row f = f_base + 16 b + lr,
  // k = k0 + kq + 256 p + 64 g
  auto elem = [&](int b, int p) -> int64_t {
    return (f_base + 16 * b + lr) * K + k0 + kq + (int64_t)sm::PIECE * p + 64 * g;
  };
  auto load_codes = [&](int b, int p, u32x4& c0, u32x4& c1, uint32_t& ab, float& cs) {
    const int64_t e = elem(b, p);
    const bool ok = (f_base + 16 * b + lr) < m && (k0 + kq + (int64_t)sm::PIECE * p + 64 * g) < K;
    c0 = bload128(rc, ok ? (uint32_t)(e / 2) : cbytes);
    c1 = bload128(rc, ok ? (uint32_t)(e / 2) + 16 : cbytes);
    const int64_t blk = e / kBlock;
    ab = bload8(rab, ok ? (uint32_t)blk : abytes);
    cs = __uint_as_float(bload32(rc2, ok ? (uint32_t)((blk >> 8) << 2) : c2bytes));
  };

  // ---- u partials (first feature groups of each chunk): slice sl (256 k of
  // the chunk) of u = x A^T, wave w taking k 64w .. 64w + 63 of the slice;
  // each wave writes its own partial ----
  const int r = Ly.r;
  const int RBn = (r + 15) >> 4;

  // first pieces' codes in flight while x lands
  constexpr int NI = sm::FBW * kPW;   // (block, piece) iterations of a wave
  u32x4 cq0[kDepth], cq1[kDepth];
  uint32_t abq[kDepth];
  float csq[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_codes(i / kPW, i % kPW, cq0[i], cq1[i], abq[i], csq[i]);

#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int id = i * 256 + tid;
    *reinterpret_cast<u32x4*>(lds + xsw(id / (sm::KC / 8), id % (sm::KC / 8))) = xr[i];
  }
  __syncthreads();

  if (fg < sm::KC / sm::PIECE) {
    const uint32_t arbytes = (uint32_t)((int64_t)r * K * 2);
    const brsrc_t ra = make_rsrc(Ly.A, arbytes);
    for (int sl = fg; sl < sm::KC / sm::PIECE; sl += Ly.ngroups) {
      float* up = Ly.upart + (((int64_t)kc * (sm::KC / sm::PIECE) + sl) * 4 + wave) * M * r;
      for (int rb = 0; rb < RBn; ++rb) {
        f32x4 ua[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) ua[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kl = sm::PIECE * sl + 64 * wave + 32 * j + 8 * g;   // k within the chunk
          const int64_t k = k0 + kl;
          const int q = 16 * rb + lr;
          const bool ok = q < r && k < K;
          const u32x4 af = bload128(ra, ok ? (uint32_t)(((int64_t)q * K + k) * 2) : arbytes);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            const u32x4 bf = *reinterpret_cast<const u32x4*>(lds + xsw(16 * tb + lr, kl / 8));
            ua[tb] = mfma16x16x32(af, bf, ua[tb]);
          }
        }
        // rows are adapter rows q = 16 rb + 4 (lane / 16) + e, column token 16 tb + lane % 16
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int t = 16 * tb + lr;
          if (t < M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q = 16 * rb + 4 * g + e;
              if (q < r) up[(int64_t)t * r + q] = ua[tb][e];
            }
          }
        }
      }
    }
  }

  // ---- main loop over (feature block, piece), codes kDepth iterations ahead ----
  f32x4 acc[sm::FBW][TB];
#pragma unroll
  for (int b = 0; b < sm::FBW; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[b][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int b = i / kPW, p = i % kPW, slot = i % kDepth;
    const u32x4 c0 = cq0[slot], c1 = cq1[slot];
    const MagLut L = make_mag_lut(tab, e4m3_decode(abq[slot]) * csq[slot]);
    if (i + kDepth < NI) load_codes((i + kDepth) / kPW, (i + kDepth) % kPW, cq0[slot], cq1[slot], abq[slot], csq[slot]);
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

  // ---- reduce the four waves' partial sums through LDS (x is no longer needed) ----
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);   // [wave][b][tb][lane]
#pragma unroll
  for (int b = 0; b < sm::FBW; ++b)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) red[((wave * sm::FBW + b) * TB + tb) * 64 + lane] = acc[b][tb];
  __syncthreads();
  float* hp = Ly.hpart + (int64_t)kc * M * m;
  for (int idx = tid; idx < sm::FBW * TB * 64; idx += 256) {
    const int ln = idx & 63;
    const int tb = (idx >> 6) % TB;
    const int b = (idx >> 6) / TB;
    f32x4 v = red[((0 * sm::FBW + b) * TB + tb) * 64 + ln];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[((w * sm::FBW + b) * TB + tb) * 64 + ln];
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
// u[t][q] = sum over chunks and slices of upart (fixed order), formed once per
// workgroup in LDS; the layer's first workgroup also writes u_out.  Each
// layer's outputs start on a workgroup boundary.
__global__ __launch_bounds__(256) void small_reduce_kernel(SmallArgs a) {
  __shared__ float su[32 * kMaxRank];
  const int64_t gid0 = (int64_t)blockIdx.x * 256;
  const int li = find_layer(a, gid0, true);
  const SmallLayer& Ly = a.L[li];
  const int M = a.M;
  const int64_t m = Ly.m;
  const int r = Ly.r;
  const int nparts = Ly.nkc * (sm::KC / sm::PIECE) * 4;   // chunks x slices x waves
  for (int idx = threadIdx.x; idx < M * r; idx += 256) {
    float uq = 0.0f;
    for (int c = 0; c < nparts; ++c) uq += Ly.upart[(int64_t)c * M * r + idx];
    su[idx] = uq;
    if (Ly.u_out && gid0 == Ly.out_begin) Ly.u_out[idx] = uq;
  }
  __syncthreads();
  const int64_t i = gid0 + threadIdx.x - Ly.out_begin;
  if (i >= (int64_t)M * m) return;
  const int t = (int)(i / m);
  const int64_t f = i % m;
  float acc = 0.0f;
  for (int c = 0; c < Ly.nkc; ++c) acc += Ly.hpart[((int64_t)c * M + t) * m + f];
  float lora = 0.0f;
  for (int q = 0; q < r; ++q) lora += su[t * r + q] * bf16_lo_to_f32((uint32_t)Ly.B[f * r + q]);
  Ly.h[i] = (uint16_t)(pack_bf16x2(acc + Ly.s * lora, 0.f) & 0xFFFFu);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int small_max_tokens() { return 32; }
int small_max_layers() { return sm::kMaxLayers; }

static inline int64_t cdiv_s(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t small_nkc(int64_t n) { return cdiv_s(n, sm::KC); }

// fp32 partial workspace of one layer: [nkc][M][m] + [nkc][8 slices][4 waves][M][r]
size_t small_ws_bytes(int64_t M, int64_t n, int64_t m, int r) {
  const int64_t nkc = small_nkc(n);
  const size_t hb = (size_t)nkc * M * m * sizeof(float);
  const size_t ub = (size_t)nkc * (sm::KC / sm::PIECE) * 4 * M * r * sizeof(float);
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
  int wg = 0;
  int64_t outs = 0;
  for (int i = 0; i < count; ++i) {
    const SmallLayerHost& h = layers[i];
    SmallLayer& L = a.L[i];
    L.x = h.x; L.codes = h.codes; L.absmax8 = h.absmax8; L.c2 = h.c2; L.A = h.A; L.B = h.B; L.h = h.h;
    L.u_out = h.u_out; L.n = h.n; L.m = h.m; L.r = h.r; L.s = h.s;
    L.nkc = (int)small_nkc(h.n);
    L.ngroups = (int)cdiv_s(cdiv_s(h.m, 16), sm::FBW);
    const size_t hb = (size_t)L.nkc * M * h.m * sizeof(float);
    L.hpart = reinterpret_cast<float*>(h.ws);
    L.upart = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(h.ws) + ((hb + 255) & ~(size_t)255));
    L.wg_begin = wg;
    L.out_begin = outs;
    wg += L.nkc * L.ngroups;
    outs += cdiv_s((int64_t)M * h.m, 256) * 256;
  }
  if (M <= 16)
    hipLaunchKernelGGL(small_fwd_kernel<1>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  else
    hipLaunchKernelGGL(small_fwd_kernel<2>, dim3((unsigned)wg), dim3(256), 0, stream, a, tab);
  hipLaunchKernelGGL(small_reduce_kernel, dim3((unsigned)(outs / 256)), dim3(256), 0, stream, a);
}

}  // namespace qlora
