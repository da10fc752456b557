// C ABI of the QLoRA adapted-linear library: argument checks, workspace
// layout, kernel dispatch and optional kernel timing.  Declared in qlora.h.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlora.h"
#include "qlora_common.h"

// Scratch of qlora_linear_fwd_static, one copy per device (see static_scratch
// below): 64 MiB, enough for the forward's split partials, u and the GEMM's
// K-split sums at every shape whose workspace fits; larger layouts drop the
// K split or are refused.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
static_assert(kStaticScratchBytes == QLORA_STATIC_SCRATCH_BYTES, "scratch size differs from the header");

namespace qlora {

// kernels (defined in the other translation units)
void launch_quantize(const float* W, int64_t numel, uint8_t* codes, uint8_t* absmax8, float* c2,
                     const Nf4Table& tab, hipStream_t stream);
struct QuantWeight {
  const float* W;
  int64_t numel;
  uint8_t* codes;
  uint8_t* absmax8;
  float* c2;
};
int max_quant_weights();
int64_t quant_groups(int64_t numel);
void launch_quantize_grouped(const QuantWeight* w, int count, const Nf4Table& tab, hipStream_t stream);
void launch_dequant(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t numel, uint16_t* out,
                    const Nf4Table& tab, hipStream_t stream);
void launch_fwd_gemm(const uint16_t* x, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                     const uint16_t* B, const float* u, uint16_t* h, int64_t M, int64_t n, int64_t m, int r,
                     float s, void* split_ws, const Nf4Table& tab, hipStream_t stream, bool sync_zeroed = false);
size_t gemm_split_ws_bytes(int64_t M, int64_t N, int64_t K);
SyncZero gemm_split_sync(int64_t M, int64_t N, int64_t K, void* split_ws);
int64_t gemm_giveup_offset(int64_t M, int64_t N, int64_t K);
void launch_dgrad_gemm(const uint16_t* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                       const uint16_t* A, const float* v, uint16_t* gx, int64_t M, int64_t n, int64_t m,
                       int64_t m_pad, int r, float s, void* split_ws, const Nf4Table& tab, hipStream_t stream,
                       const float* add, bool sync_zeroed = false);
int small_max_tokens();
int small_max_layers();
size_t small_ws_bytes(int64_t M, int64_t n, int64_t m, int r);
struct SmallLayerHost {
  const uint16_t* x; const uint8_t* codes; const uint8_t* absmax8; const float* c2;
  const uint16_t* A; const uint16_t* B; uint16_t* h; float* u_out;
  int64_t n, m; int r; float s;
  void* ws;
  DropoutDev drop{};
  float u_scale = 1.0f;
};
void launch_small_fwd(int M, const SmallLayerHost* layers, int count, const Nf4Table& tab, hipStream_t stream);
int down_proj_splits(int64_t M, int64_t K, int R);
void launch_down_proj(const uint16_t* X, int64_t M, int64_t K, const uint16_t* Y, int R, float* part, int splits,
                      float* out, hipStream_t stream, const DropoutDev* drop, float scale,
                      SyncZero z = SyncZero{});
int token_grad_splits(int64_t M, int64_t J, int R);
void launch_token_grad(const uint16_t* X, int64_t M, int64_t J, const float* Y, int R, int splits, float* part,
                       hipStream_t stream, const DropoutDev* drop, uint16_t* planes, bool planes_ready);
size_t token_planes_bytes(int64_t M, int R);
void launch_factor_planes(const float* Y, int nsplit, int64_t M, int R, uint16_t* P, float* Yout, const float* Y2,
                          uint16_t* P2, hipStream_t stream);
void launch_lora_dropout_term(const float* v, const uint16_t* A, int64_t M, int64_t n, int R, float scale,
                              const DropoutDev& drop, float* out, hipStream_t stream);
bool down_proj_bt_supported(int R);
void launch_down_proj_bt(const uint16_t* G, int64_t M, int64_t K, const uint16_t* B, int64_t m, int R, float* part,
                         int splits, hipStream_t stream);
void launch_reduce_grads(const float* bpart, int nb_split, int64_t Jb, int64_t mb, float s_b, uint16_t* grad_B,
                         const float* apart, int na_split, int64_t Ja, int64_t na, float s_a, uint16_t* grad_A, int R,
                         hipStream_t stream,
                         SyncZero z = SyncZero{});
void launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld, uint16_t* out,
                           hipStream_t stream);
void launch_pad_cols_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t cols_pad, uint16_t* out,
                          hipStream_t stream);
void launch_merge_adapter(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m, int64_t n, int r,
                          float s, const uint16_t* A, const uint16_t* B, uint16_t* out, const Nf4Table& tab,
                          hipStream_t stream);
struct AdamTensorHost {
  int64_t count;
  float* p;
  uint16_t* p16;
  const uint16_t* g;
  float* m;
  float* v;
};
void launch_adam_step(const AdamTensorHost* ts, int count, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int64_t step, hipStream_t stream);
bool gpass_supported(int R);
int gpass_splits_f(int64_t M, int64_t J, int R);
int gpass_splits_t(int64_t M);
void launch_gpass(const uint16_t* G, int64_t M, int64_t J, const uint16_t* B, int64_t m, const float* U, int R,
                  float* vpart, float* gbpart, hipStream_t stream);

namespace {

// ---------------------------------------------------------------------------
// NF4 table: Phi^-1 by bisection on Phi(x) = erfc(-x/sqrt2)/2 in double,
// polished by Newton steps, then normalized by the largest level.
// ---------------------------------------------------------------------------
double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int it = 0; it < 3; ++it) {
    const double pdf = std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
    x -= (normal_cdf(x) - p) / pdf;
  }
  return x;
}

// 16 levels, symmetric (Q[15 - j] = -Q[j]), and the fp32 midpoints.
//   qtype 0 (NF4): q_i = Phi^-1((i - 1/2)/16) / q_16
//   qtype 1 (uniform 4-bit comparison grid): (2j - 15)/15, no zero level
//   qtype 2 (edge-mean table, "QLoRA & 4-bit Fine-Tuning" Innovation 1):
//     level i is the mean of Phi^-1 at its bucket's edges i/16 and
//     (i + 1)/16, with the two outermost edges (infinite quantiles) moved to
//     the outer buckets' midpoints 1/32 and 31/32; normalized by the largest
//   qtype 3 (INT4 absmax, "QLoRA: Efficient Fine-Tuning" Step 1): k/7 for
//     k = -7..7, the zero level held twice, as -0 (index 7) and +0 (index 8)
Nf4Table build_table(int qtype) {
  Nf4Table t;
  double q[16];
  if (qtype == 0) {
    for (int i = 1; i <= 16; ++i) q[i - 1] = normal_quantile((i - 0.5) / 16.0);
    for (int j = 0; j < 16; ++j) t.q[j] = (float)(q[j] / q[15]);
  } else if (qtype == 2) {
    double qe[17];
    for (int i = 0; i <= 16; ++i) {
      const double e = i == 0 ? 0.5 / 16.0 : (i == 16 ? 1.0 - 0.5 / 16.0 : i / 16.0);
      qe[i] = normal_quantile(e);
    }
    for (int j = 0; j < 16; ++j) q[j] = 0.5 * (qe[j] + qe[j + 1]);
    for (int j = 0; j < 16; ++j) t.q[j] = (float)(q[j] / q[15]);
  } else if (qtype == 3) {
    for (int k = 0; k < 8; ++k) t.q[8 + k] = (float)(k / 7.0);
  } else {
    for (int j = 0; j < 16; ++j) t.q[j] = (float)((2.0 * j - 15.0) / 15.0);
  }
  // exact symmetry of the construction, kept exact after rounding (for the
  // INT4 grid this writes -0 at index 7)
  for (int j = 0; j < 8; ++j) t.q[j] = -t.q[15 - j];
  for (int j = 0; j < 15; ++j) t.t[j] = (float)(((double)t.q[j] + (double)t.q[j + 1]) * 0.5);
  // The quantizer finds the code of |w/c1| through a table of eighth-binade
  // intervals of [0, 1] that may hold at most one positive threshold each;
  // checked here once (with every threshold at or above 2^-4, which all the
  // tables here satisfy).
  uint32_t prev = 0;
  for (int j = 8; j < 15; ++j) {
    uint32_t b;
    std::memcpy(&b, &t.t[j], 4);
    if (b < 0x3D800000u || (j > 8 && (b >> 20) == (prev >> 20))) {
      std::fprintf(stderr, "qlora: threshold layout breaks the quantizer's interval table\n");
      std::abort();
    }
    prev = b;
  }
  return t;
}

const Nf4Table& table(int qtype = 0) {
  static const Nf4Table u = build_table(1);
  if (qtype == 1) return u;
  static const Nf4Table e = build_table(2);
  if (qtype == 2) return e;
  static const Nf4Table i4 = build_table(3);
  if (qtype == 3) return i4;
  static const Nf4Table t = build_table(0);
  return t;
}

bool valid_qtype(int32_t qtype) {
  return qtype == QLORA_QTYPE_NF4 || qtype == QLORA_QTYPE_UNIFORM4 || qtype == QLORA_QTYPE_EDGE_MEAN4 ||
         qtype == QLORA_QTYPE_INT4;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
struct Rec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<Rec> g_recs;
// Set while qlora_linear_fwd_static runs on this thread: it records no
// events (creating them and growing the record list would allocate).
thread_local bool t_prof_suppressed = false;

struct Timed {
  hipStream_t s;
  const char* name;
  hipEvent_t a = nullptr, b = nullptr;
  bool on;
  Timed(const char* nm, hipStream_t st) : s(st), name(nm) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on && !t_prof_suppressed;
    // a launch whose events cannot be made or recorded is left untimed
    if (on && (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess ||
               hipEventRecord(a, s) != hipSuccess)) {
      drop();
      on = false;
    }
  }
  ~Timed() {
    if (!on) return;
    if (hipEventRecord(b, s) != hipSuccess) {
      drop();
      return;
    }
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_recs.push_back(Rec{name, a, b});
  }
  void drop() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    a = b = nullptr;
  }
};

// ---------------------------------------------------------------------------
// checks
// ---------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;

qlora_status check_weight_shape(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0 || (n % kBlock) != 0) return QLORA_ERR_SHAPE;
  if (m >= kMaxDim || n >= kMaxDim) return QLORA_ERR_SHAPE;
  if (m > ((int64_t)1 << 40) / n) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

qlora_status check_linear(int64_t M, int64_t n, int64_t m, int32_t r, float s) {
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (M <= 0 || M >= kMaxDim) return QLORA_ERR_SHAPE;
  // the GEMM kernels address activations and the packed weight with 32-bit
  // byte offsets: M*max(n,m) < 2^30 and m*n < 2^31
  if (M >= ((int64_t)1 << 30) / (n > m ? n : m)) return QLORA_ERR_SHAPE;
  if (m >= ((int64_t)1 << 31) / n) return QLORA_ERR_SHAPE;
  if (r < 1 || r > kMaxRank) return QLORA_ERR_RANK;
  if (!std::isfinite(s)) return QLORA_ERR_VALUE;
  return QLORA_OK;
}

qlora_status hip_status() {
  return hipGetLastError() == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct WsLayout {
  size_t total = 0;
  size_t take(size_t bytes) {
    const size_t off = total;
    total += align256(bytes);
    return off;
  }
};

struct FwdWs {
  size_t part, u, ksplit, total;
  int splits;
  bool has_ksplit;
};

FwdWs fwd_ws(int64_t M, int64_t n, int64_t m, int32_t r) {
  WsLayout L;
  FwdWs w;
  if (M <= small_max_tokens()) {  // weight-streaming path: fp32 partials only
    w.splits = 0;
    w.part = w.u = w.ksplit = 0;
    w.has_ksplit = false;
    L.take(small_ws_bytes(M, n, m, r));
    w.total = L.total;
    return w;
  }
  w.splits = down_proj_splits(M, n, r);
  w.part = L.take((size_t)w.splits * M * r * sizeof(float));
  w.u = L.take((size_t)M * r * sizeof(float));
  const size_t kb = gemm_split_ws_bytes(M, m, n);  // GEMM tiles split in K
  w.has_ksplit = kb != 0;
  w.ksplit = w.has_ksplit ? L.take(kb) : 0;
  w.total = L.total;
  return w;
}

struct BwdWs {
  size_t Bt, part_uv, u, v, gA, gB, gpad, vpart, gbpart, dterm, planes, uplanes, ksplit, total;
  int su, sv, sa, sb;
  bool gpass;     // v and grad_B from one read of g
  bool has_ksplit;
  int64_t m_pad;  // row length of g as the kernels read it
};

BwdWs bwd_ws(int64_t M, int64_t n, int64_t m, int32_t r, bool dropout = false) {
  WsLayout L;
  BwdWs w;
  // The kernels read g in 16-byte pieces; rows whose length is not a
  // multiple of 8 are first copied into a zero-padded buffer of row length m
  // rounded up to 64 (the padded columns contribute nothing).
  w.m_pad = (m % 8 == 0) ? m : ((m + 63) / 64) * 64;
  w.gpad = (m % 8 == 0) ? 0 : L.take((size_t)M * w.m_pad * 2);
  w.su = down_proj_splits(M, n, r);
  w.sv = down_proj_splits(M, w.m_pad, r);
  w.sa = token_grad_splits(M, n, r);
  w.sb = token_grad_splits(M, w.m_pad, r);
  w.gpass = gpass_supported(r);
  // B^T for v = g B, except where the stream reads B itself
  w.Bt = (w.gpass || down_proj_bt_supported(r)) ? 0 : L.take((size_t)w.m_pad * r * 2);
  const int suv = w.gpass ? w.su : (w.su > w.sv ? w.su : w.sv);
  w.part_uv = L.take((size_t)suv * M * r * sizeof(float));
  w.u = L.take((size_t)M * r * sizeof(float));
  w.v = L.take((size_t)M * r * sizeof(float));
  w.gA = L.take((size_t)w.sa * n * r * sizeof(float));
  w.gB = w.gpass ? 0 : L.take((size_t)w.sb * w.m_pad * r * sizeof(float));
  w.vpart = w.gpass ? L.take((size_t)gpass_splits_f(M, w.m_pad, r) * M * r * sizeof(float)) : 0;
  w.gbpart = w.gpass ? L.take((size_t)gpass_splits_t(M) * w.m_pad * r * sizeof(float)) : 0;
  // dropout: the masked adapter part of grad_x in fp32
  w.dterm = dropout ? L.take((size_t)M * n * sizeof(float)) : 0;
  // bf16 hi / lo planes of v (grad_A) and, without the g pass, of u (grad_B)
  w.planes = L.take(token_planes_bytes(M, r));
  w.uplanes = w.gpass ? 0 : L.take(token_planes_bytes(M, r));
  // grad_x GEMM tiles split in K (few tiles, or a short last round)
  const size_t kb = gemm_split_ws_bytes(M, n, w.m_pad);
  w.ksplit = kb ? L.take(kb) : 0;
  w.has_ksplit = kb != 0;
  w.total = L.total;
  return w;
}

// Device form of a dropout request; inv_keep = 1 / (1 - p).  NULL or p = 0
// leaves the mask off.
qlora_status make_dropout(const qlora_dropout* d, DropoutDev& out, float& inv_keep) {
  out = DropoutDev{0u, 0u, 0u, 0ull, 0};
  inv_keep = 1.0f;
  if (!d) return QLORA_OK;
  if (!std::isfinite(d->p) || d->p < 0.0f || d->p >= 1.0f) return QLORA_ERR_VALUE;
  if (d->p == 0.0f) return QLORA_OK;
  const double t = std::nearbyint((double)d->p * 4294967296.0);  // ties to even
  out.thr = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  out.k0 = (uint32_t)(d->seed & 0xFFFFFFFFull);
  out.k1 = (uint32_t)(d->seed >> 32);
  out.offset = d->offset;
  out.on = 1;
  inv_keep = (float)(1.0 / (1.0 - (double)d->p));
  return QLORA_OK;
}

// ---------------------------------------------------------------------------
// Library-owned scratch of qlora_linear_fwd_static (callers that cannot
// allocate device memory).  Each device the library runs on holds its own
// copy of this array until the process ends.  In host code `scratch` only
// names the array: its device address comes from hipGetSymbolAddress, once
// per device (with that device current), and only that address is ever
// handed to kernels.  Every call on a device shares its array: calls that
// overlap on one device race.  The K-split counters that must start at zero
// are cleared by a fill kernel in the stream before each GEMM that uses them.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

qlora_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QLORA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QLORA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return QLORA_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<uint8_t*>(base) + off);
}

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" {

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "invalid shape (sizes must be positive, n a multiple of 64, within index range)";
    case QLORA_ERR_RANK: return "rank r must be in 1..128";
    case QLORA_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case QLORA_ERR_WORKSPACE: return "workspace is NULL or too small";
    case QLORA_ERR_HIP: return "a HIP launch failed";
    case QLORA_ERR_VALUE: return "invalid value (non-finite s or unknown op)";
    case QLORA_ERR_INCOMPLETE: return "a bounded wait inside a kernel ran out: that call's outputs are unreliable";
    default: return "unknown status";
  }
}

int qlora_version(void) { return 100; }

void qlora_nf4_table(float* levels, float* thresholds) {
  const Nf4Table& t = table();
  if (levels) std::memcpy(levels, t.q, sizeof(t.q));
  if (thresholds) std::memcpy(thresholds, t.t, sizeof(t.t));
}

qlora_status qlora_level_table(int32_t qtype, float* levels, float* thresholds) {
  if (!valid_qtype(qtype)) return QLORA_ERR_VALUE;
  const Nf4Table& t = table(qtype);
  if (levels) std::memcpy(levels, t.q, sizeof(t.q));
  if (thresholds) std::memcpy(thresholds, t.t, sizeof(t.t));
  return QLORA_OK;
}

qlora_status qlora_quantize_dq(int32_t qtype, const float* W, int64_t m, int64_t n, uint8_t* codes,
                               uint8_t* absmax8, float* c2, qlora_stream_t stream) {
  if (!valid_qtype(qtype)) return QLORA_ERR_VALUE;
  if (!W || !codes || !absmax8 || !c2) return QLORA_ERR_NULL;
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax8) || !aligned16(c2)) return QLORA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("quantize", s);
    launch_quantize(W, m * n, codes, absmax8, c2, table(qtype), s);
  }
  return hip_status();
}

qlora_status qlora_quantize_dq_grouped(int32_t qtype, int32_t count, const qlora_quant_weight* weights,
                                       qlora_stream_t stream) {
  if (!valid_qtype(qtype)) return QLORA_ERR_VALUE;
  if (!weights) return QLORA_ERR_NULL;
  if (count < 1 || count > max_quant_weights()) return QLORA_ERR_VALUE;
  QuantWeight w[8];
  for (int i = 0; i < count; ++i) {
    const qlora_quant_weight& q = weights[i];
    if (!q.W || !q.codes || !q.absmax8 || !q.c2) return QLORA_ERR_NULL;
    const qlora_status st = check_weight_shape(q.m, q.n);
    if (st != QLORA_OK) return st;
    if (!aligned16(q.W) || !aligned16(q.codes) || !aligned16(q.absmax8) || !aligned16(q.c2)) return QLORA_ERR_ALIGN;
    w[i] = QuantWeight{q.W, q.m * q.n, q.codes, q.absmax8, q.c2};
  }
  // m n <= 2^40 per weight: at most 8 * 2^26 groups, one workgroup each
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("quantize", s);
    launch_quantize_grouped(w, count, table(qtype), s);
  }
  return hip_status();
}

qlora_status qlora_dequant_dq(int32_t qtype, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                              int64_t m, int64_t n, qlora_bf16* W_out, qlora_stream_t stream) {
  if (!valid_qtype(qtype)) return QLORA_ERR_VALUE;
  if (!codes || !absmax8 || !c2 || !W_out) return QLORA_ERR_NULL;
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (!aligned16(codes) || !aligned16(absmax8) || !aligned16(c2) || !aligned16(W_out)) return QLORA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("dequant", s);
    launch_dequant(codes, absmax8, c2, m * n, W_out, table(qtype), s);
  }
  return hip_status();
}

qlora_status qlora_quantize_nf4_dq(const float* W, int64_t m, int64_t n, uint8_t* codes, uint8_t* absmax8,
                                   float* c2, qlora_stream_t stream) {
  if (!W || !codes || !absmax8 || !c2) return QLORA_ERR_NULL;
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (!aligned16(W) || !aligned16(codes) || !aligned16(absmax8) || !aligned16(c2)) return QLORA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("quantize", s);
    launch_quantize(W, m * n, codes, absmax8, c2, table(), s);
  }
  return hip_status();
}

qlora_status qlora_dequant_nf4_dq(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m,
                                  int64_t n, qlora_bf16* W_out, qlora_stream_t stream) {
  if (!codes || !absmax8 || !c2 || !W_out) return QLORA_ERR_NULL;
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (!aligned16(codes) || !aligned16(absmax8) || !aligned16(c2) || !aligned16(W_out)) return QLORA_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("dequant", s);
    launch_dequant(codes, absmax8, c2, m * n, W_out, table(), s);
  }
  return hip_status();
}

qlora_status qlora_merge_adapter(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m,
                                 int64_t n, int32_t r, float s, const qlora_bf16* A, const qlora_bf16* B,
                                 qlora_bf16* W_out, qlora_stream_t stream) {
  if (!codes || !absmax8 || !c2 || !A || !B || !W_out) return QLORA_ERR_NULL;
  qlora_status st = check_weight_shape(m, n);
  if (st != QLORA_OK) return st;
  if (r < 1 || r > kMaxRank) return QLORA_ERR_RANK;
  if (!std::isfinite(s)) return QLORA_ERR_VALUE;
  if ((int64_t)r * n * 2 >= ((int64_t)1 << 32)) return QLORA_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(absmax8) || !aligned16(c2) || !aligned16(A) || !aligned16(B) ||
      !aligned16(W_out))
    return QLORA_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("merge", hs);
    launch_merge_adapter(codes, absmax8, c2, m, n, r, s, A, B, W_out, table(), hs);
  }
  return hip_status();
}

qlora_status qlora_adam_step(const qlora_adam_tensor* tensors, int32_t count, float lr, float beta1, float beta2,
                             float eps, float weight_decay, int64_t step, qlora_stream_t stream) {
  if (!tensors) return QLORA_ERR_NULL;
  if (count < 1) return QLORA_ERR_SHAPE;
  if (step < 1 || !std::isfinite(lr) || lr < 0.0f || !std::isfinite(eps) || eps < 0.0f ||
      !std::isfinite(weight_decay) || !(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return QLORA_ERR_VALUE;
  std::vector<AdamTensorHost> ts((size_t)count);
  for (int i = 0; i < count; ++i) {
    const qlora_adam_tensor& t = tensors[i];
    if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq) return QLORA_ERR_NULL;
    if (t.count < 1 || t.count >= ((int64_t)1 << 40)) return QLORA_ERR_SHAPE;
    if (!aligned16(t.param) || !aligned16(t.grad) || !aligned16(t.exp_avg) || !aligned16(t.exp_avg_sq) ||
        (t.param_bf16 && !aligned16(t.param_bf16)))
      return QLORA_ERR_ALIGN;
    ts[(size_t)i] = AdamTensorHost{t.count, t.param, t.param_bf16, t.grad, t.exp_avg, t.exp_avg_sq};
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  {
    Timed tm("adam", hs);
    for (int i = 0; i < count; i += 64)
      launch_adam_step(ts.data() + i, count - i < 64 ? count - i : 64, lr, beta1, beta2, eps, weight_decay, step, hs);
  }
  return hip_status();
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t n, int64_t m, int32_t r) {
  if (check_linear(M, n, m, r, 1.0f) != QLORA_OK) return 0;
  if (op == QLORA_OP_FWD) return fwd_ws(M, n, m, r).total;
  if (op == QLORA_OP_BWD) return bwd_ws(M, n, m, r).total;
  if (op == QLORA_OP_BWD_DROPOUT) return bwd_ws(M, n, m, r, true).total;
  return 0;
}

qlora_status qlora_linear_fwd(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                              const uint8_t* codes, const uint8_t* absmax8, const float* c2, const qlora_bf16* A,
                              const qlora_bf16* B, qlora_bf16* h, float* u_out, void* workspace,
                              size_t workspace_bytes, qlora_stream_t stream) {
  return qlora_linear_fwd_ex(M, n, m, r, s, x, codes, absmax8, c2, A, B, h, u_out, nullptr, workspace,
                             workspace_bytes, stream);
}

// Checks shared by the forward entry points (everything but the workspace).
static qlora_status check_fwd_args(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                   const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                                   const qlora_bf16* A, const qlora_bf16* B, qlora_bf16* h, float* u_out) {
  qlora_status st = check_linear(M, n, m, r, s);
  if (st != QLORA_OK) return st;
  if (!x || !codes || !absmax8 || !c2 || !A || !B || !h) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(absmax8) || !aligned16(c2) || !aligned16(A) ||
      !aligned16(B) || !aligned16(h) || (u_out && !aligned16(u_out)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// The forward's launches on a checked workspace laid out by fwd_ws; with
// use_ksplit false the GEMM runs every tile whole (no K-split region needed).
static qlora_status run_fwd(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                            const uint8_t* codes, const uint8_t* absmax8, const float* c2, const qlora_bf16* A,
                            const qlora_bf16* B, qlora_bf16* h, float* u_out, const DropoutDev& dd, float inv_keep,
                            const FwdWs& w, bool use_ksplit, void* workspace, hipStream_t hs) {
  if (M <= small_max_tokens()) {
    SmallLayerHost L{x, codes, absmax8, c2, A, B, h, u_out, n, m, r, s, workspace};
    L.drop = dd;
    L.u_scale = inv_keep;
    Timed tm("fwd_small", hs);
    launch_small_fwd((int)M, &L, 1, table(), hs);
    return hip_status();
  }
  float* u = u_out ? u_out : at<float>(workspace, w.u);
  void* ksplit = (use_ksplit && w.has_ksplit) ? at<uint8_t>(workspace, w.ksplit) : nullptr;
  {
    // u's split sum also clears the GEMM's hand-off words
    Timed tm("down_proj", hs);
    launch_down_proj(x, M, n, A, r, at<float>(workspace, w.part), w.splits, u, hs, &dd, inv_keep,
                     gemm_split_sync(M, m, n, ksplit));
  }
  {
    Timed tm("fwd_gemm", hs);
    launch_fwd_gemm(x, codes, absmax8, c2, B, u, h, M, n, m, r, s, ksplit, table(), hs, true);
  }
  return hip_status();
}

qlora_status qlora_linear_fwd_ex(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                 const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                                 const qlora_bf16* A, const qlora_bf16* B, qlora_bf16* h, float* u_out,
                                 const qlora_dropout* dropout, void* workspace, size_t workspace_bytes,
                                 qlora_stream_t stream) {
  qlora_status st = check_fwd_args(M, n, m, r, s, x, codes, absmax8, c2, A, B, h, u_out);
  if (st != QLORA_OK) return st;
  DropoutDev dd;
  float inv_keep;
  st = make_dropout(dropout, dd, inv_keep);
  if (st != QLORA_OK) return st;
  const FwdWs w = fwd_ws(M, n, m, r);
  if (!workspace || workspace_bytes < w.total) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;
  return run_fwd(M, n, m, r, s, x, codes, absmax8, c2, A, B, h, u_out, dd, inv_keep, w, true, workspace,
                 reinterpret_cast<hipStream_t>(stream));
}

qlora_status qlora_linear_fwd_static(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                     const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                                     const qlora_bf16* A, const qlora_bf16* B, qlora_bf16* h, float* u_out,
                                     qlora_stream_t stream) {
  qlora_status st = check_fwd_args(M, n, m, r, s, x, codes, absmax8, c2, A, B, h, u_out);
  if (st != QLORA_OK) return st;
  const FwdWs w = fwd_ws(M, n, m, r);
  // The whole layout if it fits; otherwise the layout without the GEMM's
  // K-split region (it sits last), whose tiles then run whole.
  bool use_ksplit = true;
  if (w.total > kStaticScratchBytes) {
    use_ksplit = false;
    if (!w.has_ksplit || w.ksplit > kStaticScratchBytes) return QLORA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != QLORA_OK) return st;
  DropoutDev dd;
  float inv_keep;
  make_dropout(nullptr, dd, inv_keep);
  struct NoProfile {
    NoProfile() { t_prof_suppressed = true; }
    ~NoProfile() { t_prof_suppressed = false; }
  } no_profile;
  return run_fwd(M, n, m, r, s, x, codes, absmax8, c2, A, B, h, u_out, dd, inv_keep, w, use_ksplit, ws,
                 reinterpret_cast<hipStream_t>(stream));
}

static qlora_status check_layer(int64_t M, const qlora_linear_layer& L) {
  qlora_status st = check_linear(M, L.n, L.m, L.r, L.s);
  if (st != QLORA_OK) return st;
  if (!L.x || !L.codes || !L.absmax8 || !L.c2 || !L.A || !L.B || !L.h) return QLORA_ERR_NULL;
  if (!aligned16(L.x) || !aligned16(L.codes) || !aligned16(L.absmax8) || !aligned16(L.c2) || !aligned16(L.A) ||
      !aligned16(L.B) || !aligned16(L.h) || (L.u_out && !aligned16(L.u_out)))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

size_t qlora_grouped_workspace_bytes(int64_t M, int32_t count, const qlora_linear_layer* layers) {
  if (!layers || count < 1 || count > small_max_layers()) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    if (check_linear(M, layers[i].n, layers[i].m, layers[i].r, 1.0f) != QLORA_OK) return 0;
    total += align256(fwd_ws(M, layers[i].n, layers[i].m, layers[i].r).total);
  }
  return total;
}

qlora_status qlora_linear_fwd_grouped(int64_t M, int32_t count, const qlora_linear_layer* layers, void* workspace,
                                      size_t workspace_bytes, qlora_stream_t stream) {
  if (!layers) return QLORA_ERR_NULL;
  if (count < 1 || count > small_max_layers()) return QLORA_ERR_VALUE;
  for (int i = 0; i < count; ++i) {
    const qlora_status st = check_layer(M, layers[i]);
    if (st != QLORA_OK) return st;
  }
  const size_t need = qlora_grouped_workspace_bytes(M, count, layers);
  if (!workspace || workspace_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (M > small_max_tokens()) {
    size_t off = 0;
    for (int i = 0; i < count; ++i) {
      const qlora_linear_layer& L = layers[i];
      const size_t wb = align256(fwd_ws(M, L.n, L.m, L.r).total);
      const qlora_status st = qlora_linear_fwd(M, L.n, L.m, L.r, L.s, L.x, L.codes, L.absmax8, L.c2, L.A, L.B, L.h,
                                               L.u_out, at<uint8_t>(workspace, off), wb, stream);
      if (st != QLORA_OK) return st;
      off += wb;
    }
    return QLORA_OK;
  }
  SmallLayerHost H[8];
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    const qlora_linear_layer& L = layers[i];
    H[i] = SmallLayerHost{L.x, L.codes, L.absmax8, L.c2, L.A, L.B, L.h, L.u_out, L.n, L.m, L.r, L.s,
                          at<uint8_t>(workspace, off)};
    off += align256(fwd_ws(M, L.n, L.m, L.r).total);
  }
  {
    Timed tm("fwd_small", hs);
    launch_small_fwd((int)M, H, count, table(), hs);
  }
  return hip_status();
}

qlora_status qlora_linear_bwd(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                              const qlora_bf16* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                              const qlora_bf16* A, const qlora_bf16* B, const float* u, qlora_bf16* grad_x,
                              qlora_bf16* grad_A, qlora_bf16* grad_B, void* workspace, size_t workspace_bytes,
                              qlora_stream_t stream) {
  return qlora_linear_bwd_ex(M, n, m, r, s, x, g, codes, absmax8, c2, A, B, u, grad_x, grad_A, grad_B, nullptr,
                             workspace, workspace_bytes, stream);
}

qlora_status qlora_linear_bwd_ex(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                 const qlora_bf16* g, const uint8_t* codes, const uint8_t* absmax8,
                                 const float* c2, const qlora_bf16* A, const qlora_bf16* B, const float* u,
                                 qlora_bf16* grad_x, qlora_bf16* grad_A, qlora_bf16* grad_B,
                                 const qlora_dropout* dropout, void* workspace, size_t workspace_bytes,
                                 qlora_stream_t stream) {
  qlora_status st = check_linear(M, n, m, r, s);
  if (st != QLORA_OK) return st;
  DropoutDev dd;
  float inv_keep;
  st = make_dropout(dropout, dd, inv_keep);
  if (st != QLORA_OK) return st;
  const bool drop = dd.on != 0;
  if (!x || !g || !codes || !absmax8 || !c2 || !A || !B || !grad_A || !grad_B) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(g) || !aligned16(codes) || !aligned16(absmax8) || !aligned16(c2) ||
      !aligned16(A) || !aligned16(B) || !aligned16(grad_A) || !aligned16(grad_B) || (u && !aligned16(u)) ||
      (grad_x && !aligned16(grad_x)))
    return QLORA_ERR_ALIGN;
  const BwdWs w = bwd_ws(M, n, m, r, drop);
  if (!workspace || workspace_bytes < w.total) return QLORA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return QLORA_ERR_ALIGN;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  float* part = at<float>(workspace, w.part_uv);
  const int64_t mk = w.m_pad;
  const uint16_t* gk = g;
  if (mk != m) {
    Timed tp("transpose", hs);
    uint16_t* gp = at<uint16_t>(workspace, w.gpad);
    launch_pad_cols_bf16(g, M, m, mk, gp, hs);
    gk = gp;
  }
  const float* uu = u;
  if (!uu) {
    Timed tm("down_proj", hs);
    launch_down_proj(x, M, n, A, r, part, w.su, at<float>(workspace, w.u), hs, &dd, inv_keep);
    uu = at<float>(workspace, w.u);
  }
  float* v = at<float>(workspace, w.v);
  uint16_t* vplanes = at<uint16_t>(workspace, w.planes);
  if (w.gpass) {
    // v = g B and grad_B = s g^T u from one read of g; then v (the sum of
    // its partials) with its bf16 planes for grad_A in one launch
    Timed tm("gpass", hs);
    launch_gpass(gk, M, mk, B, m, uu, r, at<float>(workspace, w.vpart), at<float>(workspace, w.gbpart), hs);
    launch_factor_planes(at<float>(workspace, w.vpart), gpass_splits_f(M, mk, r), M, r, vplanes, v, nullptr, nullptr,
                         hs);
  } else {
    uint16_t* uplanes = at<uint16_t>(workspace, w.uplanes);
    const bool bt = down_proj_bt_supported(r);
    if (!bt) {
      Timed tm("transpose", hs);
      launch_transpose_bf16(B, m, r, mk, at<uint16_t>(workspace, w.Bt), hs);
    }
    {
      // v partials (from B itself, or from its transposed copy); then v, its
      // planes and u's planes in one launch
      Timed tm("down_proj", hs);
      if (bt)
        launch_down_proj_bt(gk, M, mk, B, m, r, part, w.sv, hs);
      else
        launch_down_proj(gk, M, mk, at<uint16_t>(workspace, w.Bt), r, part, w.sv, nullptr, hs, nullptr, 1.0f);
      launch_factor_planes(part, w.sv, M, r, vplanes, v, uu, uplanes, hs);
    }
    {
      Timed tm("token_grad", hs);
      launch_token_grad(gk, M, mk, uu, r, w.sb, at<float>(workspace, w.gB), hs, nullptr, uplanes, true);
    }
  }
  void* ksplit = (grad_x && w.has_ksplit) ? at<uint8_t>(workspace, w.ksplit) : nullptr;
  {
    Timed tm("token_grad", hs);
    // grad_A = s v^T x_d with x_d = (x * keep) / (1 - p); then the split
    // sums of grad_B and grad_A in one launch, which also clears the grad_x
    // GEMM's hand-off words
    launch_token_grad(x, M, n, v, r, w.sa, at<float>(workspace, w.gA), hs, &dd, vplanes, true);
    const SyncZero z = gemm_split_sync(M, n, w.m_pad, ksplit);
    if (w.gpass)
      launch_reduce_grads(at<float>(workspace, w.gbpart), gpass_splits_t(M), mk, m, s, grad_B,
                          at<float>(workspace, w.gA), w.sa, n, n, s * inv_keep, grad_A, r, hs, z);
    else
      launch_reduce_grads(at<float>(workspace, w.gB), w.sb, mk, m, s, grad_B, at<float>(workspace, w.gA), w.sa, n, n,
                          s * inv_keep, grad_A, r, hs, z);
  }
  if (grad_x) {
    if (drop) {
      // the adapter part s (v A) * keep / (1 - p) in fp32; the GEMM adds it
      // to g W' before rounding and runs no LoRA steps of its own
      float* dterm = at<float>(workspace, w.dterm);
      {
        Timed tm("dropout_term", hs);
        launch_lora_dropout_term(v, A, M, n, r, s * inv_keep, dd, dterm, hs);
      }
      Timed tm("dgrad_gemm", hs);
      launch_dgrad_gemm(gk, codes, absmax8, c2, A, v, grad_x, M, n, m, w.m_pad, 0, s, ksplit, table(), hs, dterm,
                        true);
    } else {
      Timed tm("dgrad_gemm", hs);
      launch_dgrad_gemm(gk, codes, absmax8, c2, A, v, grad_x, M, n, m, w.m_pad, r, s, ksplit, table(), hs, nullptr,
                        true);
    }
  }
  return hip_status();
}

qlora_status qlora_linear_check(int op, int64_t M, int64_t n, int64_t m, int32_t r, const void* workspace,
                                qlora_stream_t stream) {
  qlora_status st = check_linear(M, n, m, r, 1.0f);
  if (st != QLORA_OK) return st;
  if (op != QLORA_OP_FWD && op != QLORA_OP_BWD && op != QLORA_OP_BWD_DROPOUT) return QLORA_ERR_VALUE;
  int64_t off = -1;
  if (op == QLORA_OP_FWD) {
    if (M > small_max_tokens()) {
      const FwdWs w = fwd_ws(M, n, m, r);
      const int64_t g = gemm_giveup_offset(M, m, n);
      if (w.has_ksplit && g >= 0) off = (int64_t)w.ksplit + g;
    }
  } else {
    const BwdWs w = bwd_ws(M, n, m, r, op == QLORA_OP_BWD_DROPOUT);
    const int64_t g = gemm_giveup_offset(M, n, w.m_pad);
    if (w.has_ksplit && g >= 0) off = (int64_t)w.ksplit + g;
  }
  if (off < 0) return QLORA_OK;  // this call has no bounded wait
  if (!workspace && op == QLORA_OP_FWD) {
    // qlora_linear_fwd_static's scratch, when its layout kept the K split
    if (fwd_ws(M, n, m, r).total > kStaticScratchBytes) return QLORA_OK;
    void* ws = nullptr;
    const qlora_status st2 = static_scratch(&ws);
    if (st2 != QLORA_OK) return st2;
    workspace = ws;
  }
  if (!workspace) return QLORA_ERR_NULL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, static_cast<const uint8_t*>(workspace) + off, sizeof(word), hipMemcpyDeviceToHost, hs) !=
          hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return QLORA_ERR_HIP;
  return word ? QLORA_ERR_INCOMPLETE : QLORA_OK;
}

qlora_status qlora_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    for (auto& rec : g_recs) {
      (void)hipEventDestroy(rec.a);
      (void)hipEventDestroy(rec.b);
    }
    g_recs.clear();
  }
  g_prof_on = on != 0;
  return QLORA_OK;
}

qlora_status qlora_profile_query(const char* name, int64_t* launches, double* total_ms) {
  if (!name || !launches || !total_ms) return QLORA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t cnt = 0;
  double tot = 0.0;
  for (auto& rec : g_recs) {
    if (rec.name != name) continue;
    if (hipEventSynchronize(rec.b) != hipSuccess) return QLORA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, rec.a, rec.b) != hipSuccess) return QLORA_ERR_HIP;
    ++cnt;
    tot += ms;
  }
  *launches = cnt;
  *total_ms = tot;
  return QLORA_OK;
}

}  // extern "C"
