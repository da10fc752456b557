/*
 * qlora.h -- C ABI of the MI355X (gfx950) QLoRA adapted-linear library.
 *
 * The library computes the hot path of QLoRA fine-tuning for one linear layer:
 *   - blockwise NF4 quantization of a frozen weight with double quantization
 *     of the block constants;
 *   - the adapted forward  h = x W'^T + s (x A^T) B^T,  W' = dequant(W0);
 *   - its backward through the frozen 4-bit weight: grad_x, grad_A, grad_B.
 * Sources are the QLoRA pages cited at each entry point below.
 *
 * Conventions for every call:
 *   - All tensors are dense, row-major, and live in device memory (HBM) of
 *     the current HIP device, except where a pointer is marked "host".
 *   - bf16 tensors are passed as raw 16-bit patterns (qlora_bf16).
 *   - Every base pointer of a device tensor must be 16-byte aligned.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronizes device memory; workspaces are passed in.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *     stream).  Outputs are overwritten, never accumulated into.
 *   - Argument errors are reported synchronously, before anything is
 *     launched, and leave every output untouched.  A failed launch returns
 *     QLORA_ERR_HIP; outputs are then unspecified.
 *   - Inputs must be finite; non-finite weights or activations give
 *     unspecified (but memory-safe) results.
 *   - Calls that share a workspace must be ordered (same stream, or
 *     synchronized); calls with separate workspaces may overlap.
 */
#ifndef QLORA_H_
#define QLORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qlora_bf16;                 /* raw bfloat16 bits */
typedef struct ihipStream_t* qlora_stream_t; /* same type as hipStream_t */

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,      /* a required pointer is NULL */
  QLORA_ERR_SHAPE = -2,     /* a size <= 0, n % 64 != 0, or an index overflow */
  QLORA_ERR_RANK = -3,      /* r outside 1..128 */
  QLORA_ERR_ALIGN = -4,     /* a device pointer is not 16-byte aligned */
  QLORA_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required */
  QLORA_ERR_HIP = -6,       /* a HIP launch or query failed */
  QLORA_ERR_VALUE = -7,     /* s is not finite, or an unknown op id */
  QLORA_ERR_INCOMPLETE = -8 /* a kernel's bounded wait ran out (qlora_linear_check) */
} qlora_status;

/* Human-readable text of a status code (static storage). */
const char* qlora_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int qlora_version(void);

/*
 * The 16 NF4 levels and 15 decision thresholds the library uses (host).
 * Levels: q_i = Phi^-1((i - 1/2)/16), i = 1..16 ("QLoRA: Efficient
 * Fine-Tuning", Step 1, Eq. 2), divided by q_16 so they span exactly [-1, 1]
 * (the normalized weight range of Eq. 1), rounded to fp32.  Thresholds are
 * the fp32-rounded midpoints of adjacent levels; a normalized weight takes
 * the code of the number of thresholds strictly below it (ties go to the
 * lower code).  Derived on the host at load time.
 * levels: host float[16]; thresholds: host float[15].  Either may be NULL.
 */
void qlora_nf4_table(float* levels, float* thresholds);

/*
 * Quantize an m x n fp32 weight (out x in) to NF4 with double quantization.
 * "QLoRA: Efficient Fine-Tuning", Step 1 (Eq. 1: divide by the block absmax;
 * Eq. 2: normal-quantile levels; snap to the nearest level) and Step 2
 * (the absmax constants quantized again to an 8-bit float in blocks of 256);
 * block of 64 weights from "What is QLoRA?" ("The three pieces").
 *   W        device, m*n fp32, row-major; blocks are 64 consecutive elements
 *            along n, groups are 256 consecutive blocks (16384 elements; the
 *            last group may be partial).
 *   codes    device out, m*n/2 bytes of 4-bit codes.  Code of level L
 *            (0..15, ascending): bit 3 = sign (set for the 8 negative
 *            levels), bits 0-2 = rank of |level| (L - 8 for L >= 8, 15 - L
 *            for L < 8).  Per 8 consecutive elements e..e+7 (a 32-bit word),
 *            byte j holds element e+j in its low nibble and e+j+4 in its high
 *            nibble.
 *   absmax8  device out, m*n/64 bytes: E4M3FN (bias 7, RNE) of c1_b / c2_g,
 *            where c1_b is the fp32 absmax of block b.
 *   c2       device out, ceil(m*n/16384) fp32: c2_g = max c1_b over group g.
 * Requires m >= 1, n >= 64, n % 64 == 0.  Output is bit-identical for a
 * given W (no atomics, no reduction-order dependence).
 */
qlora_status qlora_quantize_nf4_dq(const float* W, int64_t m, int64_t n, uint8_t* codes, uint8_t* absmax8,
                                   float* c2, qlora_stream_t stream);

/*
 * Dequantize to bf16: W'_e = bf16_rne(fl32(level[code_e] * s_b)) with
 * s_b = fl32(dec(absmax8_b) * c2_g) ("QLoRA: Efficient Fine-Tuning", Step 3
 * symbols: W0 is dequantized to BF16 at run time).  This is exactly the
 * operand the forward and backward kernels build in on-chip memory.
 *   W_out    device out, m*n bf16.
 * Same shape rules as qlora_quantize_nf4_dq.
 */
qlora_status qlora_dequant_nf4_dq(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m,
                                  int64_t n, qlora_bf16* W_out, qlora_stream_t stream);

/*
 * Merge a trained adapter into the weight ("QLoRA: Efficient Fine-Tuning",
 * Real-World Impact: W_merged = W0 + B A, no adapter cost at inference;
 * "QLoRA & 4-bit Fine-Tuning", Followups to expect: dequantize to BF16, add
 * the adapter, keep a 16-bit model), with the adapter's alpha/r scale:
 *   W_out = bf16(W' + s B A),  W' = the bf16 dequantized weight above.
 *   codes, absmax8, c2: the quantized m x n weight.
 *   A        device, r x n bf16.      B  device, m x r bf16.
 *   W_out    device out, m*n bf16.
 * The product B A accumulates in fp32 and is added to W' with one fused
 * multiply-add before the single rounding to bf16, so each element is the
 * exactly rounded sum or one of its bf16 neighbours (the fp32 error is far
 * below half a bf16 unit); with B = 0 or s = 0 it is W' bit for bit.
 * Requires m >= 1, n >= 64, n % 64 == 0, r in 1..128, finite s,
 * r * n < 2^31.  Every pointer 16-byte aligned.
 */
qlora_status qlora_merge_adapter(const uint8_t* codes, const uint8_t* absmax8, const float* c2, int64_t m,
                                 int64_t n, int32_t r, float s, const qlora_bf16* A, const qlora_bf16* B,
                                 qlora_bf16* W_out, qlora_stream_t stream);

/*
 * One adapter tensor of an optimizer step (host struct; device-addressable
 * pointers: device memory, or pinned host memory for state kept in CPU RAM).
 *   count       elements (>= 1).
 *   param       fp32 master weights, updated in place.
 *   param_bf16  bf16 copy written after the update (the operand the forward
 *               and backward read), or NULL.
 *   grad        bf16 gradient (as qlora_linear_bwd writes it).
 *   exp_avg, exp_avg_sq  fp32 first and second moments, updated in place
 *               (zero before the first step).
 * Every pointer 16-byte aligned.
 */
typedef struct {
  int64_t count;
  float* param;
  qlora_bf16* param_bf16;
  const qlora_bf16* grad;
  float* exp_avg;
  float* exp_avg_sq;
} qlora_adam_tensor;

/*
 * Adam step with decoupled weight decay over `count` adapter tensors in as
 * few launches as possible (64 tensors per launch).  "QLoRA: Efficient
 * Fine-Tuning", memory-layout figure (Adam moments for the adapters only,
 * paged to CPU memory on demand); "What is QLoRA?", Worked example (fp32
 * parameter, gradient and moments, 16 bytes per trainable parameter);
 * "QLoRA & 4-bit Fine-Tuning", Innovation 3 (paged optimizer state).  With
 * t = step (>= 1), per element in fp32:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
 *   p <- p - (lr / (1 - b1^t)) m / (sqrt(v / (1 - b2^t)) + eps)
 * (the bias corrections are formed in double on the host).  Requires lr,
 * eps >= 0 and weight_decay finite, 0 <= beta1, beta2 < 1.  `tensors` is a
 * host array read before the call returns.  Results match a float64
 * evaluation of the same step to fp32 rounding.
 */
qlora_status qlora_adam_step(const qlora_adam_tensor* tensors, int32_t count, float lr, float beta1, float beta2,
                             float eps, float weight_decay, int64_t step, qlora_stream_t stream);

/* Level tables for qlora_quantize_dq / qlora_dequant_dq / qlora_level_table. */
#define QLORA_QTYPE_NF4 0        /* the NF4 levels above */
#define QLORA_QTYPE_UNIFORM4 1   /* uniform 4-bit grid (2j - 15)/15, j = 0..15 */
#define QLORA_QTYPE_EDGE_MEAN4 2 /* mean of each bucket's edge quantiles (below) */
#define QLORA_QTYPE_INT4 3       /* INT4 absmax grid k/7, k = -7..7 (below) */

/*
 * The 16 levels and 15 thresholds of a level table (host outputs, either
 * may be NULL).  QLORA_QTYPE_UNIFORM4 is the plain 4-bit comparison point of
 * "QLoRA: Efficient Fine-Tuning" Step 1 and "QLoRA & 4-bit Fine-Tuning"
 * Innovation 1 (NF4 versus uniform 4-bit quantization of normal weights):
 * 16 evenly spaced levels over [-1, 1] without a zero level, symmetric like
 * the NF4 table so the same code layout and kernels apply; thresholds are
 * the fp32 midpoints.  QLORA_QTYPE_EDGE_MEAN4 is the other normal-quantile
 * construction, of "QLoRA & 4-bit Fine-Tuning" Innovation 1: level i is the
 * mean of the normal quantiles at its bucket's edges i/16 and (i + 1)/16;
 * as printed the outermost edges (probabilities 0 and 1) have infinite
 * quantiles, so they are moved to the outer buckets' midpoints 1/32 and
 * 31/32, and the levels are normalized by the largest.  QLORA_QTYPE_INT4 is
 * symmetric 4-bit integer absmax quantization, the uniform comparison point
 * those passages name: the 15 levels k/7, k = -7..7, with the zero level
 * held twice, as -0 (index 7) and +0 (index 8), so that the table keeps the
 * sign-magnitude symmetry of the code layout; the fp32 midpoint between
 * them is 0, a normalized weight w_hat > 0 takes +0 or above and w_hat <= 0
 * takes -0 or below, and both dequantize to the value 0.  QLORA_ERR_VALUE
 * for an unknown qtype.
 */
qlora_status qlora_level_table(int32_t qtype, float* levels, float* thresholds);

/*
 * qlora_quantize_nf4_dq / qlora_dequant_nf4_dq with a chosen level table
 * (qtype 0 gives exactly those calls).  Blocks, double quantization, code
 * layout, shape rules and errors as there; QLORA_ERR_VALUE for an unknown
 * qtype.  The linear forward and backward use NF4 only.
 */
qlora_status qlora_quantize_dq(int32_t qtype, const float* W, int64_t m, int64_t n, uint8_t* codes,
                               uint8_t* absmax8, float* c2, qlora_stream_t stream);
qlora_status qlora_dequant_dq(int32_t qtype, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                              int64_t m, int64_t n, qlora_bf16* W_out, qlora_stream_t stream);

/*
 * One weight of a grouped quantization (host struct): W, its shape and its
 * outputs, each as for qlora_quantize_nf4_dq.
 */
typedef struct {
  const float* W;
  int64_t m, n;
  uint8_t* codes;
  uint8_t* absmax8;
  float* c2;
} qlora_quant_weight;

/*
 * Quantize `count` weights (for example the seven frozen weights of a
 * transformer block) in one launch, each exactly as qlora_quantize_dq with
 * the same qtype would (the same bits); one launch over all of them keeps the
 * GPU's memory pipeline full where a weight alone has too few 16384-element
 * groups to (1024 x 4096: 256 groups, one per compute unit).  The blocks of
 * 64 and groups of 256 blocks are those of "QLoRA: Efficient Fine-Tuning",
 * Steps 1 and 2.  `weights` is a host array read before the call returns;
 * count 1..8; the weights' outputs must not overlap.  Errors as for
 * qlora_quantize_dq (qtype, then the array: NULL, count), checked for every
 * weight before anything is launched.
 */
qlora_status qlora_quantize_dq_grouped(int32_t qtype, int32_t count, const qlora_quant_weight* weights,
                                       qlora_stream_t stream);

/* Operation ids for qlora_workspace_bytes. */
#define QLORA_OP_FWD 0
#define QLORA_OP_BWD 1
#define QLORA_OP_BWD_DROPOUT 2 /* qlora_linear_bwd_ex with dropout on */

/*
 * Workspace bytes needed by qlora_linear_fwd (op 0, also
 * qlora_linear_fwd_ex), qlora_linear_bwd (op 1, also qlora_linear_bwd_ex
 * without dropout) or qlora_linear_bwd_ex with dropout (op 2: an M x n fp32
 * buffer more) for these sizes; 0 on invalid arguments.  The bwd figures
 * assume u is recomputed (the most they can need).
 */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t n, int64_t m, int32_t r);

/*
 * Adapted forward ("QLoRA: Efficient Fine-Tuning", Step 3, Eq. 3, with the
 * alpha/r scale of the LoraConfig snippet):
 *   u = x A^T                      (M x r, fp32 accumulation)
 *   h = bf16(x W'^T + s u B^T)     (M x m)
 * with W' the dequantized weight (bf16, formed on chip, never in HBM).
 *   M tokens, n in-features, m out-features, r rank (1..128), s = alpha/r.
 *   x        device, M x n bf16.
 *   codes, absmax8, c2: the quantized m x n weight.
 *   A        device, r x n bf16.      B  device, m x r bf16.
 *   h        device out, M x m bf16.
 *   u_out    device out, M x r fp32, or NULL.  Keep it for the backward.
 *   workspace, workspace_bytes: at least qlora_workspace_bytes(0, ...).
 * Size limits (32-bit offsets): M * max(n, m) < 2^30 and m * n < 2^31.
 * M <= 32 takes the weight-streaming path (bound by reading the packed
 * weight); larger M the tiled MFMA path.  Both give the same results up to
 * fp32 summation order.
 */
qlora_status qlora_linear_fwd(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                              const uint8_t* codes, const uint8_t* absmax8, const float* c2, const qlora_bf16* A,
                              const qlora_bf16* B, qlora_bf16* h, float* u_out, void* workspace,
                              size_t workspace_bytes, qlora_stream_t stream);

/*
 * qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  Same arguments, results and rules as
 * qlora_linear_fwd (with a workspace of qlora_workspace_bytes(0, ...) the
 * two give identical bits).  The scratch is a library-owned device array of
 * QLORA_STATIC_SCRATCH_BYTES per device, held until the process ends; the
 * call allocates and frees nothing (with library profiling switched on it
 * records no events: qlora_profile_query does not see it).  When the
 * forward's workspace layout is
 * larger than that array, the call runs its GEMM without the K-split region
 * (every output tile whole: same results up to fp32 summation order) if the
 * rest fits, and otherwise returns QLORA_ERR_WORKSPACE before launching
 * anything.  Every call on a device shares that device's array, which keeps
 * the last call's contents: calls that overlap on one device (several
 * streams or threads without ordering) race and must not be issued.
 * qlora_linear_check(QLORA_OP_FWD, ..., NULL, stream) checks the last such
 * call.
 */
#define QLORA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
qlora_status qlora_linear_fwd_static(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                     const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                                     const qlora_bf16* A, const qlora_bf16* B, qlora_bf16* h, float* u_out,
                                     qlora_stream_t stream);

/*
 * One layer of a grouped forward: the arguments of qlora_linear_fwd for one
 * weight (all device pointers, same rules).  Host struct.
 */
typedef struct {
  int64_t n, m;
  int32_t r;
  float s;
  const qlora_bf16* x;
  const uint8_t* codes;
  const uint8_t* absmax8;
  const float* c2;
  const qlora_bf16* A;
  const qlora_bf16* B;
  qlora_bf16* h;
  float* u_out; /* may be NULL */
} qlora_linear_layer;

/*
 * Workspace bytes for qlora_linear_fwd_grouped with these layers (host
 * array of `count`); 0 on invalid arguments.
 */
size_t qlora_grouped_workspace_bytes(int64_t M, int32_t count, const qlora_linear_layer* layers);

/*
 * Forward of `count` independent adapted linear layers that share the token
 * count M (for example the seven projections of a transformer block), each
 * exactly as qlora_linear_fwd would compute it.  For M <= 32 the layers are
 * streamed by one launch (plus one launch that finishes them), which keeps
 * the GPU busy on layers too small to fill it alone; larger M runs the
 * layers one after another.  `layers` is a host array, read before the call
 * returns; count 1..8.  Errors as for qlora_linear_fwd, checked for every
 * layer before anything is launched.
 */
qlora_status qlora_linear_fwd_grouped(int64_t M, int32_t count, const qlora_linear_layer* layers, void* workspace,
                                      size_t workspace_bytes, qlora_stream_t stream);

/*
 * Backward of the forward above for upstream gradient g = dL/dh
 * ("QLoRA: Efficient Fine-Tuning", Step 4 and Eq. 5; s from the snippet):
 *   v      = g B                          (M x r, fp32)
 *   grad_x = bf16(g W' + s v A)           (M x n)   -- W0 gets no gradient
 *   grad_A = bf16(s v^T x)                (r x n)
 *   grad_B = bf16(s g^T u)                (m x r)
 *   g        device, M x m bf16.
 *   u        device, M x r fp32 from qlora_linear_fwd, or NULL to recompute.
 *   grad_x   device out, M x n bf16, or NULL to skip the input gradient.
 *   grad_A, grad_B  device out (required).
 * The reductions over tokens use fixed-order fp32 partials: results are
 * bit-identical run to run.
 */
qlora_status qlora_linear_bwd(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                              const qlora_bf16* g, const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                              const qlora_bf16* A, const qlora_bf16* B, const float* u, qlora_bf16* grad_x,
                              qlora_bf16* grad_A, qlora_bf16* grad_B, void* workspace, size_t workspace_bytes,
                              qlora_stream_t stream);

/*
 * LoRA dropout on the adapter input ("QLoRA: Efficient Fine-Tuning", the
 * LoraConfig snippet's lora_dropout, with Step 3's adapter branch): the
 * adapter reads x_d = x * keep / (1 - p) instead of x, while the frozen
 * weight still reads x.  Host struct.
 *   p       drop probability, 0 <= p < 1 (p = 0 is the plain layer).
 *   seed    Philox key: low and high 32-bit words.
 *   offset  added to every counter (advance it by ceil(M n / 4) per call
 *           for a fresh mask).
 * Mask: element e = t n + k of x takes word e % 4 of Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, SC 2011) at the 64-bit counter e / 4 + offset (low
 * word first, upper two words zero), and is kept when that word is at least
 * round(p 2^32) (ties to even, capped at 2^32 - 1).  The forward and the
 * backward with the same struct draw the same mask.
 */
typedef struct {
  float p;
  uint64_t seed;
  uint64_t offset;
} qlora_dropout;

/*
 * qlora_linear_fwd with dropout on the adapter input (NULL or p = 0: exactly
 * qlora_linear_fwd):
 *   u = (x * keep) A^T / (1 - p),   h = bf16(x W'^T + s u B^T)
 * u_out receives that u (the backward's grad_B needs it).  Workspace as for
 * qlora_linear_fwd.  QLORA_ERR_VALUE when p is outside [0, 1) or not finite.
 */
qlora_status qlora_linear_fwd_ex(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                 const uint8_t* codes, const uint8_t* absmax8, const float* c2,
                                 const qlora_bf16* A, const qlora_bf16* B, qlora_bf16* h, float* u_out,
                                 const qlora_dropout* dropout, void* workspace, size_t workspace_bytes,
                                 qlora_stream_t stream);

/*
 * qlora_linear_bwd for the forward above, with the same mask (NULL or
 * p = 0: exactly qlora_linear_bwd).  Chain rule with the mask fixed:
 *   v      = g B
 *   grad_x = bf16(g W' + s (v A) * keep / (1 - p))
 *   grad_A = bf16(s v^T (x * keep) / (1 - p))
 *   grad_B = bf16(s g^T u)
 * u: the forward's u_out (with the mask), or NULL to recompute it with the
 * mask.  The adapter part of grad_x is formed in fp32 (an M x n buffer in
 * the workspace) and added before the single rounding.  Workspace: at least
 * qlora_workspace_bytes(QLORA_OP_BWD_DROPOUT, ...) when p > 0.
 */
qlora_status qlora_linear_bwd_ex(int64_t M, int64_t n, int64_t m, int32_t r, float s, const qlora_bf16* x,
                                 const qlora_bf16* g, const uint8_t* codes, const uint8_t* absmax8,
                                 const float* c2, const qlora_bf16* A, const qlora_bf16* B, const float* u,
                                 qlora_bf16* grad_x, qlora_bf16* grad_A, qlora_bf16* grad_B,
                                 const qlora_dropout* dropout, void* workspace, size_t workspace_bytes,
                                 qlora_stream_t stream);

/*
 * Completion check of the last qlora_linear_fwd / qlora_linear_bwd(_ex)
 * call (op QLORA_OP_FWD, QLORA_OP_BWD or QLORA_OP_BWD_DROPOUT) that used
 * `workspace` with these sizes.  When a GEMM has more output tiles than the
 * GPU has compute units and its last round is at most half full, the tiles
 * of that round run as two K halves: the half that finishes second waits,
 * for a bounded time, for the other half's fp32 sum ("QLoRA: Efficient
 * Fine-Tuning", Step 3, Eq. 3: the output those tiles hold).  If that wait
 * ever ran out, the call wrote a give-up word in its workspace and this
 * returns QLORA_ERR_INCOMPLETE (that call's h or grad_x is then unreliable);
 * QLORA_OK otherwise, and always for calls without such a split.  The word
 * is cleared by the next call that uses the workspace.  With op
 * QLORA_OP_FWD, a NULL workspace means the library's scratch of
 * qlora_linear_fwd_static.  Synchronizes `stream` (it reads one word back
 * to the host).
 */
qlora_status qlora_linear_check(int op, int64_t M, int64_t n, int64_t m, int32_t r, const void* workspace,
                                qlora_stream_t stream);

/*
 * Kernel timing (tracing aid, off by default).  While enabled, every kernel
 * the library launches is bracketed by HIP events on its stream.
 * qlora_profile_enable(1) clears earlier records; (0) stops recording.
 * qlora_profile_query waits for the recorded events of kernel `name`
 * ("quantize", "dequant", "fwd_gemm", "fwd_small", "dgrad_gemm",
 * "down_proj", "token_grad", "transpose", "gpass", "dropout_term", "merge",
 * "adam") and reports the launch
 * count and the summed duration in milliseconds (host pointers).
 */
qlora_status qlora_profile_enable(int on);
qlora_status qlora_profile_query(const char* name, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H_ */
