/*
 * wq.h -- C ABI of libwq: weight-only quantized decode matvecs on AMD MI355X
 * (gfx950).
 *
 * The operation is the batch-1 decode product y = x . W^T of a linear layer
 * whose weight W [N_out][K_in] is stored quantized: it is applied once per
 * generated token, so its cost is the bytes of W it streams.  Sources, by
 * page title and section:
 *
 *   [README]   gittoolsai.com "gpt-fast" (Chinese mirror of the project
 *              README): "量化" (quantization) with "Int8 仅权重量化" and
 *              "Int4 仅权重量化" (int8 / int4 weight-only, group size 32);
 *              "基准测试" (batch-1 benchmark table: tokens/s and GB/s per
 *              format); "推测采样" (speculative sampling); "Mixtral 8x7B".
 *   [GUIDE]    onegen.ai "Efficiently implementing the Mixtral 8x7B model
 *              with gpt-fast": "Key Features" (int8/int4 weight-only
 *              quantization; a draft model's tokens verified by the larger
 *              model).
 *   [TAGS]     awesome-repositories.com "meta-pytorch/gpt-fast": tag
 *              "Grouped Quantization".
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every buffer is DEVICE memory owned by the caller.  The library allocates
 *   nothing.  Its only state: a thread-local error text, per-device host
 *   caches (device check, occupancy; safe across host threads) and the
 *   static device scratch of moe_top2_gemv_noalloc.  Passing a host pointer
 *   is outside the contract (the kernel would fault).
 * - Row-major layouts; bf16 values are passed as their uint16 bit patterns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *   is enqueued and the call returns without synchronising.
 * - Outputs must not alias inputs.  Where both `y_f32` and `y_bf16` are
 *   accepted, either may be NULL but not both; y_bf16 is the fp32 result
 *   rounded to nearest-even.
 * - Return value: a wq_status.  Arguments are checked on the host before
 *   anything is launched; a non-OK return launched nothing, except
 *   WQ_ERR_LAUNCH, which reports a failed launch.  No call aborts or prints;
 *   wq_last_error() gives the detail of the calling thread's last failure.
 * - Weights must be finite.  This is not checked; the result of a
 *   non-finite weight is unspecified.
 * - Alignment: x, weight and code pointers 16-byte aligned (WQ_ERR_ALIGN).
 * - Sizes: n >= 0, k >= 0 (n == 0 is a no-op).  K limits per format are
 *   stated at each call; a larger K returns WQ_ERR_SHAPE.
 * - Only gfx950 devices are supported (WQ_ERR_DEVICE otherwise).
 * - Results are deterministic: the same inputs give bitwise the same
 *   outputs (fixed reduction order, no atomics).
 */
#ifndef WQ_H
#define WQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_ERR_NULL = 1,   /* a required pointer is NULL                       */
  WQ_ERR_SHAPE = 2,  /* a size is negative, unsupported or inconsistent  */
  WQ_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned                 */
  WQ_ERR_DEVICE = 4, /* no current HIP device, or it is not gfx950       */
  WQ_ERR_LAUNCH = 5  /* the HIP runtime reported a launch failure        */
} wq_status;

/* ------------------------------------------------------------------------ */
/* Quantizers (offline: once per weight, not per token) -- [README] "Int8   */
/* 仅权重量化", "Int4 仅权重量化"; [TAGS] "Grouped Quantization".            */
/* ------------------------------------------------------------------------ */

/*
 * int8 weight-only, per output row (symmetric).
 *   in : w      fp32 [n][k], k % 4 == 0 (16-byte aligned)
 *   out: q      int8 [n][k]    codes in [-127, 127]
 *        scale  bf16 [n]       s = bf16(fp32(max_k |w[r][k]| / 127))
 * q[r][k] = round-half-even of the exact quotient w[r][k] / s (the stored
 * bf16 s), clamped to [-127, 127]; a zero scale gives zero codes.  Hence
 * |w - q s| <= s / 2.  Codes are bit-identical to the CPU oracle's.
 * q 4-byte and scale 2-byte aligned; no upper limit on k.
 */
int wq_quantize_int8(const float* w, int64_t n, int64_t k, int8_t* q, uint16_t* scale,
                     void* stream);

/*
 * int4 weight-only, groups of 32 consecutive inputs of one row (asymmetric).
 *   in : w        fp32 [n][k], k % 32 == 0 (w, qpacked 16-byte aligned,
 *                  sz 4-byte aligned)
 *   out: qpacked  u8   [n][k/2]    byte j = code(2j) | code(2j+1) << 4
 *        sz       bf16 [n][k/32][2] = (scale s, zero z) per group
 * z = bf16(min of the group) is what code 0 decodes to; t = fp32(max - z);
 * s = bf16(fp32(t / 15)) if t > 0 else 0.  code = round-half-even of the
 * exact quotient (w - z) / s clamped to [0, 15] (0 when s == 0); the value a
 * code stands for is z + code * s.  0.625 byte per weight.  Bit-identical to
 * the CPU oracle.
 */
int wq_quantize_int4g32(const float* w, int64_t n, int64_t k, uint8_t* qpacked, uint16_t* sz,
                        void* stream);

/*
 * int4 with a chosen group size -- [README] "Int4 仅权重量化" (the int4
 * quantizer takes a group size; the benchmark rows show 32);
 * [TAGS] "Grouped Quantization".  As wq_quantize_int4g32 with groups of
 * `group` consecutive inputs, group one of 32, 64, 128, 256, or group == k
 * (one group per output row, "per-channel"; k a positive multiple of 32):
 *   sz bf16 [n][k/group][2]; 0.5 + 4/group bytes per weight.
 * k % group == 0.  Errors: WQ_ERR_SHAPE for another group size.
 */
int wq_quantize_int4(const float* w, int64_t n, int64_t k, int32_t group, uint8_t* qpacked, uint16_t* sz,
                     void* stream);

/* ------------------------------------------------------------------------ */
/* Decode matvecs, batch 1 -- [README] "基准测试" (Base / 8-bit / 4-bit     */
/* (G=32) rows: the per-token linear layers of batch-1 generation).         */
/* Accumulation is fp32.                                                    */
/* ------------------------------------------------------------------------ */

/*
 * Unquantized baseline.  x bf16 [k]; w bf16 [n][k];
 * y[r] = sum_k x[k] * w[r][k].   k % 8 == 0, k <= 65536.
 */
int wq_gemv_bf16(const uint16_t* x, const uint16_t* w, int64_t n, int64_t k, float* y_f32,
                 uint16_t* y_bf16, void* stream);

/*
 * int8 per-row.  x bf16 [k]; q int8 [n][k]; scale bf16 [n] (as written by
 * wq_quantize_int8); y[r] = scale[r] * sum_k x[k] * q[r][k].
 * k % 16 == 0, k <= 65536.
 */
int wq_gemv_int8(const uint16_t* x, const int8_t* q, const uint16_t* scale, int64_t n, int64_t k,
                 float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * int4 G=32.  x bf16 [k]; qpacked, sz as written by wq_quantize_int4g32;
 * y[r] = sum_g ( s[r][g] * sum_{k in g} x[k] code[r][k] + z[r][g] * sum_{k in g} x[k] ).
 * k % 32 == 0, k <= 131072.
 */
int wq_gemv_int4g32(const uint16_t* x, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                    int64_t k, float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * int4 with groups of `group` inputs (32, 64, 128, 256, or k: one group per
 * row), qpacked and sz as written by wq_quantize_int4 with that group; the
 * same sum over groups of `group`.  k % group == 0 (k % 32 == 0 for a
 * per-row group), k <= 131072.  group == 32 is wq_gemv_int4g32.
 * Errors: WQ_ERR_SHAPE for another group size.
 */
int wq_gemv_int4(const uint16_t* x, const uint8_t* qpacked, const uint16_t* sz, int64_t n, int64_t k,
                 int32_t group, float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * Speculative-decoding verify -- [GUIDE] "Key Features" (the larger model
 * checks the draft's tokens), [README] "推测采样".  The m draft tokens go
 * through one int4 G=32 linear in one pass, each weight read once:
 *   x bf16 [m][k], 1 <= m <= 8; y [m][n]; row i of y equals
 *   wq_gemv_int4g32 applied to row i of x (to fp32 rounding).
 * k % 32 == 0, k <= 131072.  From two tokens on the matrix cores (each weight
 * decoded once for all tokens).  The environment variable
 * WQ_SMALLM_ENGINE=valu (read at each call) moves 2, 3 and 5 tokens to the
 * vector ALU where its plans reach (k <= 32768 for int4, 16384 for int8),
 * for comparison; =mfma or unset keeps the matrix cores (measured faster).
 * On the matrix cores, 2..5 tokens over large matrices (k >= 8192 within
 * one activation window, at least 1280 blocks of 32 rows) run a kernel
 * whose workgroups claim row blocks from a per-call counter in a static
 * device array of 1024 slots, each launch taking the next slot and leaving
 * it zeroed: up to 1024 such launches may be in flight on one device at
 * once.  WQ_SMALLM_KERNEL=split or =claim (read at each call) forces the
 * fixed-stride or the claiming kernel wherever a row fits one activation
 * window, for comparison; results agree to fp32 rounding and each kernel's
 * are reproducible bit for bit.
 */
int wq_gemm_smallM(const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz,
                   int64_t n, int64_t k, float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * The same verify product through int4 weights with groups of `group`
 * inputs (32, 64, 128, 256, or k: one group per row), qpacked and sz as
 * written by wq_quantize_int4 with that group -- [TAGS] "Grouped
 * Quantization".  k % group == 0 (k % 32 == 0 for a per-row group); limits
 * as wq_gemm_smallM.  group == 32 is wq_gemm_smallM.
 */
int wq_gemm_smallM_int4(const uint16_t* x, int64_t m, const uint8_t* qpacked, const uint16_t* sz, int64_t n,
                        int64_t k, int32_t group, float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * Speculative-decoding verify through an int8 linear -- [GUIDE] "Key
 * Features", [README] "推测采样" (the verify pass), with the int8 weights of
 * [README] "Int8 仅权重量化".  x bf16 [m][k], 1 <= m <= 8; q, scale as written
 * by wq_quantize_int8; y [m][n] with y[t][r] = scale[r] * sum_k x[t][k] q[r][k];
 * row t of y equals wq_gemv_int8 applied to row t of x (to fp32 rounding).
 * Each weight is read once (m >= 2: on the matrix cores; WQ_SMALLM_ENGINE and
 * WQ_SMALLM_KERNEL as for wq_gemm_smallM, the claiming kernel taken by
 * default from 98304 rows on, for k from 8192 to 32768, with the same
 * per-call slots).  k % 16 == 0; k <= 65536 for m == 1 (the one-token
 * matvec), k <= 2^24 and n * k <= 0xFFFFFF00 for m >= 2.  scale 2-byte
 * aligned.
 */
int wq_gemm_smallM_int8(const uint16_t* x, int64_t m, const int8_t* q, const uint16_t* scale, int64_t n,
                        int64_t k, float* y_f32, uint16_t* y_bf16, void* stream);

/*
 * Top-2 mixture-of-experts decode step for one token, int8 per-row experts
 * -- [README] "Mixtral 8x7B" (sparse MoE, int8 on one GPU).
 *   x       bf16 [dim]
 *   logits  fp32 [e]                 router logits (e == 8)
 *   w13     int8 [e][2f][dim], s13 bf16 [e][2f]   rows 0..f-1: W1 (gate),
 *                                                 rows f..2f-1: W3 (up)
 *   w2      int8 [e][dim][f],  s2  bf16 [e][dim]
 *   work    fp32 [2][f]          caller-provided scratch (overwritten)
 *   sel     int32 [2] or NULL    selected experts, larger gate first
 *   gates   fp32 [2] or NULL     their renormalised gates
 * Routing: softmax over the e logits, keep the two largest (equal logits:
 * lower index first), renormalise the pair (g_a = 1 / (1 + exp(l_b - l_a))).
 * Each selected expert computes a = silu(W1 x) * (W3 x) in fp32 and
 * o = W2 a; y = g_a o_a + g_b o_b.  Only the two selected experts' weights
 * are read; routing happens on the device (no host synchronisation).
 * dim % 16 == 0, f % 16 == 0, 16 <= dim <= 32768, 16 <= f <= 32768; x, w13,
 * w2 and work 16-byte aligned.
 */
int moe_top2_gemv(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                  const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim,
                  int64_t f, float* work, float* y_f32, uint16_t* y_bf16, int32_t* sel,
                  float* gates, void* stream);

/*
 * moe_top2_gemv without the caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments as moe_top2_gemv minus
 * `work`, same results (bitwise: the same kernels run); the fp32 [2][f]
 * SwiGLU intermediate lives in a static device array of the library (one per
 * device, 128 KiB, held until the process ends), so f <= 16384
 * (WQ_ERR_SHAPE beyond).  Allocates nothing and calls no allocating routine.
 * Every call on one device shares that device's array: calls that overlap on
 * one device (different streams, or host threads without ordering) race and
 * give unspecified results; calls ordered on one stream are safe.  The first
 * call on a device looks the array's address up once (with that device
 * current).  The W13 launch writes the whole intermediate before the W2
 * launch reads it, so no contents carry over from an earlier call.
 */
int moe_top2_gemv_noalloc(const uint16_t* x, const float* logits, int64_t e, const int8_t* w13,
                          const uint16_t* s13, const int8_t* w2, const uint16_t* s2, int64_t dim,
                          int64_t f, float* y_f32, uint16_t* y_bf16, int32_t* sel, float* gates,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* A whole decode step in one launch -- [README] "基准测试" (tokens/s of a  */
/* batch-1 step is the time to stream every linear layer once).             */
/* ------------------------------------------------------------------------ */

enum {
  WQ_FORMAT_BF16 = 1,
  WQ_FORMAT_INT8 = 2,
  WQ_FORMAT_INT4G32 = 3,
  /* int4 with larger groups (wq_quantize_int4) */
  WQ_FORMAT_INT4G64 = 4,
  WQ_FORMAT_INT4G128 = 5,
  WQ_FORMAT_INT4G256 = 6,
  /* int4 with one group per row (wq_quantize_int4 with group == k): each
     matrix's sz is [n][1][2]; k % 32 == 0 */
  WQ_FORMAT_INT4PC = 7
};

/* One linear layer of a step, in the layout of the single-matrix calls:
 *   x    bf16 [m][k]   (16-byte aligned)
 *   w    bf16 [n][k] | int8 [n][k] | int4 packed [n][k/2]   (16-byte aligned)
 *   aux  NULL (bf16) | bf16 scale [n] (int8) | sz [n][k/G][2] (int4 with groups of G, G = k per row;
 *        4-byte aligned)
 *   y_f32 / y_bf16  [m][n], either may be NULL but not both. */
typedef struct {
  const void* x;
  const void* w;
  const void* aux;
  int64_t n;
  int64_t k;
  float* y_f32;
  uint16_t* y_bf16;
} wq_matrix;

/* Filled by wq_decode_step_prepare; pass it unchanged to wq_decode_step_run. */
typedef struct {
  int32_t format;
  int32_t m;
  int32_t count;
  int32_t groups;
  int64_t total_batches;
  const void* workspace;
} wq_step_plan;

/* Upper bound of the device workspace a plan of `count` matrices needs. */
int64_t wq_decode_step_workspace_bytes(int32_t count);

/*
 * Plans `count` independent matvecs of one format (m token rows each: m = 1
 * for bf16, 1 <= m <= 8 for int8 and for int4 with any group size) as ONE
 * persistent launch: every
 * workgroup streams an equal share of the step's weight bytes as a contiguous
 * range of row batches across the matrices, so no matrix pays its own
 * launch, ramp-up and drain.  Results equal the single-matrix calls' to fp32
 * rounding (the per-row reduction order may differ).
 * Validates every matrix on the host (null -> sizes -> alignment; k must be a
 * positive multiple of 8 / 16 / G per format (32 for a per-row group) and within the kernel's row
 * limit: with one token row the activations are staged whole in LDS, so
 * k <= 80896 (bf16), 36864 (int8), 73728 (int4); int4 with 2..8 token rows
 * k <= 131072; int8 with 2..8 token rows k <= 2^24 and n * k <= 0xFFFFFF00),
 * then writes the launch description into `workspace` (device
 * memory, 16-byte aligned, `workspace_bytes` long, caller-owned; it must
 * stay allocated and unmodified while the plan is used).  This copy is
 * synchronous: prepare once, outside any graph capture.  The matrices'
 * buffers must stay where they are for as long as the plan is run.
 */
int wq_decode_step_prepare(int32_t format, int32_t m, const wq_matrix* mats, int32_t count,
                           void* workspace, int64_t workspace_bytes, wq_step_plan* plan);

/* Launches a prepared step on `stream` (asynchronous; may be captured into a
 * HIP graph).  Runs of one plan must not overlap (they share its workspace,
 * which carries balance state that each run measures and the next run uses
 * to cut the step into per-CU ranges: the measured speed of each workgroup,
 * and for int4 with 2..8 token rows the relative cost of rows longer than
 * one activation window); runs of plans that share output buffers race. */
int wq_decode_step_run(const wq_step_plan* plan, void* stream);

/* ------------------------------------------------------------------------ */
/* Top-2 MoE decode over many layers in two launches -- [README] "Mixtral   */
/* 8x7B" (a token's MoE layers are streamed once per decode step).          */
/* ------------------------------------------------------------------------ */

/* One MoE layer, with the buffers and layouts of moe_top2_gemv. */
typedef struct {
  const void* x;          /* bf16 [dim], 16-byte aligned */
  const float* logits;    /* fp32 [e] */
  const int8_t* w13;      /* int8 [e][2f][dim], 16-byte aligned */
  const uint16_t* s13;    /* bf16 [e][2f] */
  const int8_t* w2;       /* int8 [e][dim][f], 16-byte aligned */
  const uint16_t* s2;     /* bf16 [e][dim] */
  float* work;            /* fp32 [2][f], 16-byte aligned; caller scratch (overwritten) */
  float* y_f32;           /* [dim] or NULL */
  uint16_t* y_bf16;       /* [dim] or NULL (not both NULL) */
  int32_t* sel;           /* [2] or NULL */
  float* gates;           /* [2] or NULL */
} wq_moe_layer;

/* Filled by wq_moe_step_prepare; pass it unchanged to wq_moe_step_run. */
typedef struct {
  int64_t dim;
  int64_t f;
  int32_t e;
  int32_t count;
  int32_t grid13;
  int32_t grid2;
  const void* workspace;
} wq_moe_plan;

/* Device workspace a plan of `count` layers needs (bytes). */
int64_t wq_moe_step_workspace_bytes(int32_t count);

/*
 * Plans `count` independent MoE layers (each its own token, logits, experts,
 * work buffer and output; every layer computes exactly what moe_top2_gemv
 * computes for it, to fp32 rounding) as two persistent launches: the W13
 * pass of every layer, then the W2 pass of every layer.  All layers share
 * e == 8, dim and f, with dim % 16 == 0, f % 16 == 0, 16 <= dim <= 14336 and
 * 16 <= f <= 16384 (a layer's activations are staged whole in LDS).
 * Validates every layer on the host (null -> sizes -> alignment), then copies
 * the layer descriptors and the two launches' initial balance state into
 * `workspace` (device memory, 16-byte aligned, caller-owned, unmodified
 * while the plan is used).  The copy is synchronous: prepare once, outside
 * any graph capture.
 */
int wq_moe_step_prepare(int64_t e, int64_t dim, int64_t f, const wq_moe_layer* layers, int32_t count,
                        void* workspace, int64_t workspace_bytes, wq_moe_plan* plan);

/* Launches a prepared MoE step on `stream` (asynchronous; may be captured
 * into a HIP graph).  Runs of one plan must not overlap (each run measures
 * its workgroups' speeds into the workspace and later runs cut their per-CU
 * ranges from them); runs of plans that share buffers must not overlap
 * either. */
int wq_moe_step_run(const wq_moe_plan* plan, void* stream);

/* Static text for a wq_status value ("unknown status" otherwise). */
const char* wq_status_string(int status);

/* Detail of the calling thread's last non-OK return ("" if none).  The
 * pointer stays valid until the thread's next failing call. */
const char* wq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
