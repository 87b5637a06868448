/*
 * gq.h -- C ABI of libgq: group-wise asymmetric MinMax weight quantization
 * (INT4 with groups of 128, INT2 with groups of 64, and 8-bit blocks with
 * groups of 128 for rows kept at higher precision) and the weight-only
 * low-bit matmul that consumes the packed format, for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources the operations follow (page title, then the part of the page):
 *   GreenBitAI, "只需单卡 RTX 3090 低比特量化训练就能实现 LLaMA-3 8B 全参微调":
 *     two-stage quantization -- a group-wise MinMax quantizer with
 *     round-to-nearest, INT4 (group size 128) and INT2 (group size 64) as the
 *     only base representations; Layer-mix (one bit-width per linear) and
 *     Channel-mix (bit-width per block of output channels) layouts.
 *   "大模型量化实战：从原理到4-bit部署的完整指南", section 2.2 -- the affine
 *     quantizer Q(x) = round(x/s) + z, s = (x_max - x_min)/(q_max - q_min),
 *     z = round(0 - x_min/s), z kept inside the integer range; section 4.2
 *     -- one layer (lm_head) kept at 8 bits inside a 4-bit model; section
 *     5.1 -- a zero-point configuration with groups of 128, the group size
 *     taken here for 8-bit blocks (the pages give none).
 *   "Low-bit Quantization: Slimming Large Models to the Extreme", "Zero
 *     Point" -- dequantized value = (quantized value - zero_point) x scale.
 *   "A Survey of Low-bit Large Language Models" (paper review), sections
 *     5.2 and 6.2 -- weight-only quantization dequantizes and then runs an
 *     FP16 matmul; its speed-up comes from moving fewer weight bytes.
 *
 * Conventions for every entry point
 *   - W is the weight of a linear layer y = x . W^T, stored [N][K] row-major
 *     (N output channels, K input channels, K contiguous).  Groups run along
 *     K.  x is [M][K] and y is [M][N], both row-major.
 *   - Per group of g weights: lo = min, hi = max (fp32);
 *     s32 = (hi - lo) / (2^b - 1) (fp32, correctly rounded);
 *     S = fp16(s32) rounded to nearest even, replaced by 1.0 if it is zero;
 *     z = clamp(rint(-lo / S), 0, 2^b - 1) stored as uint8;
 *     code = clamp(rint(w / S) + z, 0, 2^b - 1); rint rounds half to even
 *     and the divisions are correctly rounded fp32 divisions.
 *   - Packed codes: each row of a block is K*b/8 bytes; uint32 word j of a
 *     row holds codes k = j*32/b + i at bits [b*i, b*i + b), little-endian.
 *     Scales (fp16 bit patterns) and zeros (uint8) are [rows][K/g] per block.
 *     Blocks are stored back to back in block order: block i's codes start at
 *     byte sum_{j<i} block_n*K*b_j/8 and its scales/zeros at group
 *     sum_{j<i} block_n*K/g_j.
 *   - Pointers marked DEVICE are device (HBM) memory of the current HIP
 *     device; HOST pointers are read during the call only.  The caller owns
 *     every buffer; the library allocates nothing and keeps no per-call state.
 *   - All GPU work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream) and is asynchronous: a GQ_OK return means the work was
 *     enqueued.  Calls are reentrant; calls that share an output buffer must
 *     be ordered by the caller.
 *   - Errors: argument checks run on the host before anything is enqueued and
 *     return a non-zero gq_status without side effects.  A failed kernel
 *     launch returns GQ_ERR_HIP.  No exception crosses the ABI, nothing is
 *     printed and nothing aborts.
 */
#ifndef GQ_H
#define GQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Under C++ both enums have int as their fixed underlying type (the size C
 * gives them), so any int a C or foreign-function caller passes is a valid
 * value that the checks below can reject, not undefined behaviour. */
#ifdef __cplusplus
#define GQ_ENUM_INT : int
#else
#define GQ_ENUM_INT
#endif

typedef enum gq_status GQ_ENUM_INT {
  GQ_OK = 0,
  GQ_ERR_NULL_ARG = 1,   /* a required pointer is NULL                          */
  GQ_ERR_SHAPE = 2,      /* K<=0, N<0, M<0, N % block_n, K % g, too many blocks */
  GQ_ERR_BITS = 3,       /* a bit-width other than 2, 4 or 8                    */
  GQ_ERR_ALIGNMENT = 4,  /* a device pointer is not 16-byte aligned             */
  GQ_ERR_DTYPE = 5,      /* unsupported dtype for this argument                 */
  GQ_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than required             */
  GQ_ERR_HIP = 7,        /* the HIP runtime refused a launch                    */
  GQ_ERR_TOO_LARGE = 8,  /* gq_linear_noalloc: scratch need above the static size */
  GQ_ERR_UNSUPPORTED = 9 /* a layout with 8-bit blocks on a path without an 8-bit
                            kernel (gq_linear with M > 4, gq_linear_dx)          */
} gq_status;

typedef enum gq_dtype GQ_ENUM_INT { GQ_BF16 = 0, GQ_FP16 = 1, GQ_FP32 = 2 } gq_dtype;

/* Device flag bits OR-ed into *flags by gq_quantize_pack and gq_fake_quant. */
#define GQ_FLAG_NONFINITE 1u      /* a group held NaN or Inf; its codes are unspecified   */
#define GQ_FLAG_SCALE_OVERFLOW 2u /* (hi-lo)/(2^b-1) rounded to fp16 infinity (> 65504)   */
/* A finite group whose zero point rint(-lo/S) fell outside [0, 2^b - 1] and
 * was clamped (its values all of one sign, away from 0): its codes saturate
 * at the clamp, so its largest (or smallest) values dequantize with an error
 * above S/2.  Reported, not an error: the format keeps z in the code range. */
#define GQ_FLAG_ZERO_CLAMPED 4u

/* Largest number of bit-width blocks in one layout. */
#define GQ_MAX_BLOCKS 1024

/* Bit-width map of one linear (the mixed-precision layouts of GreenBitAI's
 * two-stage quantization).  N/block_n blocks of block_n consecutive output
 * channels; bits[i] in {4, 2, 8} is block i's width (INT4 uses groups of 128,
 * INT2 groups of 64; 8 marks a block kept at higher precision, groups of
 * 128, as section 4.2 of the 4-bit deployment guide keeps lm_head at 8 bits).
 * A uniform linear (Layer-mix) has block_n == N and one entry; Channel-mix
 * uses block_n == 128.  Rules: N % block_n == 0; when there is more than one
 * block, block_n % 128 == 0; K is a positive multiple of 128 if any block is
 * INT4 or 8-bit, else of 64.  `bits` is a HOST array.  Layouts with 8-bit
 * blocks are accepted by gq_packed_bytes, gq_quantize_pack, gq_dequant,
 * gq_fake_quant, gq_linear / gq_linear_noalloc with M <= 4 and the grouped
 * decode calls; the other paths return GQ_ERR_UNSUPPORTED. */
typedef struct gq_layout {
  int32_t K;
  int32_t N;
  int32_t block_n;
  const uint8_t *bits;
} gq_layout;

/* Sizes of the three packed buffers for `layout`, in bytes (HOST outputs).
 * codes: sum over blocks of block_n*K*b/8, b bits per weight with nothing
 * between codes (the dense sizes of the memory table of "Low-bit
 * Quantization: Slimming Large Models to the Extreme": INT4 35 GB and INT2
 * 17.5 GB for 70e9 weights); scales: 2 bytes per group; zeros: 1 byte per
 * group.  Pure host computation. */
gq_status gq_packed_bytes(const gq_layout *layout, size_t *codes_bytes,
                          size_t *scales_bytes, size_t *zeros_bytes);

/* Quantize W and pack it (GreenBitAI group-wise MinMax; section 2.2 of the
 * 4-bit deployment guide).
 *   w      DEVICE fp32 [N][K], 16-byte aligned, read only.
 *   codes  DEVICE, gq_packed_bytes codes bytes, 16-byte aligned, written.
 *   scales DEVICE fp16 bit patterns, 2-byte aligned, written.
 *   zeros  DEVICE uint8, written.
 *   flags  DEVICE uint32 or NULL; GQ_FLAG_* bits are OR-ed in (never cleared).
 * Codes, scales and zeros are bit-identical to the definition above.  A group
 * holding NaN/Inf sets GQ_FLAG_NONFINITE and gets unspecified codes. */
gq_status gq_quantize_pack(const gq_layout *layout, const float *w, uint32_t *codes,
                           uint16_t *scales, uint8_t *zeros, uint32_t *flags, void *stream);

/* Dequantize: w_out[n][k] = (code - z) * S ("Zero Point" of the low-bit
 * tutorial).  The value is exact in fp32; GQ_BF16 and GQ_FP16 outputs are
 * that value rounded to nearest even.
 *   codes/scales/zeros  DEVICE, as written by gq_quantize_pack.
 *   w_out  DEVICE [N][K] of out_dtype, 16-byte aligned. */
gq_status gq_dequant(const gq_layout *layout, const uint32_t *codes, const uint16_t *scales,
                     const uint8_t *zeros, gq_dtype out_dtype, void *w_out, void *stream);

/* Fake quantization: w_out = (code - z) * S with S, z and the codes of
 * gq_quantize_pack, without packing -- the forward of a FakeQuantize module
 * in quantization-aware training ("大模型量化实战：从原理到4-bit部署的完整指南",
 * section 5.2: quantize and dequantize in the forward, FP32 gradient in the
 * backward).  Equal to gq_quantize_pack followed by gq_dequant, bit for bit,
 * in one pass over w.  The straight-through backward is the identity
 * (dL/dw = dL/dw_out: a MinMax range clips no weight), so it has no entry
 * point.
 *   w      DEVICE fp32 [N][K], 16-byte aligned, read only.
 *   w_out  DEVICE [N][K] of out_dtype (GQ_FP32 exact; GQ_BF16 / GQ_FP16
 *          rounded to nearest even), 16-byte aligned, written; may not alias w.
 *   flags  DEVICE uint32 or NULL; GQ_FLAG_* bits as for gq_quantize_pack. */
gq_status gq_fake_quant(const gq_layout *layout, const float *w, gq_dtype out_dtype, void *w_out,
                        uint32_t *flags, void *stream);

/* Workspace gq_linear needs for this layout, M and activation dtype (HOST
 * output *bytes; may be 0): room for the fp16 activations and the split-K
 * fp32 partials of the floating-point matmul that weight-only quantization
 * runs after dequantization (the survey review, section 5.2); 0 for M <= 4.
 * GQ_ERR_UNSUPPORTED for 8-bit blocks with M > 4.  Pure host computation. */
gq_status gq_linear_workspace_bytes(const gq_layout *layout, int32_t M, gq_dtype act,
                                    size_t *bytes);

/* Weight-only low-bit matmul y = x . W_hat^T with W_hat = (code - z) * S
 * (the survey review, sections 5.2 and 6.2: dequantize, then a floating-point
 * matmul; dequantization happens in registers, W_hat never reaches memory).
 *   act    GQ_BF16 or GQ_FP16: dtype of x and y.
 *   x      DEVICE [M][K] act, 16-byte aligned.
 *   y      DEVICE [M][N] act, 2-byte aligned, written (bf16/fp16 rounded to
 *          nearest even from an fp32 accumulator).
 *   workspace  DEVICE, 256-byte aligned, at least gq_linear_workspace_bytes;
 *          may be NULL when that is 0.  Overwritten (needs no
 *          initialisation); calls that share a workspace must be ordered on
 *          one stream.
 * Kernels by M:
 *   M <= 4       bandwidth-bound dot-product kernel; (code - z) and S are
 *                applied exactly in fp32.
 *   4 < M <= 32  MFMA on the activations as given (bf16 or fp16), the
 *                codes as exact B + q values and the zero point as the exact
 *                constant -(B + z), accumulated per group in fp32; each
 *                group's scale is applied in fp32 after its MFMAs.  Long K ranges,
 *                and small layers that would leave CUs idle, are split
 *                across workgroups (fp32 partials in the workspace, summed in
 *                split order).
 *   M > 32       MFMA GEMM that rounds each dequantized weight once to fp16
 *                (the FP16 matmul of the survey review); activations are
 *                rescaled per row by a power of two so that their fp16 form
 *                is exact; small M splits K across workgroups, and with
 *                256 x 256 tiles the tiles of an incomplete last round are
 *                split along K (fp32 parts in the workspace, summed in part
 *                order).
 * Every path is deterministic.  Results agree with the fp64 product of the
 * dequantized weights to about the bf16 output rounding (normwise relative
 * error <= 2e-3). */
gq_status gq_linear(const gq_layout *layout, int32_t M, gq_dtype act, const void *x,
                    const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                    void *y, void *workspace, size_t workspace_bytes, void *stream);

/* gq_linear without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory around the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as gq_linear (bit for bit); the
 * workspace those kernels need is a static device array of
 * GQ_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends.  The array is scratch: no kernel needs it
 * initialised, and each call overwrites what the previous call left.
 * Calls on one GPU that may overlap in time (on different streams) share
 * the array and race: the caller orders them.  A call whose workspace need
 * (gq_linear_workspace_bytes) exceeds GQ_NOALLOC_SCRATCH_BYTES returns
 * GQ_ERR_TOO_LARGE before anything is enqueued; M <= 4, the small-batch
 * path on most layers and prefill GEMMs up to about M * K = 2^24 fit.
 * The first call on a device resolves that device's array address
 * (hipGetSymbolAddress, with the device current); no call allocates. */
#define GQ_NOALLOC_SCRATCH_BYTES (64u << 20)
gq_status gq_linear_noalloc(const gq_layout *layout, int32_t M, gq_dtype act, const void *x,
                            const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                            void *y, void *stream);

/* ---------------------------------------------------------- grouped decode
 * Many independent decode linears (M <= 4) in as few launches as their
 * kernel classes allow, for a Layer-mix model pass (GreenBitAI's Layer-mix
 * layout: one bit-width per linear; the survey review, section 6.2: the
 * speed-up of weight-only quantization is the weight bytes not moved, so a
 * decode pass should stream its packed weights without a launch ramp and
 * tail per linear).  Each output is y_i = x_i . W_hat_i^T exactly as
 * gq_linear computes it for M <= 4 (same arithmetic, same rounding, bit for
 * bit).  Linears may mix INT4, INT2 and Channel-mix layouts and shapes; they
 * share M and the activation dtype.  Outputs must not alias inputs or each
 * other: the linears of one call run concurrently.
 *
 * Use: gq_group_plan_bytes, then gq_group_plan into a HOST buffer of that
 * size; copy the bytes unchanged into DEVICE memory (16-byte aligned) once;
 * then every gq_linear_group(plan, plan_dev, stream) runs the whole group.
 * The plan records the device pointers of every item, so it is rebuilt when
 * a buffer moves.  No workspace is needed. */
typedef struct gq_group_item {
  gq_layout layout;       /* bit map of the linear (HOST bits, read by gq_group_plan only) */
  const void *x;          /* DEVICE [M][K] act, 16-byte aligned                        */
  const uint32_t *codes;  /* DEVICE packed codes, 16-byte aligned                      */
  const uint16_t *scales; /* DEVICE fp16 bit patterns, 2-byte aligned                  */
  const uint8_t *zeros;   /* DEVICE uint8                                              */
  void *y;                /* DEVICE [M][N] act, 2-byte aligned, written                */
} gq_group_item;

/* Bytes of the plan of `count` items (HOST output *bytes).  Checks every item
 * as gq_linear would (GQ_ERR_SHAPE also for M outside 1..4 or count outside
 * 1..65535).  Pure host computation. */
gq_status gq_group_plan_bytes(int32_t count, const gq_group_item *items, int32_t M, gq_dtype act,
                              size_t *bytes);

/* Encode the plan into `plan` (HOST, plan_bytes >= gq_group_plan_bytes).
 * Pure host computation; returns the same errors as gq_group_plan_bytes and
 * GQ_ERR_WORKSPACE when plan_bytes is too small. */
gq_status gq_group_plan(int32_t count, const gq_group_item *items, int32_t M, gq_dtype act,
                        void *plan, size_t plan_bytes);

/* Run every linear of a plan.  plan: the HOST plan (launch configuration);
 * plan_dev: a DEVICE byte copy of it, 16-byte aligned, which the kernels
 * read (it must equal `plan`; it is not checked on the device).  Returns
 * GQ_ERR_SHAPE if `plan` is not a plan of this library version. */
gq_status gq_linear_group(const void *plan, const void *plan_dev, void *stream);

/* Workspace gq_linear_dx needs for this layout, M and dtype (HOST output
 * *bytes; may be 0): the fp16 form of dy and the fp32 partials of the
 * data-gradient product (GreenBitAI, the Q-SFT paragraph: training through
 * the quantized weights).  Returns GQ_ERR_SHAPE where gq_linear_dx would (N
 * not a multiple of 8, or buffers past 2 GiB) and GQ_ERR_UNSUPPORTED for
 * 8-bit blocks.  Pure host computation. */
gq_status gq_linear_dx_workspace_bytes(const gq_layout *layout, int32_t M, gq_dtype act,
                                       size_t *bytes);

/* Data gradient of gq_linear: dx = dy . W_hat, dx[m][k] = sum_n dy[m][n] *
 * W_hat[n][k], the product back-propagation needs to train through the
 * packed weights (GreenBitAI, the Q-SFT and Bitorch Engine paragraphs:
 * full-parameter fine-tuning in the quantized weight space).  Same
 * arithmetic as the M > 32 path of gq_linear: each dequantized weight rounded
 * once to fp16, dy rescaled per row by a power of two so that its fp16 form is
 * exact, MFMA with fp32 accumulation, x 2^e and round to nearest even.
 *   act    GQ_BF16 or GQ_FP16: dtype of dy and dx.
 *   dy     DEVICE [M][N] act, 16-byte aligned; N must be a multiple of 8.
 *   dx     DEVICE [M][K] act, 2-byte aligned, written.
 *   workspace  DEVICE, 256-byte aligned, at least
 *          gq_linear_dx_workspace_bytes; overwritten; calls sharing it must
 *          be ordered on one stream.
 * Work is tiled 256 (m) x 256 (k); the reduction over n is split across
 * workgroups when the tiles alone would leave CUs idle (fp32 parts in the
 * workspace, summed in part order).  Deterministic.  N == 0 writes zeros.
 * Errors: GQ_ERR_SHAPE for N % 8 != 0 (and the layout rules of gq_linear). */
gq_status gq_linear_dx(const gq_layout *layout, int32_t M, gq_dtype act, const void *dy,
                       const uint32_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       void *dx, void *workspace, size_t workspace_bytes, void *stream);

/* A group-wise quantized KV cache for one decode step of attention (the
 * review of "A Survey of Low-bit Large Language Models": KV-cache
 * compression with low-bit formats, a quantization window that keeps the
 * newest tokens unquantized).  `batch` sequences of equal length; per
 * sequence t_packed packed tokens followed by t_window dense tokens.
 *   Packed part: the output of gq_quantize_pack for the fp32 cache
 *   [batch * t_packed][kv_heads * head_dim] with one uniform layout
 *   {K = kv_heads * head_dim, N = batch * t_packed, block_n = N, bits}:
 *   one row per token (sequence b's rows are b * t_packed ..), groups of 128
 *   (INT4) or 64 (INT2) features.  DEVICE pointers, 16-byte aligned codes.
 *   Window: DEVICE bf16 [batch][t_window][kv_heads][head_dim], 16-byte
 *   aligned (may be NULL when t_window is 0).
 * Rules: head_dim = 128; q_heads / kv_heads in {1, 2, 4, 8};
 * t_packed + t_window >= 1; t_window <= 1024; packed code bytes < 2 GiB. */
typedef struct gq_kv_cache {
  int32_t batch;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t bits;
  int32_t t_packed;
  int32_t t_window;
  const uint32_t *k_codes;
  const uint16_t *k_scales;
  const uint8_t *k_zeros;
  const uint32_t *v_codes;
  const uint16_t *v_scales;
  const uint8_t *v_zeros;
  const void *k_window;
  const void *v_window;
} gq_kv_cache;

/* Workspace gq_kv_attention needs (HOST output *bytes): the per-split
 * softmax statistics and partial outputs of the decode attention over the
 * quantized cache (the survey review's KV-cache bullet).  Pure host. */
gq_status gq_kv_attention_workspace_bytes(const gq_kv_cache *cache, size_t *bytes);

/* One decode step: for every sequence b and query head h (key/value head
 * h / (q_heads / kv_heads)), out = softmax(q . K^T / sqrt(head_dim)) . V over
 * the packed tokens (dequantized: (code - z) * S) and the window tokens.
 *   q    DEVICE bf16 [batch][q_heads][head_dim], 16-byte aligned.
 *   out  DEVICE bf16 [batch][q_heads][head_dim], written (round to nearest
 *        even of an fp32 result).
 *   workspace  DEVICE, 256-byte aligned, >= the workspace size; overwritten.
 * q . K^T multiplies exact fp16 forms (q rescaled per head by a power of
 * two, codes as 1024 + c, the zero point as -(1024 + z)) with fp32
 * accumulation; softmax and P . V run in fp32.  Deterministic. */
gq_status gq_kv_attention(const gq_kv_cache *cache, const void *q, void *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *gq_status_string(gq_status status);

#ifdef __cplusplus
}
#endif
#endif /* GQ_H */
