/*
 * lema.h -- C ABI of liblema.so: the per-layer mixed-precision AdamW update
 * of streamed fine-tuning on one AMD Instinct MI355X (gfx950).
 *
 * Source of the method (the pages this library implements):
 *   LEMA README ("LEMA: Layer-wise Efficient Memory Abstraction"),
 *     "Quick Start": trainable parameters go to torch.optim.AdamW with
 *       lr = 1e-4 (all other settings at AdamW's defaults);
 *     "Selective Full Fine-Tuning": the optimizer is a per-layer AdamW whose
 *       states and gradient accumulators are fp32 and live in host RAM; a
 *       checkpoint stores an fp32 delta (updated minus original weight);
 *     "TensorStore: Unified Streaming Core": optimizer states stream through
 *       a slot-pool address space between RAM and VRAM;
 *   LLMScale fine-tuning VRAM page, memory note and FAQ: mixed-precision
 *     Adam holds 16 bytes per trained parameter (bf16 weight, bf16 gradient,
 *     fp32 master weight, fp32 m, fp32 v).
 *
 * Arithmetic (the pages print no formula; this is the fixed reading).  All
 * operations are IEEE binary32, rounded to nearest even, no fused
 * multiply-add, correctly rounded sqrt and division, subnormals kept:
 *   g     = grad (bf16 widened exactly, or the fp32 accumulator)
 *   w1    = w * decay                     decay     = fp32(1 - lr*wd)
 *   m'    = b1*m + omb1*g                 b1, omb1  = fp32(beta1), fp32(1-beta1)
 *   v'    = b2*v + omb2*(g*g)             b2, omb2  = fp32(beta2), fp32(1-beta2)
 *   d     = sqrt(v')*ibc2 + eps           ibc2      = fp32(1/sqrt(1-beta2^t))
 *   w'    = w1 - step*(m'/d)              step      = fp32(lr/(1-beta1^t))
 *   weight_bf16 = round-to-nearest-even bf16 of w'
 *   delta = w' - f32(orig)                (only when requested)
 * The constants are computed in double (beta^t by square-and-multiply, low
 * bit first) and rounded to fp32 once.
 *
 * Conventions for every call:
 *   - Arrays are 1-D, contiguous, little-endian; bf16 values are passed as
 *     their uint16 bit patterns.  Device pointers must be device memory (or
 *     memory the GPU can address) of the current HIP device.
 *   - fp32 pointers must be 4-byte aligned and bf16 pointers 2-byte aligned
 *     (else LEMA_ERR_ALIGN).  Any further alignment is optional; 16-byte
 *     aligned fp32 arrays and 8-byte aligned bf16 arrays take the vector path.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Compute calls are
 *     asynchronous on it; the caller keeps the arrays alive until it is done.
 *   - Every argument is validated before any HIP call: on any error nothing
 *     is enqueued and nothing is modified.  HIP failures return LEMA_ERR_HIP
 *     and lema_last_hip_error() gives the raw hipError_t of this thread.
 *   - Calls that launch kernels refuse a stream that is capturing a HIP
 *     graph (LEMA_ERR_CAPTURE, nothing enqueued): their launch tables live
 *     in a cache whose entries may be reused after the call, which a
 *     captured graph would outlive.  (A table of at most 2048 bytes of the
 *     fp32 step, accumulation and merge travels in the kernel arguments
 *     instead; those calls are refused as well, so that whether a call may
 *     be captured does not depend on its segment count.)
 *   - Nothing aborts, throws or prints across this ABI.
 *   - The caller owns all tensors, streams and the step counter t; the
 *     library is stateless apart from caches of small launch tables.
 */
#ifndef LEMA_H
#define LEMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------- statuses */

typedef int32_t lema_status;

#define LEMA_OK              0
#define LEMA_ERR_NULL       (-1)  /* a required pointer is NULL, or orig/delta unpaired */
#define LEMA_ERR_SIZE       (-2)  /* negative count/numel, or a size beyond a limit    */
#define LEMA_ERR_HPARAM     (-3)  /* hyperparameter or step out of range               */
#define LEMA_ERR_DTYPE      (-4)  /* unknown gradient dtype                            */
#define LEMA_ERR_OVERLAP    (-5)  /* two arrays overlap where one of them is written   */
#define LEMA_ERR_NOT_PINNED (-6)  /* host memory is not page-locked                    */
#define LEMA_ERR_HIP        (-7)  /* the HIP runtime reported an error                 */
#define LEMA_ERR_ALIGN      (-8)  /* pointer not aligned to its element size           */
#define LEMA_ERR_CAPTURE    (-9)  /* the stream is capturing a HIP graph               */
#define LEMA_ERR_IO         (-10) /* a checkpoint file could not be read or written,   */
                                  /* or is not a well-formed safetensors file          */
#define LEMA_ERR_NOT_FOUND  (-11) /* a requested tensor is not in the checkpoint file  */

/* Static string naming a status (never NULL). */
const char *lema_status_string(lema_status s);

/* hipError_t of the last LEMA_ERR_HIP returned on the calling thread, else 0. */
int32_t lema_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t lema_version(void);

/* --------------------------------------------------------------- AdamW */

typedef enum {
    LEMA_GRAD_BF16 = 0,  /* grad is bf16 bit patterns (one micro-batch)   */
    LEMA_GRAD_FP32 = 1,  /* grad is an fp32 accumulator (lema_grad_accum) */
    LEMA_GRAD_Q8   = 2   /* grad is an int8 accumulator with row scales
                            (lema_grad_accum_q8); lema_adamw_step_q8 only  */
} lema_grad_dtype;

/*
 * One trainable tensor (one "addressable segment" of the LEMA README intro).
 * Every array has `numel` elements.  master, exp_avg and exp_avg_sq are
 * updated in place; no other two arrays of any segment in a call may
 * overlap (LEMA_ERR_OVERLAP).
 */
typedef struct {
    float          *master;      /* fp32 master weight, in/out (required)        */
    float          *exp_avg;     /* m, fp32, in/out (required)                   */
    float          *exp_avg_sq;  /* v, fp32, in/out (required)                   */
    const void     *grad;        /* bf16 bits or fp32 accumulator, in (required) */
    uint16_t       *weight_bf16; /* out: bf16 of the new master (required)       */
    const uint16_t *orig_bf16;   /* in: base weight; non-NULL iff delta non-NULL */
    float          *delta;       /* out: new master - f32(orig) (optional)       */
    int64_t         numel;       /* >= 0; 0 makes the segment a no-op            */
} lema_adamw_seg;

/* Hyperparameters of one call (one parameter group). */
typedef struct {
    double  lr;            /* >= 0                                        */
    double  beta1;         /* 0 <= beta1 < 1                              */
    double  beta2;         /* 0 <= beta2 < 1                              */
    double  eps;           /* > 0                                         */
    double  weight_decay;  /* >= 0 (decoupled)                            */
    int64_t step;          /* t >= 1: the number of the step being taken  */
    int32_t grad_dtype;    /* lema_grad_dtype, one per call               */
    int32_t reserved;      /* must be 0                                   */
} lema_adamw_args;

/* The fp32 constants one call uses (see the arithmetic above). */
typedef struct {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float eps, decay, step_size, inv_bias_correction2_root;
} lema_adamw_consts;

/*
 * Derive the fp32 constants for `args` (host only, no GPU needed).
 * Errors: LEMA_ERR_NULL, LEMA_ERR_HPARAM, LEMA_ERR_DTYPE.
 */
lema_status lema_adamw_constants(const lema_adamw_args *args, lema_adamw_consts *out);

/*
 * One AdamW step over `nseg` segments (LEMA README, "Quick Start" and
 * "Selective Full Fine-Tuning": the per-layer AdamW over fp32 states; the
 * LLMScale page's 16-byte layout; the checkpoint delta of "Selective Full
 * Fine-Tuning").  Elementwise and asynchronous on `stream`.
 *   segs : host array of nseg descriptors holding device pointers; it is
 *          read during the call only.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_HPARAM, LEMA_ERR_DTYPE,
 *         LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP, LEMA_ERR_HIP.
 */
lema_status lema_adamw_step(const lema_adamw_seg *segs, int32_t nseg,
                            const lema_adamw_args *args, void *stream);

/*
 * lema_adamw_step for callers that cannot allocate memory: code that must
 * not call hipMalloc (tight serving or training loops, harnesses that
 * forbid allocation).  Same arguments, kernels and results as
 * lema_adamw_step, but nothing is allocated on the device or the host: the
 * launch table goes into a fixed array of device memory that each GPU holds
 * from the library's first use there until the process ends (table bytes of
 * LEMA_NOALLOC_MAX_SEGMENTS segments, about 84 KiB), written through kernel
 * arguments on `stream` ahead of the step.
 *   nseg : at most LEMA_NOALLOC_MAX_SEGMENTS (else LEMA_ERR_SIZE, nothing
 *          enqueued)
 * Every call on one GPU overwrites that GPU's array.  Calls on one stream
 * are ordered; calls that overlap on one GPU from different streams race
 * for the array (undefined results), so such callers serialize them.  A
 * capturing stream is refused (LEMA_ERR_CAPTURE), as for the other calls.
 * Errors: as lema_adamw_step.
 */
#define LEMA_NOALLOC_MAX_SEGMENTS 1024
lema_status lema_adamw_step_noalloc(const lema_adamw_seg *segs, int32_t nseg,
                                    const lema_adamw_args *args, void *stream);

/*
 * The step on an fp32 accumulator with the last micro-batch folded in:
 * per element g = acc + f32(last), the same fp32 addition lema_grad_accum
 * performs, so the results are bit-identical to lema_grad_accum(last) followed
 * by lema_adamw_step on the accumulator, while the accumulator is only read
 * (it is not updated).  It saves one pass over the accumulator (LEMA README,
 * "Selective Full Fine-Tuning": fp32 gradient accumulation feeding the
 * per-layer AdamW step).
 *   segs        : as for lema_adamw_step; segs[i].grad is the fp32 accumulator
 *   last_bf16   : host array of nseg device pointers; last_bf16[i] holds the
 *                 bf16 bits of segment i's last micro-batch (numel elements)
 *   args        : args->grad_dtype must be LEMA_GRAD_FP32 (else LEMA_ERR_DTYPE)
 * Errors: as lema_adamw_step.
 */
lema_status lema_adamw_step_accum(const lema_adamw_seg *segs, const uint16_t *const *last_bf16,
                                  int32_t nseg, const lema_adamw_args *args, void *stream);

/*
 * The step on the fp32 sum of K bf16 micro-batch gradients that are all
 * resident at once: per element g = f32(g_1), then g = g + f32(g_k) for
 * k = 2..K in order, the additions lema_grad_accum performs, so the results
 * are bit-identical to K lema_grad_accum calls (the first overwriting)
 * followed by lema_adamw_step on the accumulator (LEMA README, "Selective
 * Full Fine-Tuning": fp32 gradient accumulation feeding the per-layer AdamW
 * step).  The sum stays in registers: no accumulator array is read or
 * written, so one call moves 2K + 26 B per parameter (2K + 32 with delta)
 * instead of the 10 B per micro-batch and extra accumulator read of the
 * separate calls.  For callers that keep the micro-batch gradients.
 *   segs  : as for lema_adamw_step, with segs[i].grad NULL (LEMA_ERR_NULL
 *           otherwise)
 *   grads : host array of nseg * nmb device pointers; grads[i * nmb + k] is
 *           the bf16 gradient of micro-batch k + 1 for segment i
 *   nmb   : K, 1 .. LEMA_MAX_MICROBATCHES (else LEMA_ERR_SIZE)
 *   args  : args->grad_dtype must be LEMA_GRAD_BF16 (else LEMA_ERR_DTYPE)
 * Errors: as lema_adamw_step.
 */
#define LEMA_MAX_MICROBATCHES 16
lema_status lema_adamw_step_microbatches(const lema_adamw_seg *segs,
                                         const uint16_t *const *grads, int32_t nseg,
                                         int32_t nmb, const lema_adamw_args *args,
                                         void *stream);

/* ------------------------------------------------ gradient accumulation */

/* One accumulator and the bf16 micro-batch gradient added into it. */
typedef struct {
    float          *acc;        /* fp32 accumulator, in/out (required) */
    const uint16_t *grad_bf16;  /* bf16 bits, in (required)            */
    int64_t         numel;      /* >= 0                                */
} lema_accum_seg;

/*
 * fp32 gradient accumulation of one bf16 micro-batch (LEMA README,
 * "Selective Full Fine-Tuning": gradient accumulation is fp32):
 *   overwrite = 1 : acc = f32(g)        (first micro-batch; -0 kept)
 *   overwrite = 0 : acc = acc + f32(g)  (later micro-batches, in order)
 * A plain sum: any 1/K averaging belongs in the loss scale.  Asynchronous on
 * `stream`.  Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_ALIGN,
 * LEMA_ERR_OVERLAP, LEMA_ERR_HIP.
 */
lema_status lema_grad_accum(const lema_accum_seg *segs, int32_t nseg,
                            int32_t overwrite, void *stream);

/* ----------------------------------------------------------- merge delta */

/* One tensor of a merge: base checkpoint weight, saved delta, output. */
typedef struct {
    const uint16_t *base_bf16;    /* bf16 bits of the base weight, in (required) */
    const float    *delta;        /* fp32 delta (updated - original), in (required) */
    uint16_t       *merged_bf16;  /* out: the servable bf16 weight (required)     */
    int64_t         numel;        /* >= 0                                         */
} lema_merge_seg;

/*
 * Servable weights from a base checkpoint and a saved delta (LEMA README,
 * "Selective Full Fine-Tuning": merge_delta(base, delta, merged)):
 *   merged = bf16 round-to-nearest-even of (f32(base) + delta)
 * one binary32 addition per element.  Merging the delta a step wrote next to
 * its bf16 weight reproduces that weight.  The file I/O of the original tool
 * is the caller's.  Asynchronous on `stream`.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP,
 * LEMA_ERR_HIP.
 */
lema_status lema_merge_delta(const lema_merge_seg *segs, int32_t nseg, void *stream);

/* ------------------------------------------- int8 rows with row scales */

/*
 * Quantized optimizer moments and gradient accumulators (LEMA README,
 * "Quantization": the opt_state_bits and grad_acc_bits settings of 8 keep
 * Adam's moments and the gradient accumulators as int8 codes with a scale
 * per row, widened to fp32 only within the step).  The pages give no
 * formula; the format read here is
 * symmetric absmax scaling:
 *   - a tensor of numel elements is cut into rows of row_len consecutive
 *     elements, the last row possibly shorter: rows = ceil(numel / row_len)
 *     (row_len = in for a 2-D [out x in] weight gives its matrix rows);
 *   - row r stores int8 codes q in [-127, 127] and one fp32 scale s[r];
 *   - dequantize: x = f32(q) * s[r], one binary32 multiplication;
 *   - quantize  : a = largest |x| of the row (NaN if the row has a NaN),
 *                 s[r] = a / 127 (binary32 division); if s[r] is finite and
 *                 > 0, q = round-half-even(x / s[r]) (binary32 division)
 *                 clamped to [-127, 127], else every code of the row is 0.
 *                 An all-zero row stores s = 0; a row holding an infinity or
 *                 a NaN stores s = inf or NaN and dequantizes to NaN.
 * Scales are fp32 arrays of `rows` entries; codes are int8 arrays of numel.
 * row_len must lie in 1 .. LEMA_Q8_MAX_ROW (else LEMA_ERR_SIZE).  int8 arrays
 * need no alignment; 4-byte aligned codes, 16-byte aligned fp32 and 8-byte
 * aligned bf16 arrays with row_len a multiple of 4 take the vector path.
 */
#define LEMA_Q8_MAX_ROW 16384

typedef enum {
    LEMA_STATE_FP32 = 0,  /* exp_avg / exp_avg_sq are fp32 arrays         */
    LEMA_STATE_Q8   = 1   /* exp_avg / exp_avg_sq are int8 codes + scales */
} lema_state_dtype;

/*
 * One trainable tensor of lema_adamw_step_q8.  As lema_adamw_seg, plus the
 * row scales of every int8 array and the row length.  master, the moments
 * and their scales are updated in place; no two arrays may overlap where
 * one is written (LEMA_ERR_OVERLAP).
 */
typedef struct {
    float          *master;            /* fp32 master weight, in/out (required)     */
    void           *exp_avg;           /* m: int8 codes or fp32, in/out (required)   */
    float          *exp_avg_scale;     /* m's fp32 row scales, in/out (int8 m only)   */
    void           *exp_avg_sq;        /* v: int8 codes or fp32, in/out (required)   */
    float          *exp_avg_sq_scale;  /* v's row scales, in/out (int8 v only)       */
    const void     *grad;              /* bf16 bits, fp32 or int8 codes (required)   */
    const float    *grad_scale;        /* grad's row scales (LEMA_GRAD_Q8 only)      */
    uint16_t       *weight_bf16;       /* out: bf16 of the new master (required)     */
    const uint16_t *orig_bf16;         /* in: base weight; non-NULL iff delta is     */
    float          *delta;             /* out: new master - f32(orig) (optional)     */
    int64_t         numel;             /* >= 0; 0 makes the segment a no-op          */
    int64_t         row_len;           /* 1 .. LEMA_Q8_MAX_ROW when any array is int8 */
} lema_adamw_q8_seg;

/*
 * One AdamW step with quantized moments and/or a quantized gradient
 * accumulator (LEMA README, "Quantization": int8 state is widened to fp32
 * within the step and nowhere else).  Per row:
 *   m, v  = dequantized moments (moment_dtype LEMA_STATE_Q8) or the fp32 ones
 *   g     = bf16 widened, the fp32 accumulator, or the dequantized int8 one
 *   the fp32 step of lema_adamw_step, element for element (same arithmetic,
 *   same master, bf16 weight and delta outputs), then for int8 moments the
 *   new m and v are quantized with fresh row scales.
 *   segs        : host array of nseg descriptors (device pointers), read
 *                 during the call only
 *   args        : args->grad_dtype is LEMA_GRAD_BF16, LEMA_GRAD_FP32 or
 *                 LEMA_GRAD_Q8
 *   moment_dtype: lema_state_dtype, for every segment of the call
 * With fp32 moments and a bf16 or fp32 gradient this is lema_adamw_step.
 * Asynchronous on `stream`.  Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE,
 * LEMA_ERR_HPARAM, LEMA_ERR_DTYPE, LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP,
 * LEMA_ERR_HIP.
 */
lema_status lema_adamw_step_q8(const lema_adamw_q8_seg *segs, int32_t nseg,
                               const lema_adamw_args *args, int32_t moment_dtype, void *stream);

/* One int8 gradient accumulator and the bf16 micro-batch added into it. */
typedef struct {
    int8_t         *acc;        /* int8 codes, in/out (required)            */
    float          *acc_scale;  /* row scales, in/out (required)            */
    const uint16_t *grad_bf16;  /* bf16 bits, in (required)                 */
    int64_t         numel;      /* >= 0                                     */
    int64_t         row_len;    /* 1 .. LEMA_Q8_MAX_ROW                     */
} lema_accum_q8_seg;

/*
 * int8 gradient accumulation of one bf16 micro-batch (LEMA README,
 * "Quantization": grad_acc_bits = 8):
 *   overwrite = 1 : acc = Q(f32(g))                (first micro-batch)
 *   overwrite = 0 : acc = Q(D(acc) + f32(g))       (later ones, in order)
 * with D and Q the dequantization and quantization above and one binary32
 * addition per element.  Asynchronous on `stream`.  Errors: LEMA_ERR_NULL,
 * LEMA_ERR_SIZE, LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP, LEMA_ERR_HIP.
 */
lema_status lema_grad_accum_q8(const lema_accum_q8_seg *segs, int32_t nseg,
                               int32_t overwrite, void *stream);

/* One tensor converted between fp32 and int8 codes with row scales. */
typedef struct {
    float   *x;        /* fp32 values (required)             */
    int8_t  *codes;    /* int8 codes (required)              */
    float   *scale;    /* ceil(numel/row_len) scales (required) */
    int64_t  numel;    /* >= 0                               */
    int64_t  row_len;  /* 1 .. LEMA_Q8_MAX_ROW               */
} lema_q8_tensor;

/*
 * Convert whole tensors: lema_quantize_rows reads x and writes codes and
 * scales; lema_dequantize_rows reads codes and scales and writes x.  They
 * set up and inspect quantized state (fp32 moments of a checkpoint into the
 * int8 classes and back).  Asynchronous on `stream`.  Errors: LEMA_ERR_NULL,
 * LEMA_ERR_SIZE, LEMA_ERR_ALIGN, LEMA_ERR_OVERLAP, LEMA_ERR_HIP.
 */
lema_status lema_quantize_rows(const lema_q8_tensor *t, int32_t n, void *stream);
lema_status lema_dequantize_rows(const lema_q8_tensor *t, int32_t n, void *stream);

/* --------------------------------------- slot-pool streaming (host RAM) */

/*
 * The TensorStore of the LEMA README ("TensorStore: Unified Streaming Core";
 * "Selective Full Fine-Tuning": fp32 optimizer states live in RAM), reduced
 * to two tiers: page-locked host RAM and a pool of HBM slots.  Each layer's
 * master, m, v and bf16 gradient are copied host->HBM into a slot, the AdamW
 * step runs there, and master, m, v and the bf16 weight are copied back to
 * the layer's host arrays, with the copy of the next layer overlapping the
 * step of the current one.
 */
typedef struct lema_slot_pool lema_slot_pool;

/*
 * Create a pool over a caller-owned device region of nslots * slot_bytes
 * bytes (borrowed, not freed by the library).  copy_stream carries every
 * host<->HBM copy, compute_stream every kernel; they must differ.  nslots
 * must be >= 2.  The pool owns only HIP events and small table buffers.
 * Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE, LEMA_ERR_HIP.
 */
lema_status lema_slot_pool_create(void *device_base, size_t slot_bytes, int32_t nslots,
                                  void *copy_stream, void *compute_stream,
                                  lema_slot_pool **out);

/*
 * Optional: carry the slot -> host copies on their own stream, so that both
 * PCIe directions are busy at once (the upload of layer i+1 runs beside the
 * write-back of layer i).  NULL restores the single copy stream.  The stream
 * must differ from the pool's copy and compute streams (else LEMA_ERR_NULL).
 */
lema_status lema_slot_pool_set_writeback_stream(lema_slot_pool *pool, void *stream);

/* Destroy a pool (waits for its outstanding work).  NULL is a no-op. */
lema_status lema_slot_pool_destroy(lema_slot_pool *pool);

/*
 * One layer of host-resident state.  In each host_segs entry the pointers
 * are page-locked HOST pointers (lema_host_alloc): master, exp_avg,
 * exp_avg_sq, grad (bf16 only) are read and master, exp_avg, exp_avg_sq,
 * weight_bf16 are written back; orig_bf16 and delta must be NULL.
 */
typedef struct {
    const lema_adamw_seg *host_segs;
    int32_t               nseg;
} lema_layer;

typedef struct {
    double h2d_bytes, d2h_bytes;  /* bytes copied in each direction         */
    double h2d_ms, d2h_ms;        /* summed copy durations, per layer and direction */
    double kernel_ms;             /* summed AdamW kernel durations          */
    double copy_busy_ms;          /* time at least one copy was running     */
    double wall_ms;               /* first copy start .. last copy end      */
    double last_kernel_ms;        /* duration of the last layer's kernel    */
    double host_in_ms;            /* staged only: host copies into the upload ring   */
    double host_out_ms;           /* staged only: host copies out of the write-back ring */
    double call_ms;               /* host clock over the whole call         */
} lema_stream_stats;

/*
 * Stream `nlayers` layers through the pool with one AdamW step each (bf16
 * gradients, args->grad_dtype must be LEMA_GRAD_BF16).  Layer i uses slot
 * i mod nslots.  Blocks until the last copy back has completed.  `stats`
 * may be NULL.  Errors: LEMA_ERR_NULL, LEMA_ERR_SIZE (a layer does not fit a
 * slot), LEMA_ERR_HPARAM, LEMA_ERR_DTYPE, LEMA_ERR_ALIGN,
 * LEMA_ERR_NOT_PINNED, LEMA_ERR_HIP.  Every argument error is found before
 * the first copy, and then nothing is enqueued.  A HIP failure after copies
 * began returns only once the pool's streams have finished what was already
 * enqueued; the host state then holds some layers stepped, some not, and
 * possibly one layer partly written back.  (Test hook: with the environment
 * variable LEMA_FAULT_INJECT=copy:<n>, the n-th copy a streaming call would
 * enqueue fails with hipErrorUnknown instead, from the host.)
 */
lema_status lema_slot_stream(lema_slot_pool *pool, const lema_layer *layers, int32_t nlayers,
                             const lema_adamw_args *args, lema_stream_stats *stats);

/*
 * lema_slot_stream for host state that is not page-locked: ordinary memory or
 * a memory-mapped file (the disk tier of the LEMA README's "Triple-Buffer
 * Pipeline: Disk -> pinned RAM -> VRAM"; "Selective Full Fine-Tuning": fp32
 * states in RAM with an mmap disk backend).  A layer's arrays move in pieces
 * of at most 128 MiB, each a span of the slot that holds arrays adjacent
 * there (one copy between slot and ring, one host copy per array part):
 *   caller memory -> page-locked upload ring -> slot[i mod nslots]
 *   slot[i mod nslots] -> page-locked write-back ring -> caller memory
 * The two rings (16 chunks of 128 MiB each, 4 GiB in all) are allocated by
 * the pool on first use and freed with it.  `host_threads` host threads
 * (0 = up to 16), split between the two directions, do the copies between
 * the caller's memory and the rings, piece by piece, so that a layer's first
 * upload starts after one piece's host copy and a write-back's host copies
 * follow its DMA.  The calling thread enqueues the uploads and steps; a
 * second thread of the library (on the pool's device) enqueues the
 * write-backs and copies them out.  A HIP failure on either thread returns
 * LEMA_ERR_HIP with its raw code in the calling thread's
 * lema_last_hip_error().
 * On a single copy stream each layer's write-back is enqueued after the next
 * layer's uploads.  Blocks until every layer is written back.  In `stats`,
 * as for lema_slot_stream, copy times are per layer and direction (first
 * piece's start to last piece's end); a wait for the host inside a layer's
 * transfer shows as a lower h2d/d2h rate, not as uncovered time.
 * Same arguments and errors as lema_slot_stream, except that host memory need
 * not be page-locked (no LEMA_ERR_NOT_PINNED); LEMA_ERR_SIZE also for
 * host_threads outside 0..256.
 */
lema_status lema_slot_stream_staged(lema_slot_pool *pool, const lema_layer *layers,
                                    int32_t nlayers, const lema_adamw_args *args,
                                    int32_t host_threads, lema_stream_stats *stats);

/*
 * One layer of host-resident state for lema_slot_stream_q8: int8 moments
 * with row scales and/or an int8 gradient accumulator, kept quantized in
 * host memory.  Every array named by a segment is a host pointer; orig_bf16
 * and delta must be NULL.
 */
typedef struct {
    const lema_adamw_q8_seg *host_segs;
    int32_t                  nseg;
} lema_layer_q8;

/*
 * The slot-pool streaming of lema_slot_stream / lema_slot_stream_staged for
 * quantized host state (LEMA README, "Quantization": host memory, and the
 * memory-mapped disk tier, hold int8 codes and row scales, which are widened
 * to fp32 only on the GPU within the step).  Per segment, the
 * master, the moments (int8 codes and row scales, or fp32) and the gradient
 * (bf16, fp32, or int8 codes and row scales) are copied in, the step of
 * lema_adamw_step_q8 runs on the slot, and the master, the moments and
 * their scales and the bf16 weight are copied back.  With int8 moments and
 * a bf16 gradient that is 8 B per parameter each way instead of 14.
 *   moment_dtype : lema_state_dtype of every segment
 *   staged       : 0 = host arrays are page-locked and copied directly
 *                  (LEMA_ERR_NOT_PINNED otherwise); 1 = any host memory,
 *                  moved through the pool's page-locked rings by
 *                  `host_threads` threads (0 = up to 16)
 * args->grad_dtype may be LEMA_GRAD_BF16, LEMA_GRAD_FP32 or LEMA_GRAD_Q8.
 * Errors: as lema_slot_stream, plus LEMA_ERR_DTYPE for an unknown
 * moment_dtype and LEMA_ERR_SIZE for a row length outside 1..LEMA_Q8_MAX_ROW
 * or host_threads outside 0..256.
 */
lema_status lema_slot_stream_q8(lema_slot_pool *pool, const lema_layer_q8 *layers,
                                int32_t nlayers, const lema_adamw_args *args,
                                int32_t moment_dtype, int32_t staged, int32_t host_threads,
                                lema_stream_stats *stats);

/* Page-locked host allocation of exactly `bytes` bytes (hipHostMalloc). */
lema_status lema_host_alloc(void **out, size_t bytes);
lema_status lema_host_free(void *p);

/* ----------------------------------------------------------- checkpoints
 *
 * LEMA README, "Features" (interval-based automatic checkpointing of the
 * full fine-tuning delta with the optimizer states) and "Selective Full
 * Fine-Tuning" (a checkpoint holds the small fp32 delta, updated minus
 * original, plus the optimizer state; training resumes from it, and
 * merge_delta turns a base model and a delta file into a servable one).
 *
 * A checkpoint file is a safetensors file, the format of the pages'
 * checkpoints and of merge_delta: an 8-byte little-endian header length N,
 * N bytes of JSON naming every tensor with its dtype ("F32", "BF16" or
 * "I8"), its 1-D shape [numel] and its byte range [begin, end) in the data
 * that follows, padded with spaces to a multiple of 8; then the tensors'
 * bytes back to back, in the order given.  The JSON's "__metadata__" object
 * holds {"format": "lema-checkpoint", "step": "<t>"}, t being the last step
 * taken.  Which tensors to store is the caller's choice: the fp32 master, m
 * and v (or their int8 codes and row scales) for a bit-exact resume, the
 * delta for merge_delta.
 *
 * Both calls are synchronous: they copy between the tensors and the file
 * through page-locked staging buffers on `stream` (the copies overlap the
 * file reads and writes) and return once the data has arrived, having
 * synchronized `stream`.  Tensors may be in device memory or in host memory,
 * so the host-resident state of a streamed run is checkpointed in place.
 * They refuse a capturing stream (LEMA_ERR_CAPTURE).
 */
typedef enum { LEMA_DT_F32 = 0, LEMA_DT_BF16 = 1, LEMA_DT_I8 = 2 } lema_dtype;

typedef struct {
    const char *name;     /* 1 .. 255 bytes of printable ASCII other than the  */
                          /* double quote and the backslash; unique in a call  */
    int32_t     dtype;    /* lema_dtype                                         */
    int32_t     reserved; /* 0                                                  */
    void       *data;     /* read by save, written by load: device memory, or  */
                          /* host memory (page-locked or not: the state of a   */
                          /* streamed run lives there); NULL only if numel == 0 */
    int64_t     numel;    /* >= 0                                               */
} lema_ckpt_tensor;

/* Writes the n tensors and the step t to `path`.  The file is written under
 * a temporary name of its own in the same directory (`path` + ".tmp." and a
 * unique suffix), flushed to storage and then renamed over `path`, so a save
 * that fails leaves an earlier file at `path` intact and removes its
 * temporary file, and concurrent saves to one path each leave a whole file
 * (the last rename wins).
 * Errors: LEMA_ERR_NULL (path, t with n > 0, a name, or data with numel > 0),
 * LEMA_ERR_SIZE (n < 0, numel < 0, a bad or repeated name, reserved != 0),
 * LEMA_ERR_DTYPE, LEMA_ERR_CAPTURE, LEMA_ERR_IO, LEMA_ERR_HIP. */
lema_status lema_checkpoint_save(const char *path, const lema_ckpt_tensor *t, int32_t n,
                                 int64_t step, void *stream);

/* Reads the n named tensors of the safetensors file `path` into their device
 * buffers and its step into *step (-1 when the metadata holds no integer
 * step; step may be NULL).  Every requested tensor must be in the file with the same dtype
 * and element count; other tensors of the file are ignored, so files from
 * other writers load as long as they hold the requested names.  The whole
 * header is parsed and checked, and every request matched, before any
 * device memory is written.
 * Errors: as for lema_checkpoint_save, and LEMA_ERR_NOT_FOUND (a requested
 * name is not in the file), LEMA_ERR_DTYPE or LEMA_ERR_SIZE (it is, with
 * another dtype or element count), LEMA_ERR_IO (the file cannot be read, is
 * shorter than its header says, or its header is not valid safetensors
 * JSON).  Only a read or HIP error after all checks have passed can leave
 * the device buffers partly written. */
lema_status lema_checkpoint_load(const char *path, const lema_ckpt_tensor *t, int32_t n,
                                 int64_t *step, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LEMA_H */
