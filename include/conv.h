/*
 * conv.h — C ABI of the MI355X (gfx950) 2-D convolution forward library
 * (libconvfwd.so).
 *
 * Operation (ONNX Conv / ConvTranspose, as stated on "Convolution, pooling and
 * resize" (OneGpu docs), section "Layout and operands", and "Convolutions"
 * (ml-interview-book, part 4 ch. 2), sections 2.1, 2.3 and 2.5):
 *
 *   Conv:   y[n,co,oh,ow] = act( fl( fl( sum_{ci',kh,kw} x[n, g*Cin/G+ci', ih, iw]
 *                                         * w[co, ci', kh, kw] ) + b[co] ) + r[n,co,oh,ow] ) )
 *           ih = oh*stride_h - pad_top + kh*dil_h,  iw = ow*stride_w - pad_left + kw*dil_w,
 *           taps outside the input contribute zero; g = co / (Cout/G); no kernel flip.
 *           Ho = floor((H + pad_top + pad_bottom - dil_h*(KH-1) - 1) / stride_h) + 1.
 *   ConvTranspose: the adjoint scatter of Conv with the same geometry (each input value
 *           places a scaled copy of the kernel at stride s; overlaps add), computed as a
 *           GEMM into float32 columns followed by a gathering col2im (one thread per
 *           output element, no atomics).
 *           Ho = stride_h*(H-1) + out_pad_h + dil_h*(KH-1) + 1 - pad_top - pad_bottom.
 *
 * The epilogue runs in this order, each step rounded in float32: sum, bias,
 * residual addition, activation; a float16 output is then rounded to nearest even.
 *
 * Layouts (all dense, row-major, no padding between rows):
 *   x        NCHW  [n, c_in, h, w]
 *   w        Conv: OIHW [c_out, c_in/groups, kh, kw];
 *            ConvTranspose: [c_in, c_out/groups, kh, kw]
 *   bias     [c_out]                    (optional)
 *   residual same shape as y            (optional; may alias y exactly)
 *   y        NCHW  [n, c_out, Ho, Wo]
 * Element types: CONV_F32 (float32 everywhere), CONV_F16 or CONV_BF16 (16-bit
 * operands and output, float32 accumulation).  Every operand pointer is a base device pointer;
 * the element offsets in conv_problem are added to it (arena-style placement).
 *
 * Ownership and execution: device buffers belong to the caller.  conv_forward and
 * conv_transpose_forward only enqueue work on the given HIP stream (NULL = the
 * default stream); they never synchronise, allocate or free.  The caller keeps every
 * buffer alive until the stream has finished the work.
 *
 * Errors: every shape, argument, overlap and scratch check runs on the host before
 * anything is enqueued; on error nothing is enqueued and a non-zero status returns.
 * Only CONV_ERR_DEVICE (a launch the runtime refused) can follow partial enqueueing.
 *
 * Threading: all calls are reentrant; the library holds no mutable global state.
 */
#ifndef CONVFWD_CONV_H
#define CONVFWD_CONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    CONV_OK = 0,
    CONV_ERR_ARG = 1,     /* null required pointer, bad enum, transpose flag mismatch,
                             misaligned scratch, a variant override that cannot run */
    CONV_ERR_SHAPE = 2,   /* dims < 1, channels not divisible by groups, stride or
                             dilation < 1, pads < 0, output extent < 1, output padding
                             outside [0, stride), int64 overflow, an operand above
                             2^31-1 elements, grid beyond device limits */
    CONV_ERR_OVERLAP = 3, /* scratch overlaps an operand; y overlaps x, w or bias;
                             y overlaps the residual other than exactly */
    CONV_ERR_SCRATCH = 4, /* scratch smaller than one image's need */
    CONV_ERR_DEVICE = 5   /* the HIP runtime refused a launch */
};

/* Element type of x, w, bias, residual and y ("Convolution, pooling and resize",
 * "Layout and operands": float, and half in and out with float32 accumulation).
 * CONV_BF16 is bfloat16 in and out with float32 accumulation, the same kernels
 * as float16 with the bfloat16 MFMA instructions (no page fixes a bfloat16
 * tolerance; the library's tests hold it to 1.6e-2 * sum|w*x|). */
typedef enum { CONV_F32 = 0, CONV_F16 = 1, CONV_BF16 = 2 } conv_dtype;

/* Fused activations (the list of "Layout and operands"), ONNX definitions:
 * relu max(0,v); tanh; sigmoid 1/(1+e^-v); silu v*sigmoid(v);
 * hard_sigmoid clamp(alpha*v+beta, 0, 1); hard_swish v*clamp(v/6+1/2, 0, 1);
 * clip clamp(v, alpha, beta); leaky_relu v >= 0 ? v : alpha*v. */
typedef enum {
    CONV_ACT_IDENTITY = 0,
    CONV_ACT_RELU = 1,
    CONV_ACT_TANH = 2,
    CONV_ACT_SIGMOID = 3,
    CONV_ACT_SILU = 4,
    CONV_ACT_HARD_SIGMOID = 5,
    CONV_ACT_HARD_SWISH = 6,
    CONV_ACT_CLIP = 7,
    CONV_ACT_LEAKY_RELU = 8
} conv_activation;

/* ONNX auto_pad modes. */
typedef enum {
    CONV_AUTO_PAD_NOTSET = 0,
    CONV_AUTO_PAD_SAME_UPPER = 1,
    CONV_AUTO_PAD_SAME_LOWER = 2,
    CONV_AUTO_PAD_VALID = 3
} conv_auto_pad;

/* Kernel variants ("Variants" table of the OneGpu page, re-designed for gfx950).
 * AUTO lets the planner choose from the shape and dtype alone. */
typedef enum {
    CONV_VARIANT_AUTO = 0,
    CONV_VARIANT_IMPLICIT_GEMM = 1,     /* generic implicit GEMM, window gathered per k-block */
    CONV_VARIANT_POINTWISE_GEMM = 2,    /* 1x1, stride 1, no pad: GEMM on x as it lies */
    CONV_VARIANT_DEPTHWISE_DIRECT = 3,  /* one input channel per group, direct, no MFMA */
    CONV_VARIANT_TRANSPOSE_GEMM_COL2IM = 4, /* ConvTranspose: GEMM + gathering col2im */
    CONV_VARIANT_IMPLICIT_GEMM_HALO = 5, /* implicit GEMM with the input halo tile staged
                                            once per channel chunk and reused for all taps;
                                            its row-shift path splits k itself when its
                                            grid fills at most half the compute units */
    CONV_VARIANT_IMPLICIT_GEMM_ROWBAND = 6, /* stride 2, few input channels (image stems):
                                              a ring of staged input rows per output-row
                                              band, kw taps read as consecutive halves */
    CONV_VARIANT_IMPLICIT_GEMM_GROUPED = 7, /* 8 input channels per group: the group's
                                              padded planes staged whole, one workgroup
                                              per (image, group) */
    CONV_VARIANT_WINOGRAD = 8  /* Winograd F(2x2, 3x3) ("Convolutions", section 2.6):
                                  3x3, stride 1, dilation 1, 16-bit operands, input
                                  channels per group a multiple of 16.  Never chosen by
                                  AUTO: its transformed operands are rounded to 16 bits,
                                  which adds rounding of cross terms that the direct sum
                                  does not have, so its error is not bounded by
                                  tol * sum|w*x| for every input (it meets the bound on
                                  the tests' distributions).  Needs scratch for the
                                  transformed weights, 16 * c_out * c_in/groups * 2 bytes,
                                  whatever the batch (conv_scratch_size reports it as
                                  both figures; no image chunking). */
} conv_variant;

/* The problem: shape, explicit pads, stride, dilation, groups, fused activation
 * and element offsets ("Layout and operands": ConvProblem / ConvTransposeProblem). */
typedef struct conv_problem {
    int64_t n, c_in, h, w;          /* input NCHW */
    int64_t c_out;                  /* output channels */
    int64_t kh, kw;                 /* kernel extent */
    int64_t groups;
    int64_t stride_h, stride_w;
    int64_t dil_h, dil_w;
    int64_t pad_top, pad_left, pad_bottom, pad_right; /* explicit, >= 0 */
    int64_t out_pad_h, out_pad_w;   /* ConvTranspose output_padding, in [0, stride) */
    int64_t x_off, w_off, b_off, r_off, y_off; /* element offsets added to the pointers */
    int32_t transpose;              /* 0 Conv, 1 ConvTranspose */
    int32_t activation;             /* conv_activation */
    float act_alpha, act_beta;      /* hard_sigmoid alpha/beta; clip lo/hi; leaky alpha */
    int32_t has_bias, has_residual; /* 0/1: whether bias / residual are applied */
    int32_t variant_override;       /* conv_variant; 0 = AUTO; others force a variant
                                       (CONV_ERR_ARG if it cannot run the shape) */
    int32_t split_override;         /* split-k ranges; 0 = AUTO, 1 = whole k, R > 1 forces R.
                                       The halo variant splits only on its row-shift
                                       path (3x3 stride 1, rows of at most 14 outputs)
                                       and only into R equal ranges of whole 64-channel
                                       stages (CONV_ERR_ARG otherwise); under AUTO a
                                       forced R that no row-shift split allows goes to
                                       the generic implicit GEMM. */
} conv_problem;

/* Output extent (the OutputExtent / TransposeOutputExtent analog): writes Ho, Wo.
 * Pure host; never touches the device.  Returns CONV_OK or CONV_ERR_SHAPE/ARG. */
int conv_output_extent(const conv_problem* p, int64_t* ho, int64_t* wo);

/* Resolve ONNX auto_pad (and, for ConvTranspose, output_shape) into explicit pads,
 * written into *p (the WithAutoPad analog).  output_shape_hw may be NULL; when
 * given ({Ho, Wo}) it applies to ConvTranspose only.  Conv SAME_*: Ho = ceil(H/s),
 * total pad = max(0, (Ho-1)s + d(k-1) + 1 - H), SAME_UPPER puts the odd unit at the
 * end, SAME_LOWER at the begin; VALID zeroes the pads; NOTSET keeps them.
 * ConvTranspose: total = s(H-1) + out_pad + d(k-1) + 1 - Ho_requested (Ho_requested
 * defaults to s*H under SAME_*), SAME_UPPER puts the odd unit at the end, any other
 * mode with an output shape at the begin.  Pure host. */
int conv_resolve_auto_pad(conv_problem* p, int auto_pad, const int64_t* output_shape_hw);

/* Scratch the planned variant needs, in bytes, for the whole batch and for one
 * image ("Convolution, pooling and resize", "Layout and operands":
 * Scratch(problem, half) says how much a shape needs, nothing for the variants
 * that gather windows while they multiply).  Zero for the direct, pointwise and
 * unsplit implicit variants; R float32 partial planes per image when k is split
 * into R ranges ("Variants", split k); c_out*kh*kw*h*w float32 columns per image
 * for ConvTranspose other than kernel = stride = 2.  A scratch buffer between
 * the two runs the batch in chunks of whole images, which changes no bit of the
 * result.  Shape-only: the plan is made for gfx950's 256 compute units and
 * never queries the HIP runtime, so every device gets the same answer. */
int conv_scratch_size(const conv_problem* p, int dtype, uint64_t* bytes_whole_batch,
                      uint64_t* bytes_per_image);

/* Name of the variant the planner picks ("Convolution, pooling and resize",
 * "Variants": DescribeVariant names what a device runs), NUL-terminated, e.g.
 * "implicit_gemm_halo.f16.rowshift.r14.n32", "depthwise_direct.f32.wave.col14".
 * Shape-only (no HIP runtime call; the same string on every device).  Returns
 * CONV_ERR_ARG when len is too small, or the validation status of the problem. */
int conv_describe_variant(const conv_problem* p, int dtype, char* buf, uint64_t len);

/* Conv forward: the cross-correlation above with the fused epilogue
 * ("Convolution, pooling and resize", "Layout and operands": operands are
 * buffers plus element offsets, the epilogue is sum, bias, residual,
 * activation, each rounded in float32; "Variants": the layer class picks the
 * kernel; "Convolutions" sections 2.1 and 2.4: output size, convolution as a
 * matrix product with the window gathered, never unfolded into a column
 * matrix).  x, w, y are required device pointers; bias and residual are read
 * only when has_bias / has_residual are set (then they are required).  scratch
 * may be NULL when conv_scratch_size reports zero; it must be 16-byte aligned and
 * must not overlap any operand.  stream is a hipStream_t (NULL = default stream).
 * Requires p->transpose == 0.  Asynchronous: returns once the work is enqueued.
 * Errors: CONV_ERR_ARG / SHAPE / OVERLAP / SCRATCH before anything is enqueued;
 * CONV_ERR_DEVICE if the runtime refuses a launch. */
int conv_forward(const conv_problem* p, int dtype, const void* x, const void* w,
                 const void* bias, const void* residual, void* y, void* scratch,
                 uint64_t scratch_bytes, void* stream);

/* ConvTranspose forward ("Convolution, pooling and resize", "Variants": the
 * product of the transposed weights with the input, then a gathering col2im, one
 * thread per output element and no atomics, with the same epilogue;
 * "Convolutions" section 2.5 and section 6: the adjoint scatter of Conv and the
 * output_padding that picks among the stride's preimages).  Same contract as
 * conv_forward, with p->transpose == 1, w in [c_in, c_out/groups, kh, kw] layout,
 * and scratch for the float32 columns when conv_scratch_size reports any (kernel
 * = stride = 2 without padding needs none: each output takes exactly one tap). */
int conv_transpose_forward(const conv_problem* p, int dtype, const void* x, const void* w,
                           const void* bias, const void* residual, void* y, void* scratch,
                           uint64_t scratch_bytes, void* stream);

/* Pre-flight ("Convolution, pooling and resize", "Layout and operands": sizes
 * are checked before anything is recorded, and a scratch range may share the
 * operands' arena only where it overlaps none of them): runs every check
 * conv_forward (p->transpose == 0) or conv_transpose_forward (p->transpose == 1)
 * would run on these arguments (shape, enums, pointers, overlap, scratch) and
 * returns the status that call would return before enqueueing, without
 * enqueueing or any HIP runtime call.  Pointers are compared, never read. */
int conv_check(const conv_problem* p, int dtype, const void* x, const void* w,
               const void* bias, const void* residual, const void* y, const void* scratch,
               uint64_t scratch_bytes);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  conv_forward (p->transpose == 0) or conv_transpose_forward
 * (p->transpose == 1) with the same arguments except the scratch: the split-k
 * planes and ConvTranspose columns live in a 64 MiB array the library holds per
 * GPU (a device global, kept until the process ends), so the call allocates
 * nothing and gives the same bits as those calls.  A batch whose scratch need
 * exceeds 64 MiB runs in chunks of whole images (same bits); a problem whose
 * one image needs more than 64 MiB returns CONV_ERR_SCRATCH before anything is
 * enqueued.  Every call on one GPU shares that GPU's array and every kernel
 * that uses it writes all of it that it reads, so nothing needs clearing; two
 * calls that overlap in time on one GPU (different streams, or different host
 * threads) race on it and must be serialised by the caller.  The first call on
 * a device resolves the array's address there (CONV_ERR_DEVICE if that fails). */
int conv_forward_noalloc(const conv_problem* p, int dtype, const void* x, const void* w,
                         const void* bias, const void* residual, void* y, void* stream);

/* Static, human-readable text for a status code (the shape errors are the
 * GpuKernelShapeException analog of "Convolution, pooling and resize",
 * "Layout and operands": raised before anything is recorded). */
const char* conv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_CONV_H */
