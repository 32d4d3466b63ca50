/*
 * pool.h — C ABI of the MI355X (gfx950) pooling forward (libconvfwd.so, beside
 * the convolution of conv.h, whose status codes and element types it shares).
 *
 * Operations ("Convolution, pooling and resize" (OneGpu docs), section "Pooling
 * and resize"; ONNX MaxPool, AveragePool, GlobalMaxPool, GlobalAveragePool):
 *
 *   window of output (n, c, oh, ow): taps ih = oh*stride_h - pad_top + kh*dil_h,
 *   iw = ow*stride_w - pad_left + kw*dil_w for kh < KH, kw < KW.  A tap is real
 *   inside the input, a padding tap inside the pads, and beyond the padding
 *   otherwise (only in ceil mode).
 *   MaxPool:     the largest real tap; NaN taps are skipped unless every real tap
 *                is NaN (then NaN); +0 counts as larger than -0; a window with no
 *                real tap gives the lowest finite value of the element type
 *                (-3.4028235e38 float, -65504 half, -3.3895314e38 bfloat16).
 *                Bit-exact: the result is one of the inputs (or that constant).
 *   AveragePool: the float32 sum of the real taps in (kh, kw) row-major order
 *                divided by the count of real taps, plus the padding taps when
 *                count_include_pad is set (taps beyond the padding never count);
 *                a zero count gives NaN (0/0).
 *   Output extent: floor((H + pt + pb - dil_h*(KH-1) - 1) / stride_h) + 1, or with
 *   ceil_mode the division rounded up, after which a last window that starts
 *   inside the end padding ((Ho-1)*stride_h - pad_top >= H) is dropped.
 *   GlobalMaxPool / GlobalAveragePool: one value per (n, c) plane, y [n, c, 1, 1];
 *   the max under the rules above, the mean as a fixed halving tree of float32
 *   sums over the plane (pairs i, i + ceil(m/2) while m > 1, for a plane of up
 *   to 4096 elements; larger planes sum chunks of 4096 that way, then the chunk
 *   sums), divided by H*W.  The order depends on H*W only, so reruns are
 *   bit-identical.
 *
 * Layout: x NCHW [n, c, h, w], y NCHW [n, c, Ho, Wo], dense, at base + element
 * offset.  Element types (conv_dtype): CONV_F32, CONV_F16, CONV_BF16; the
 * average accumulates in float32 and rounds once to the element type.
 *
 * Ownership, errors and threading as in conv.h: device buffers are the caller's;
 * pool_forward only enqueues on the stream, never allocates or synchronises;
 * every check runs on the host before anything is enqueued; calls are reentrant.
 */
#ifndef CONVFWD_POOL_H
#define CONVFWD_POOL_H

#include <stdint.h>

#include "conv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    POOL_MAX = 0,
    POOL_AVERAGE = 1,
    POOL_GLOBAL_MAX = 2,
    POOL_GLOBAL_AVERAGE = 3
} pool_kind;

/* The problem ("Layout and operands": PoolProblem): shape, window, stride,
 * dilation, explicit pads, ceil_mode, count_include_pad and element offsets.
 * For the global kinds only n, c, h, w, the offsets and kind are read. */
typedef struct pool_problem {
    int64_t n, c, h, w;
    int64_t kh, kw;
    int64_t stride_h, stride_w;
    int64_t dil_h, dil_w;
    int64_t pad_top, pad_left, pad_bottom, pad_right;  /* explicit, >= 0 */
    int64_t x_off, y_off;      /* element offsets added to the pointers */
    int32_t kind;              /* pool_kind */
    int32_t ceil_mode;         /* 0/1 */
    int32_t count_include_pad; /* 0/1 (average only) */
    int32_t reserved;          /* must be 0 */
} pool_problem;

/* Output extent (the GpuWindow.OutputExtent analog of "Layout and operands"),
 * with the ceil_mode rule above; 1 x 1 for the global kinds.  Pure host.
 * Returns CONV_OK, CONV_ERR_ARG (bad enum or flag) or CONV_ERR_SHAPE (dims,
 * stride or dilation < 1, pads < 0, no window fits, an operand above 2^31-1
 * elements, int64 overflow). */
int pool_output_extent(const pool_problem* p, int64_t* ho, int64_t* wo);

/* Resolve ONNX auto_pad (conv_auto_pad values) into explicit pads, as for Conv
 * ("Layout and operands": WithAutoPad): SAME_* keeps Ho = ceil(H/s) with total
 * pad max(0, (Ho-1)s + d(k-1) + 1 - H), SAME_UPPER puts the odd unit at the end,
 * SAME_LOWER at the begin; VALID zeroes the pads; NOTSET keeps them.  Pure host. */
int pool_resolve_auto_pad(pool_problem* p, int auto_pad);

/* Name of the kernel the planner picks for a shape, NUL-terminated, e.g.
 * "pool.max.f16.band8", "pool.global_average.f32.tree".  Shape-only (no HIP
 * runtime call).  CONV_ERR_ARG when len is too small. */
int pool_describe_variant(const pool_problem* p, int dtype, char* buf, uint64_t len);

/* Every check pool_forward runs (shape, enums, null pointers, y overlapping x),
 * returning the status it would return, with no HIP runtime call. */
int pool_check(const pool_problem* p, int dtype, const void* x, const void* y);

/* Pooling forward: x and y are required device pointers (base + element
 * offsets); y must not overlap x.  stream is a hipStream_t (NULL = default).
 * Asynchronous: returns once the work is enqueued.  Errors: CONV_ERR_ARG /
 * SHAPE / OVERLAP before anything is enqueued; CONV_ERR_DEVICE if the runtime
 * refuses the launch. */
int pool_forward(const pool_problem* p, int dtype, const void* x, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_POOL_H */
