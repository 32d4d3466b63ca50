/*
 * conv_integer.h — C ABI of the MI355X (gfx950) ConvInteger forward
 * (libconvfwd.so; status codes and the problem struct are conv.h's).
 *
 * Operation ("Convolution, pooling and resize" (OneGpu docs), section
 * "ConvInteger"; ONNX ConvInteger):
 *
 *   y[n,co,oh,ow] = sum_{ci',kh,kw} (x[n, g*Cin/G+ci', ih, iw] - x_zero)
 *                                   * (w[co, ci', kh, kw] - w_zero[co])
 *
 * over the real taps (ih = oh*stride_h - pad_top + kh*dil_h, likewise iw), in
 * int32 with wrap-around: the exact integer sum modulo 2^32, as two's
 * complement.  A padded tap is the real value zero, which is the quantized
 * value x_zero, so it adds nothing.  The geometry is conv_problem's (strides,
 * dilations, asymmetric pads, groups, 1-D as height 1); the transposed, fused
 * epilogue, variant and split fields must be zero (CONV_ERR_ARG otherwise).
 * The result is exact: the same bits on every device and run.
 *
 * Layout: x NCHW [n, c_in, h, w] of 8-bit elements, w OIHW [c_out, c_in/groups,
 * kh, kw] of 8-bit elements, y NCHW [n, c_out, Ho, Wo] of int32, each at base +
 * element offset (x_off, w_off in bytes of 1-byte elements, y_off in int32
 * elements; b_off and r_off unused).  x_type and w_type (convi_type) say
 * whether each operand is uint8 or int8, in any mix.  x_zero points to one
 * element of x's type; w_zero to one element of w's type, or to c_out of them
 * when w_zero_per_channel is 1; either may be NULL for a zero point of 0.
 * Zero points live in device memory, like the operands.
 *
 * Ownership, errors and threading as in conv.h: buffers are the caller's; the
 * forward only enqueues, never allocates or synchronises; every check runs on
 * the host before anything is enqueued.
 */
#ifndef CONVFWD_CONV_INTEGER_H
#define CONVFWD_CONV_INTEGER_H

#include <stdint.h>

#include "conv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x and of w. */
typedef enum { CONVI_U8 = 0, CONVI_I8 = 1 } convi_type;

/* Name of the kernel that runs ("conv_integer.<x><w>.implicit_gemm.i8mfma.t64x64").
 * Shape-only; CONV_ERR_ARG when len is too small. */
int conv_integer_describe_variant(const conv_problem* p, int x_type, int w_type, char* buf,
                                  uint64_t len);

/* Every check conv_integer_forward runs (shape, enums, unused fields zero, null
 * pointers, y overlapping x, w or a zero point), with no HIP runtime call. */
int conv_integer_check(const conv_problem* p, int x_type, int w_type, const void* x,
                       const void* w, const void* x_zero, const void* w_zero,
                       int w_zero_per_channel, const void* y);

/* ConvInteger forward on `stream` (a hipStream_t, NULL = default).  x, w, y are
 * required device pointers; y must not overlap x, w or the zero points.
 * Asynchronous.  Errors: CONV_ERR_ARG / SHAPE / OVERLAP before anything is
 * enqueued, CONV_ERR_DEVICE if the runtime refuses the launch. */
int conv_integer_forward(const conv_problem* p, int x_type, int w_type, const void* x,
                         const void* w, const void* x_zero, const void* w_zero,
                         int w_zero_per_channel, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVFWD_CONV_INTEGER_H */
