"""The variant the planner names for each workload layer.  The plan is a
function of the shape alone, so the same strings hold on the CPU (no device)
and on the GPU; the CPU tier and the GPU tier both assert them."""

EXPECTED_PLANS = {
    "w1_conv3x3_f32": "implicit_gemm.f32.t64x64.split1",
    "w2_bottleneck3x3_f16": "implicit_gemm_halo.f16.rowshift.r14.n32",
    "w3a_stem7x7s2_f16": "implicit_gemm_rowband.f16.rows14",
    "w3b_pointwise_f16": "pointwise_gemm.f16.t128x128.k64",
    "w4a_depthwise5x5_f32": "depthwise_direct.f32.wave.col14",
    "w4b_depthwise3x3s2_f32": "depthwise_direct.f32.wave.col4",
    "w4c_pointwise_f32": "pointwise_gemm.f32.t256x16.strip",
    "w5a_dilated_grouped_f16": "implicit_gemm_grouped.f16.c8.n8",
    "w5b_convtranspose2x2s2_f16": "transpose_gemm_col2im.f16.fused_k2s2.t128x64",
    "x1_late3x3_512_7x7_f16": "implicit_gemm_halo.f16.rowshift.r8.n32.split8",
    "x2_bottleneck3x3_bf16": "implicit_gemm_halo.bf16.rowshift.r14.n32",
    "x3_bottleneck3x3_f16_winograd": "winograd_f2x2_3x3.f16.band4x7.c64",
}


def layer_problem(cf, layer):
    return cf.make_problem(layer.n, layer.c_in, layer.h, layer.w, layer.c_out, layer.kh,
                           layer.kw, groups=layer.groups, stride=layer.stride,
                           dilation=layer.dilation, pads=layer.pads, out_pad=layer.out_pad,
                           transpose=layer.transpose, act=layer.act, bias=layer.bias,
                           residual=layer.residual, variant=layer.variant)
