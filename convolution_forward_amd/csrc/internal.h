// Internal declarations shared by the host dispatcher and the kernel files.
// Nothing here is part of the public ABI (include/convfwd.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "convfwd.h"

namespace convfwd {

// A validated dense problem: NHWC X with element strides, KKIO F, NHWC Y.
struct DenseProblem {
    const void *X;
    int64_t xs[4];
    const void *F;
    const float *bias;
    void *Y;
    int64_t ys[4];
    int N, H, W, Cin, KH, KW, Cout, Ho, Wo;
    conv_dtype xdt, ydt;
    // Window: stride, padding before each axis (the padding after only
    // shapes Ho and Wo), dilation, groups. The lecture's operator is
    // sh = sw = dh = dw = groups = 1, pt = pl = 0.
    int sh, sw, pt, pl, dh, dw, groups;
};

// True for the lecture's restricted operator (unit stride, no padding, no
// dilation, one group).
inline bool plain_window(const DenseProblem &p)
{
    return p.sh == 1 && p.sw == 1 && p.pt == 0 && p.pl == 0 && p.dh == 1 && p.dw == 1 && p.groups == 1 &&
           p.Ho == p.H - p.KH + 1 && p.Wo == p.W - p.KW + 1;
}

// A validated depthwise problem: contiguous NCHW X, [C*mult,KH,KW] w, NCHW Y.
struct DwProblem {
    const float *X;
    const float *w;
    const float *bias;
    float *Y;
    int N, C, H, W, mult, KH, KW, sh, sw, ph, pw, dh, dw, Ho, Wo;
    int pb, pr;         // padding after each axis (ph, pw are the padding before)
    conv_dw_mode mode;
};

// Dense kernels.
hipError_t launch_dense_direct(const DenseProblem &p, hipStream_t s);
bool dense_band_supports(const DenseProblem &p);
bool dense_pw_supports(const DenseProblem &p);
hipError_t launch_dense_pw(const DenseProblem &p, hipStream_t s);
hipError_t launch_dense_band(const DenseProblem &p, int gpack, hipStream_t s);
bool dense_mfma_bf16_supports(const DenseProblem &p);
hipError_t launch_dense_mfma_bf16(const DenseProblem &p, hipStream_t s);
bool dense_gemm_bf16_supports(const DenseProblem &p);
hipError_t launch_dense_gemm_bf16(const DenseProblem &p, hipStream_t s);
bool dense_mfma_f32_supports(const DenseProblem &p);
hipError_t launch_dense_mfma_f32(const DenseProblem &p, hipStream_t s);
bool dense_gemm_f32_supports(const DenseProblem &p);
bool dense_f32x6_supports(const DenseProblem &p);
hipError_t launch_dense_f32x6(const DenseProblem &p, hipStream_t s);
hipError_t launch_dense_gemm_f32(const DenseProblem &p, hipStream_t s);

// Depthwise kernels.
hipError_t launch_dw_direct(const DwProblem &p, hipStream_t s);
bool dw_tiled_supports(const DwProblem &p);
bool dw_pad_supports(const DwProblem &p);
bool dw_waves_supports(const DwProblem &p);
hipError_t launch_dw_waves(const DwProblem &p, hipStream_t s);
bool dw_planes_supports(const DwProblem &p);
bool dw_rows_supports(const DwProblem &p);
hipError_t launch_dw_rows(const DwProblem &p, hipStream_t s);
hipError_t launch_dw_planes(const DwProblem &p, hipStream_t s);
hipError_t launch_dw_pad(const DwProblem &p, hipStream_t s);
hipError_t launch_dw_tiled(const DwProblem &p, hipStream_t s);

// A validated explicit patch-matrix problem: NHWC X with element strides,
// cols contiguous [N*Ho*Wo, KH*KW*Cin] of the same dtype.
struct Im2colProblem {
    const void *X;
    int64_t xs[4];
    void *cols;
    int N, H, W, Cin, KH, KW, Ho, Wo;
    int sh, sw, pt, pl, dh, dw;
    conv_dtype dtype;
};

hipError_t launch_im2col(const Im2colProblem &p, hipStream_t s);

// Streaming copies used for bandwidth / counter calibration.
hipError_t launch_copy_bytes(const void *src, void *dst, int64_t bytes, hipStream_t s);
hipError_t launch_copy_wide(const void *src, void *dst, int64_t bytes, hipStream_t s);

}  // namespace convfwd
