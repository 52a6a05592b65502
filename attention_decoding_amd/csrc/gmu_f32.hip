// fp32 Gated Memory Unit (Paper-Notes reading notes on "Decoder-Hybrid-Decoder
// Architecture for Efficient Reasoning with Long Generation", section 关键设计):
//   H = M ⊙ SiLU(X W1^T),  Y = H W2^T,  all in fp32.
// This path exists for full-precision checking of small shapes; it is a plain
// one-output-per-thread kernel pair with sequential fp32 accumulation along K.
#include "device.hpp"
#include "launch.hpp"

#include <math.h>

namespace sambay {

namespace {

__global__ __launch_bounds__(256) void gmu_f32_gate_kernel(const float *__restrict__ M, const float *__restrict__ X,
                                                           const float *__restrict__ W1, float *__restrict__ H,
                                                           int64_t rows, int64_t d_model, int64_t d_inner) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * d_inner) return;
    const int64_t r = idx / d_inner, k = idx % d_inner;
    const float *x = X + r * d_model;
    const float *w = W1 + k * d_model;
    float z = 0.f;
    for (int64_t c = 0; c < d_model; ++c) z = fmaf(x[c], w[c], z);
    H[idx] = M[idx] * (z / (1.f + expf(-z)));
}

__global__ __launch_bounds__(256) void gmu_f32_out_kernel(const float *__restrict__ H, const float *__restrict__ W2,
                                                          float *__restrict__ Y, int64_t rows, int64_t d_model,
                                                          int64_t d_inner) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * d_model) return;
    const int64_t r = idx / d_model, o = idx % d_model;
    const float *hp = H + r * d_inner;
    const float *w = W2 + o * d_inner;
    float y = 0.f;
    for (int64_t k = 0; k < d_inner; ++k) y = fmaf(hp[k], w[k], y);
    Y[idx] = y;
}

}  // namespace

hipError_t launch_gmu_f32(const float *M, const float *X, const float *W1, const float *W2, float *Y, float *H,
                          int64_t rows, int64_t d_model, int64_t d_inner, hipStream_t stream) {
    const int64_t n1 = rows * d_inner, n2 = rows * d_model;
    TimingScope ts(kTimeGmuF32, stream);
    hipLaunchKernelGGL(gmu_f32_gate_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, stream, M, X, W1, H,
                       rows, d_model, d_inner);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gmu_f32_out_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, stream, H, W2, Y, rows,
                       d_model, d_inner);
    return hipGetLastError();
}

}  // namespace sambay
