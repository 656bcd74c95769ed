// kda_calib.hip -- a kernel of known MFMA instruction count (counter calibration).
#include "kda_calib.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One dependent chain of MFMAs per wave; the waves sharing a SIMD (a launch of a few
// thousand workgroups holds several per SIMD) keep its matrix unit fed between them.
__global__ __launch_bounds__(256) void mfma_calib_kernel(int iters, float *out) {
    const int l = threadIdx.x;
    bf16x8 a, b;
    for (int s = 0; s < 8; ++s) {
        a[s] = (__bf16)(0.001f * (float)((l + s) & 7));
        b[s] = (__bf16)(0.002f * (float)((l * 3 + s) & 7));
    }
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    out[blockIdx.x * 256 + l] = c[0] + c[1] + c[2] + c[3];
}

}  // namespace

extern "C" int kda_calib_mfma(int n_workgroups, int iters, float *out, void *stream) {
    if (n_workgroups < 1 || iters < 1 || !out) return 1;
    hipLaunchKernelGGL(mfma_calib_kernel, dim3(n_workgroups), dim3(256), 0, (hipStream_t)stream, iters, out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : 1000 + (int)e;
}
