// Test helper (not part of the library): run the hardware 16x16x32 bf16
// matrix instruction on operand fragments stored in lane order, so the
// tests can check that the fragment layout the oracle defines is the one
// the instruction consumes.  For block g: D = A_frag[g] x B_frag[g], each
// fragment 64 lanes x 8 bf16; lane l's four fp32 results go to d[g][l][0..3].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void k_mfma_probe(const bf16x8* __restrict__ a, const bf16x8* __restrict__ b,
                                                   f32x4* __restrict__ d) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[i], acc, 0, 0, 0);
    d[i] = acc;
}

extern "C" __attribute__((visibility("default"))) int mfma_probe_16x16x32_bf16(const void* a_frag, const void* b_frag,
                                                                             void* d_out, int n_blocks,
                                                                             void* stream) {
    if (n_blocks < 0 || !a_frag || !b_frag || !d_out) return -1;
    if (n_blocks == 0) return 0;
    hipLaunchKernelGGL(k_mfma_probe, dim3(n_blocks), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bf16x8*>(a_frag), static_cast<const bf16x8*>(b_frag),
                       static_cast<f32x4*>(d_out));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
