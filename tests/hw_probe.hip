// Test helper (not part of the library): hardware probes that pin the lane
// layouts the kernels rely on.
//
// mfma_probe_16x16x32_bf16: run the 16x16x32 bf16 matrix instruction on
// operand fragments stored in lane order, so the tests can check that the
// fragment layout the oracle defines is the one the instruction consumes.
// For block g: D = A_frag[g] x B_frag[g], each fragment 64 lanes x 8 bf16;
// lane l's four fp32 results go to d[g][l][0..3].
//
// tr16_probe: one wave fills 16 KiB of LDS with halfword i = i, each lane
// issues one ds_read_b64_tr_b16 at its own byte address, and the four
// halfwords every lane receives are written out, so the tests can check the
// instruction's lane semantics.
//
// tr8_probe: the same for the 8-bit transpose read ds_read_b64_tr_b8: LDS
// byte i holds (i >> shift) & 0xff (two runs, shift 0 and 8, name every byte
// of a 16 KiB window), each lane reads at its own address and the eight
// bytes every lane receives are written out.
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

struct TrAddrs {
    int32_t a[64];
};

__global__ __launch_bounds__(64) void k_tr16_probe(TrAddrs addrs, uint16_t* __restrict__ out) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    __shared__ uint16_t lds[8192];
    for (int i = threadIdx.x; i < 8192; i += 64) lds[i] = static_cast<uint16_t>(i);
    __syncthreads();
    const int a = addrs.a[threadIdx.x];
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) uint8_t*)lds + a));
    for (int j = 0; j < 4; ++j) out[threadIdx.x * 4 + j] = static_cast<uint16_t>(v[j]);
}

// addrs: 64 host byte offsets, each 8-byte aligned and at most 16384 - 8;
// d_out: device buffer of 256 uint16.  Returns -1 for a bad offset (nothing
// launched), -3 on a launch error, 0 otherwise.
extern "C" __attribute__((visibility("default"))) int tr16_probe(const int32_t* addrs, void* d_out, void* stream) {
    if (!addrs || !d_out) return -1;
    TrAddrs t;
    for (int l = 0; l < 64; ++l) {
        if (addrs[l] < 0 || addrs[l] > 16384 - 8 || addrs[l] % 8) return -1;
        t.a[l] = addrs[l];
    }
    hipLaunchKernelGGL(k_tr16_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), t,
                       static_cast<uint16_t*>(d_out));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

__global__ __launch_bounds__(64) void k_tr8_probe(TrAddrs addrs, int shift, uint8_t* __restrict__ out) {
    typedef int v2i32 __attribute__((ext_vector_type(2)));
    __shared__ uint8_t lds[16384];
    for (int i = threadIdx.x; i < 16384; i += 64) lds[i] = static_cast<uint8_t>(i >> shift);
    __syncthreads();
    const int a = addrs.a[threadIdx.x];
    const v2i32 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i32*)((__attribute__((address_space(3))) uint8_t*)lds + a));
    for (int j = 0; j < 8; ++j) out[threadIdx.x * 8 + j] = static_cast<uint8_t>(v[j / 4] >> (8 * (j % 4)));
}

// As tr16_probe; shift is 0 or 8; d_out holds 512 bytes.
extern "C" __attribute__((visibility("default"))) int tr8_probe(const int32_t* addrs, int shift, void* d_out,
                                                               void* stream) {
    if (!addrs || !d_out || (shift != 0 && shift != 8)) return -1;
    TrAddrs t;
    for (int l = 0; l < 64; ++l) {
        if (addrs[l] < 0 || addrs[l] > 16384 - 8 || addrs[l] % 8) return -1;
        t.a[l] = addrs[l];
    }
    hipLaunchKernelGGL(k_tr8_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), t, shift,
                       static_cast<uint8_t*>(d_out));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
