// roof_probe.hip -- microbenchmarks behind the roofline figures of the
// benchmark (libbdssm_probe.so; measurement only, not part of the scan
// library).  Each entry point enqueues one launch on the given stream; the
// caller times it with events on that stream.
//
//   probe_fma    fp32 FMA issue rate: 8 independent FMA chains per lane
//   probe_exp    v_exp_f32 issue rate: 8 independent exp2 chains per lane
//   probe_mix    the forward scan's operation mix per (token, state):
//                dt * A' (mul), exp2, (dt * x) * B (mul), state FMA, with 16
//                states per lane as in chunk_state_kernel
//   probe_read   HBM read bandwidth: a grid-stride float4 sum over a buffer
//   probe_empty  an empty kernel: the launch floor of a grid of that shape
//
// Work per launch (for the caller's rate):
//   probe_fma / probe_exp: grid * block * iters * 8 operations
//   probe_mix: grid * block * iters * 16 elements (5 issue slots each if exp2
//              takes two) plus one mul per (lane, iteration)
//   probe_read: n_vec4 * 16 bytes
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void fma_kernel(float *out, int iters, float b, float c) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (float)(threadIdx.x + i) * 1e-3f;
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(a[i], b, c);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += a[i];
    if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // never true; keeps the chains live
}

__global__ __launch_bounds__(256) void exp_kernel(float *out, int iters) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (float)(threadIdx.x % 7 + i) * 0.1f;
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = __builtin_amdgcn_exp2f(-a[i]);   // stays in (0, 1]
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += a[i];
    if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(64) void mix_kernel(float *out, int iters, const float *A, const float *Bv) {
    float h[16], a2[16], bb[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) { h[n] = 0.f; a2[n] = A[n]; bb[n] = Bv[n]; }
    float d = 0.3f + (float)(threadIdx.x & 7) * 1e-3f;
    const float x = 0.7f;
    // unrolled by two so that the states alternate between register sets
    // instead of being moved back at the loop's end
#pragma unroll 2
    for (int it = 0; it < iters; ++it) {
        const float v = d * x;                        // dt * x, once per (token, channel)
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const float dA = __builtin_amdgcn_exp2f(d * a2[n]);
            h[n] = __builtin_fmaf(dA, h[n], v * bb[n]);
        }
        d = __builtin_fmaf(d, -1e-7f, d);            // a new step size each token
    }
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) s += h[n];
    if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const float4 *__restrict__ src, int64_t n, float *out) {
    float s = 0.f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float4 v = src[i];
        s += (v.x + v.y) + (v.z + v.w);
    }
    if (s == 12345.678f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void empty_kernel() {}

int status() { return hipGetLastError() == hipSuccess ? 0 : -6; }

}  // namespace

extern "C" {

// grid workgroups of 256 lanes; out: a buffer of grid * 256 floats (written
// only in the never-taken case that keeps the arithmetic alive).
int probe_fma(float *out, int grid, int iters, void *stream) {
    hipLaunchKernelGGL(fma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters, 0.999f, 1e-3f);
    return status();
}

int probe_exp(float *out, int grid, int iters, void *stream) {
    hipLaunchKernelGGL(exp_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    return status();
}

// grid one-wave workgroups (64 lanes); A, Bv: 16 floats each (device)
int probe_mix(float *out, const float *A, const float *Bv, int grid, int iters, void *stream) {
    hipLaunchKernelGGL(mix_kernel, dim3(grid), dim3(64), 0, (hipStream_t)stream, out, iters, A, Bv);
    return status();
}

// src: n_vec4 float4 values (device, 16-byte aligned); out: grid * 256 floats
int probe_read(const void *src, int64_t n_vec4, float *out, int grid, void *stream) {
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const float4 *)src, n_vec4,
                       out);
    return status();
}

// an empty kernel on a (gx, gy, gz) grid of `block`-lane workgroups
int probe_empty(int gx, int gy, int gz, int block, void *stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(gx, gy, gz), dim3(block), 0, (hipStream_t)stream);
    return status();
}

}  // extern "C"
