// synth_gen.hip - the seeded input generator of synth_gen.c, for the GPU.
//
// Same counters, same Philox4x32-10 rounds, same Irwin-Hall normal, same
// fp32 Student-t(2) and 16-level quantiser, same bfloat16 rounding; only
// integer operations and correctly rounded fp32 operations are used, so the
// output bits equal the host generator's (a GPU test compares them).  This
// file holds none of the optimizer's arithmetic; it only fills input arrays.
// Built with -ffp-contract=off and IEEE fp32 division and square root.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u, kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
constexpr uint32_t kPurposeGrad = 1u, kPurposeParam = 2u;

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kW0;
            k1 += kW1;
        }
        const uint64_t p0 = (uint64_t)kM0 * c[0];
        const uint64_t p1 = (uint64_t)kM1 * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[1] = (uint32_t)p1;
        c[3] = (uint32_t)p0;
        c[0] = n0;
        c[2] = n2;
    }
}

__device__ __forceinline__ float irwin_hall8(const uint32_t w[4]) {
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += (int32_t)(w[i] & 0xFFFFu) + (int32_t)(w[i] >> 16);
    return (float)(s - 262140) * (1.0f / 65536.0f);
}

__device__ __forceinline__ float student2(uint32_t w) {
    const float u = (float)(2u * (w >> 9) + 1u) * (1.0f / 16777216.0f);
    return (2.0f * u - 1.0f) / sqrtf(2.0f * u * (1.0f - u));
}

__device__ __forceinline__ float quantise16(float v) {
    const float delta = 1.0f / 4096.0f;
    float q = rintf(v / delta);
    if (q < -8.0f) q = -8.0f;
    if (q > 7.0f) q = 7.0f;
    return q * delta;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

__global__ void k_grad_bf16(uint32_t seed, uint32_t tensor, uint32_t step, uint32_t worker, int kind, float scale,
                            int quantise, uint64_t e0, uint64_t n, uint16_t* __restrict__ out) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        uint32_t c[4] = {(uint32_t)(e0 + i), tensor, step, worker};
        philox4x32_10(c, seed, kPurposeGrad);
        const float v0 = kind == 0 ? irwin_hall8(c) : student2(c[0]);
        float v = v0 * scale;
        if (quantise) v = quantise16(v);
        out[i] = f32_to_bf16_rne(v);
    }
}

__global__ void k_param_f32(uint32_t seed, uint32_t tensor, float scale, uint64_t e0, uint64_t n,
                            float* __restrict__ out) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        uint32_t c[4] = {(uint32_t)(e0 + i), tensor, 0u, 0u};
        philox4x32_10(c, seed, kPurposeParam);
        out[i] = irwin_hall8(c) * scale;
    }
}

dim3 grid_for(uint64_t n) {
    uint64_t b = (n + 255) / 256;
    if (b > 65536u) b = 65536u;
    if (b == 0) b = 1;
    return dim3((uint32_t)b);
}

}  // namespace

extern "C" {

// Gradient bits (bfloat16) for elements [e0, e0+n) of one tensor into device
// memory `out`, on `stream`.  Returns a hipError_t.
int synth_gpu_grad_bf16(uint32_t seed, uint32_t tensor, uint32_t step, uint32_t worker, int kind, float scale,
                        int quantise, uint64_t e0, uint64_t n, uint16_t* out, void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_grad_bf16, grid_for(n), dim3(256), 0, (hipStream_t)stream, seed, tensor, step, worker, kind,
                       scale, quantise, e0, n, out);
    return (int)hipGetLastError();
}

int synth_gpu_param_f32(uint32_t seed, uint32_t tensor, float scale, uint64_t e0, uint64_t n, float* out,
                        void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(k_param_f32, grid_for(n), dim3(256), 0, (hipStream_t)stream, seed, tensor, scale, e0, n, out);
    return (int)hipGetLastError();
}

}  // extern "C"
