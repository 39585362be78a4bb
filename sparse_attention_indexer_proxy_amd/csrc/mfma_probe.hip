// Practical ceilings of the two rooflines the indexer is measured against.
//
//   mfma_probe [seconds-per-test]
//
// prints one JSON line:
//   mfma_bf16_random_tflops  v_mfma_f32_16x16x32_bf16 issued back to back
//                            from registers, operands drawn at random (the
//                            sustained clock under a dense MFMA load depends
//                            on how many operand bits toggle)
//   mfma_bf16_zero_tflops    the same loop with all-zero operands
//   copy_gbs                 a device-to-device copy of 2 GiB (read + write
//                            bytes over time)
//
// The MFMA loop has the occupancy of the fused proxy scan (two waves per
// SIMD) and four independent accumulator chains per wave, so it is bound by
// the matrix pipe, not by dependences.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                              \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(1);                                                                          \
        }                                                                                     \
    } while (0)

constexpr int kThreads = 256;       // 4 waves per workgroup
constexpr int kMfmaPerIter = 64;    // 16 (A fragments) x 4 (accumulators)

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_loop(
    const uint4 *__restrict__ src, float *__restrict__ out, int iters)
{
    const int l = threadIdx.x & 63;
    bf16x8 a[16], b[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = __builtin_bit_cast(bf16x8, src[i * 64 + l]);
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, src[(16 + i) * 64 + l]);
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[j], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

static double time_mfma(const uint4 *src, float *out, int blocks, int iters)
{
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(kThreads), 0, 0, src, out, iters / 8);  // warm-up
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e0, 0));
    hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(kThreads), 0, 0, src, out, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    const double flops = double(blocks) * (kThreads / 64) * double(iters) * kMfmaPerIter * 16.0 * 16.0 * 32.0 * 2.0;
    return flops / (ms * 1e-3) / 1e12;
}

int main(int argc, char **argv)
{
    const double seconds = argc > 1 ? atof(argv[1]) : 0.5;
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    const int blocks = cus * 2;  // 8 waves per CU = 2 per SIMD

    // operands: 20 fragments x 64 lanes x 16 B
    const size_t n16 = 20 * 64 * 8;
    std::vector<uint16_t> h(n16);
    uint32_t x = 0x9E3779B9u;
    for (size_t i = 0; i < n16; ++i) {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        // bf16 with a random sign and mantissa, exponent in [2^-4, 2^3]
        const uint16_t sign = (x >> 31) << 15;
        const uint16_t expo = static_cast<uint16_t>(123 + (x >> 8) % 8) << 7;
        h[i] = sign | expo | static_cast<uint16_t>(x & 0x7F);
    }
    uint4 *src_rand, *src_zero;
    float *out;
    CHECK(hipMalloc(&src_rand, n16 * 2));
    CHECK(hipMalloc(&src_zero, n16 * 2));
    CHECK(hipMalloc(&out, size_t(blocks) * kThreads * sizeof(float)));
    CHECK(hipMemcpy(src_rand, h.data(), n16 * 2, hipMemcpyHostToDevice));
    CHECK(hipMemset(src_zero, 0, n16 * 2));

    // size the loop to about `seconds` at 2 PFLOP/s
    const double per_iter = double(blocks) * (kThreads / 64) * kMfmaPerIter * 16.0 * 16.0 * 32.0 * 2.0;
    int iters = static_cast<int>(seconds * 2.0e15 / per_iter);
    if (iters < 64) iters = 64;
    const double t_rand = time_mfma(src_rand, out, blocks, iters);
    const double t_zero = time_mfma(src_zero, out, blocks, iters);

    // copy: 2 GiB device to device
    const size_t bytes = size_t(2) << 30;
    void *a, *b;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMemset(a, 1, bytes));
    CHECK(hipMemcpy(b, a, bytes, hipMemcpyDeviceToDevice));  // warm-up
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const int reps = 5;
    CHECK(hipEventRecord(e0, 0));
    for (int r = 0; r < reps; ++r) CHECK(hipMemcpyAsync(b, a, bytes, hipMemcpyDeviceToDevice, 0));
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const double copy_gbs = 2.0 * double(bytes) * reps / (ms * 1e-3) / 1e9;

    printf("{\"mfma_bf16_random_tflops\": %.1f, \"mfma_bf16_zero_tflops\": %.1f, \"copy_gbs\": %.1f, "
           "\"cus\": %d, \"mfma_waves_per_simd\": 2}\n",
           t_rand, t_zero, copy_gbs, cus);
    CHECK(hipFree(a));
    CHECK(hipFree(b));
    CHECK(hipFree(src_rand));
    CHECK(hipFree(src_zero));
    CHECK(hipFree(out));
    return 0;
}
