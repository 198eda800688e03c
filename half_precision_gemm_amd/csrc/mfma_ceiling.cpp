// mfma_ceiling — measures the MFMA-only throughput ceiling of the GPU for
// v_mfma_f32_32x32x16_f16 on operands like the benchmark's (fp16 values drawn
// uniformly from [-1, 1)), and the shader clock it runs at.
//
// Every wave keeps 16 independent 32×32 fp32 accumulators and issues MFMAs
// back to back on register-resident operands: no memory traffic, no LDS, no
// barriers.  What remains is the matrix core rate at the clock the power
// limit allows for this data, i.e. the highest rate any fp16 GEMM kernel can
// reach on these inputs.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWGs = 1024, kThreads = 256, kIters = 4000, kChains = 16;

__global__ void __launch_bounds__(256, 1)
mfma_loop(const half8 *__restrict__ src, float *__restrict__ out, long long *__restrict__ stamps)
{
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const half8 a0 = src[4 * t + 0], b0 = src[4 * t + 1];
    const half8 a1 = src[4 * t + 2], b1 = src[4 * t + 3];
    floatx16 acc[kChains];
    for (int i = 0; i < kChains; ++i)
        acc[i] = floatx16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const long long c0 = clock64(), w0 = wall_clock64();
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16((i & 1) ? a1 : a0, (i & 2) ? b1 : b0,
                                                            acc[i], 0, 0, 0);
    }
    const long long c1 = clock64(), w1 = wall_clock64();
    float s = 0.f;
    for (int i = 0; i < kChains; ++i)
        for (int j = 0; j < 16; ++j)
            s += acc[i][j];
    out[t] = s;                                  // keeps the loop live
    if (threadIdx.x == 0) {
        stamps[4 * blockIdx.x + 0] = c1 - c0;    // shader clock cycles
        stamps[4 * blockIdx.x + 1] = w1 - w0;    // 100 MHz wall-clock ticks
    }
}

#define CHECK(x)                                                                             \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            fprintf(stderr, "mfma_ceiling: %s failed: %s\n", #x, hipGetErrorString(e_));     \
            return 1;                                                                        \
        }                                                                                    \
    } while (0)

int main()
{
    // Operands: fp16 values uniform in [-1, 1) from a fixed 32-bit LCG.
    std::vector<_Float16> h((size_t)kWGs * kThreads * 4 * 8);
    uint32_t x = 12345u;
    for (auto &v : h) {
        x = x * 1664525u + 1013904223u;
        v = (_Float16)((float)((x >> 8) & 0xffff) / 32768.0f - 1.0f);
    }
    half8 *src = nullptr;
    float *out = nullptr;
    long long *stamps = nullptr;
    CHECK(hipMalloc(&src, h.size() * sizeof(_Float16)));
    CHECK(hipMalloc(&out, (size_t)kWGs * kThreads * sizeof(float)));
    CHECK(hipMalloc(&stamps, (size_t)kWGs * 4 * sizeof(long long)));
    CHECK(hipMemcpy(src, h.data(), h.size() * sizeof(_Float16), hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const double flops = (double)kWGs * (kThreads / 64) * kIters * kChains * 2.0 * 32 * 32 * 16;
    double best = 0, best_ghz = 0;
    std::vector<long long> st((size_t)kWGs * 4);
    for (int rep = 0; rep < 5; ++rep) {
        CHECK(hipEventRecord(e0, 0));
        hipLaunchKernelGGL(mfma_loop, dim3(kWGs), dim3(kThreads), 0, 0, src, out, stamps);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1, 0));
        CHECK(hipEventSynchronize(e1));
        float ms = 0;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        CHECK(hipMemcpy(st.data(), stamps, st.size() * sizeof(long long), hipMemcpyDeviceToHost));
        double cyc = 0, ticks = 0;
        for (int i = 0; i < kWGs; ++i) {
            cyc += (double)st[4 * i];
            ticks += (double)st[4 * i + 1];
        }
        const double tf = flops / (ms * 1e-3) / 1e12;
        const double ghz = cyc / (ticks / 100e6) / 1e9;
        if (tf > best) {
            best = tf;
            best_ghz = ghz;
        }
    }
    printf("{\"mfma_ceiling_tflops\": %.1f, \"clock_ghz\": %.3f, \"instruction\": "
           "\"v_mfma_f32_32x32x16_f16\", \"operands\": \"fp16 uniform [-1,1)\", \"repeats\": 5}\n",
           best, best_ghz);
    hipFree(src);
    hipFree(out);
    hipFree(stamps);
    return 0;
}
