// GPU checks of the pack's quantisation arithmetic (combine_moe_layout_02_amd/csrc/pack_rows.h),
// run by tests/test_gpu_quant_native.py, which compares what this program writes with the oracle.
//
//   quant_gpu cvt OUT
//       Every non-negative finite fp32 value q (bit patterns 0 .. 0x7F7FFFFF) through e4m3fn_pack4:
//       writes uint32 first[256] (the smallest q, as bits, whose code is c; 0xFFFFFFFF if none),
//       then uint64 counts of q whose code is below the code of the previous q (the encoder must be
//       monotone) and of q whose negation does not give the code with the sign bit set.
//   quant_gpu div SCALES OUT
//       SCALES: float32 scales. For every scale and every finite bf16 x: the code bytes of
//       x / scale as the pack computes it (div_by_scale with y = 1 / scale) for E4M3FN and for
//       INT8, written as uint8 [n][65536] each; then uint64 counts, over all pairs with
//       |x / scale| <= 449, of quotients that differ from the IEEE division for |x / scale| >= 2^-11
//       and of codes that differ from the codes of the IEEE quotient.
//   quant_gpu divcount SCALES OUT
//       The same counts only (for scale lists too long to write every code).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pack_rows.h"

using namespace moe::rows;

#define CHECK_HIP(x)                                                                   \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
            std::exit(2);                                                              \
        }                                                                              \
    } while (0)

constexpr uint32_t kFiniteEnd = 0x7F800000u;  // first non-finite bit pattern
constexpr int kCvtBlocks = 8192, kCvtThreads = 256;

__device__ inline uint32_t code_of_bits(uint32_t u) {
    return e4m3fn_pack4(__uint_as_float(u), 0.0f, 0.0f, 0.0f) & 0xFFu;
}

// Thread i walks a contiguous chunk of bit patterns and compares each code with the previous one.
__global__ void cvt_kernel(uint32_t *first, unsigned long long *counts) {
    const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t chunk = (kFiniteEnd + nthreads - 1) / nthreads;
    const uint64_t begin = i * chunk;
    const uint64_t end = begin + chunk < kFiniteEnd ? begin + chunk : kFiniteEnd;
    if (begin >= end) return;
    uint32_t prev = begin > 0 ? code_of_bits((uint32_t)begin - 1) : 0xFFFFFFFFu;
    unsigned long long bad_mono = 0, bad_sign = 0;
    for (uint64_t b = begin; b < end; ++b) {
        const uint32_t u = (uint32_t)b;
        const float q = __uint_as_float(u);
        const uint32_t both = e4m3fn_pack4(q, -q, 0.0f, 0.0f);
        const uint32_t c = both & 0xFFu, cn = (both >> 8) & 0xFFu;
        if (cn != (c | 0x80u)) ++bad_sign;
        if (prev != 0xFFFFFFFFu && c < prev) ++bad_mono;
        if (c != prev) atomicMin(&first[c], u);
        prev = c;
    }
    if (bad_mono) atomicAdd(&counts[0], bad_mono);
    if (bad_sign) atomicAdd(&counts[1], bad_sign);
}

__device__ inline uint32_t i8(float q) { return int8_code(q); }

// grid (256, n) x 256 lanes: lane j of block (bx, s) takes bf16 pattern bx * 256 + j and scale s.
__global__ void div_kernel(const float *scales, uint8_t *e4m3_out, uint8_t *int8_out,
                           unsigned long long *counts) {
    const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;  // < 65536
    const uint64_t o = (uint64_t)blockIdx.y * 65536u + j;
    const float scale = scales[blockIdx.y];
    const float x = __uint_as_float(j << 16);
    if (!__builtin_isfinite(x)) {
        e4m3_out[o] = 0;
        int8_out[o] = 0;
        return;
    }
    const float q = div_by_scale(x, scale, 1.0f / scale);
    const float ref = x / scale;  // IEEE round-to-nearest division
    const uint32_t ce = e4m3fn_pack4(q, 0.0f, 0.0f, 0.0f) & 0xFFu;
    const uint32_t ci = i8(q);
    e4m3_out[o] = (uint8_t)ce;
    int8_out[o] = (uint8_t)ci;
    const float a = fabsf(ref);
    if (a > 449.0f) return;
    if (a >= 0x1p-11f && __float_as_uint(q) != __float_as_uint(ref)) atomicAdd(&counts[0], 1ull);
    if (ce != (e4m3fn_pack4(ref, 0.0f, 0.0f, 0.0f) & 0xFFu) || ci != i8(ref)) atomicAdd(&counts[1], 1ull);
}

static int run_cvt(const char *out_path) {
    uint32_t *d_first;
    unsigned long long *d_counts;
    CHECK_HIP(hipMalloc(&d_first, 256 * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc(&d_counts, 2 * sizeof(unsigned long long)));
    CHECK_HIP(hipMemset(d_first, 0xFF, 256 * sizeof(uint32_t)));
    CHECK_HIP(hipMemset(d_counts, 0, 2 * sizeof(unsigned long long)));
    hipLaunchKernelGGL(cvt_kernel, dim3(kCvtBlocks), dim3(kCvtThreads), 0, 0, d_first, d_counts);
    CHECK_HIP(hipGetLastError());
    CHECK_HIP(hipDeviceSynchronize());
    uint32_t first[256];
    unsigned long long counts[2];
    CHECK_HIP(hipMemcpy(first, d_first, sizeof(first), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_counts, sizeof(counts), hipMemcpyDeviceToHost));
    FILE *f = std::fopen(out_path, "wb");
    if (!f) return 1;
    std::fwrite(first, sizeof(uint32_t), 256, f);
    std::fwrite(counts, sizeof(unsigned long long), 2, f);
    std::fclose(f);
    CHECK_HIP(hipFree(d_first));
    CHECK_HIP(hipFree(d_counts));
    std::printf("quant_gpu cvt: non-monotone %llu, sign mismatches %llu\n", counts[0], counts[1]);
    return 0;
}

static int run_div(const char *scales_path, const char *out_path, bool write_codes) {
    FILE *f = std::fopen(scales_path, "rb");
    if (!f) return 1;
    std::vector<float> scales;
    float v;
    while (std::fread(&v, sizeof(float), 1, f) == 1) scales.push_back(v);
    std::fclose(f);
    const size_t n = scales.size();
    if (n < 1 || n > 65535) return 1;
    for (float s : scales)
        if (!(s >= kFastDivMinScale && s <= 0x1.fffffep127f)) return 1;  // the fast path's range
    float *d_scales;
    uint8_t *d_e4m3, *d_int8;
    unsigned long long *d_counts;
    CHECK_HIP(hipMalloc(&d_scales, n * sizeof(float)));
    CHECK_HIP(hipMalloc(&d_e4m3, n * 65536));
    CHECK_HIP(hipMalloc(&d_int8, n * 65536));
    CHECK_HIP(hipMalloc(&d_counts, 2 * sizeof(unsigned long long)));
    CHECK_HIP(hipMemcpy(d_scales, scales.data(), n * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_counts, 0, 2 * sizeof(unsigned long long)));
    hipLaunchKernelGGL(div_kernel, dim3(256, (unsigned)n), dim3(256), 0, 0, d_scales, d_e4m3, d_int8,
                       d_counts);
    CHECK_HIP(hipGetLastError());
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<uint8_t> e4m3, int8;
    if (write_codes) {
        e4m3.resize(n * 65536);
        int8.resize(n * 65536);
        CHECK_HIP(hipMemcpy(e4m3.data(), d_e4m3, e4m3.size(), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(int8.data(), d_int8, int8.size(), hipMemcpyDeviceToHost));
    }
    unsigned long long counts[2];
    CHECK_HIP(hipMemcpy(counts, d_counts, sizeof(counts), hipMemcpyDeviceToHost));
    FILE *o = std::fopen(out_path, "wb");
    if (!o) return 1;
    if (write_codes) {
        std::fwrite(e4m3.data(), 1, e4m3.size(), o);
        std::fwrite(int8.data(), 1, int8.size(), o);
    }
    std::fwrite(counts, sizeof(unsigned long long), 2, o);
    std::fclose(o);
    CHECK_HIP(hipFree(d_scales));
    CHECK_HIP(hipFree(d_e4m3));
    CHECK_HIP(hipFree(d_int8));
    CHECK_HIP(hipFree(d_counts));
    std::printf("quant_gpu div: %zu scales, quotient mismatches %llu, code mismatches %llu\n", n,
                counts[0], counts[1]);
    return 0;
}

int main(int argc, char **argv) {
    if (argc == 3 && std::strcmp(argv[1], "cvt") == 0) return run_cvt(argv[2]);
    if (argc == 4 && std::strcmp(argv[1], "div") == 0) return run_div(argv[2], argv[3], true);
    if (argc == 4 && std::strcmp(argv[1], "divcount") == 0) return run_div(argv[2], argv[3], false);
    std::fprintf(stderr, "usage: %s cvt OUT | %s div SCALES OUT | %s divcount SCALES OUT\n", argv[0],
                 argv[0], argv[0]);
    return 1;
}
