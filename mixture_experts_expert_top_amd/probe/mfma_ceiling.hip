// Sustained MFMA rate of the whole chip, for the roofline's measured ceiling.
//
// Every CU runs 8 waves (two per SIMD) that issue nothing but independent
// MFMAs: bf16 32x32x16 or block-scaled E4M3 32x32x64 (scale 1), 8
// accumulators a wave.  The operands are either constant or random (random
// sign and mantissa, bounded exponents: no NaN or Inf codes).  The clock is
// power-limited, and operand bit toggling costs power, so the random case
// is the ceiling that a GEMM on training data can approach.  Each
// workgroup also reads the shader clock (s_memtime) against the 100 MHz
// real-time counter (s_memrealtime) around its loop.
//
// Output: one line per case,
//   <dtype> <operands> <iters> <ms> <TFLOP/s> <GHz>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kBlocks = 256;    // one workgroup a CU
constexpr int kThreads = 512;   // 8 waves

__device__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU;
  return x ^ (x >> 16);
}

// bf16 with random sign and mantissa, binade 2^-3 .. 2^1
__device__ __bf16 rand_bf16(uint32_t h) {
  const uint32_t e = 124u + (h >> 8) % 5u;
  return __builtin_bit_cast(__bf16, static_cast<uint16_t>((h & 0x807fu) | (e << 7)));
}

// four E4M3 codes with random sign and mantissa, exponent field 4..11
__device__ uint32_t rand_e4m3x4(uint32_t h) {
  uint32_t w = 0;
  for (int q = 0; q < 4; ++q) {
    const uint32_t r = mix32(h + 0x9e3779b9u * (q + 1));
    w |= (((r & 0x87u) | ((4u + (r >> 8) % 8u) << 3)) & 0xffu) << (8 * q);
  }
  return w;
}

template <bool kFp8, bool kRandom>
__global__ __launch_bounds__(kThreads) void mfma_loop(int iters, float* sink,
                                                      unsigned long long* clk) {
  const int tid = threadIdx.x;
  const uint32_t seed = (blockIdx.x * kThreads + tid) * 64u;
  f32x16 c[8] = {};
  unsigned long long r0, t0, t1, r1;
  if constexpr (kFp8) {
    i32x8 a[4], b[4];
    for (int s = 0; s < 4; ++s)
      for (int i = 0; i < 8; ++i) {
        a[s][i] = static_cast<int>(kRandom ? rand_e4m3x4(mix32(seed + s * 8 + i)) : 0x38383838u);
        b[s][i] = static_cast<int>(kRandom ? rand_e4m3x4(mix32(~(seed + s * 8 + i))) : 0x30303030u);
      }
    r0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < 8; ++m)
          c[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              a[m & 3], b[(m >> 2) + 2 * h], c[m], 0, 0, 0, 127, 0, 127);
    }
    t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
  } else {
    bf16x8 a[4], b[4];
    for (int s = 0; s < 4; ++s)
      for (int i = 0; i < 8; ++i) {
        a[s][i] = kRandom ? rand_bf16(mix32(seed + s * 8 + i)) : (__bf16)(0.001f * (tid % 64 + i));
        b[s][i] = kRandom ? rand_bf16(mix32(~(seed + s * 8 + i))) : (__bf16)(0.002f * (i + 1));
      }
    r0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < 8; ++m)
          c[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              a[m & 3], b[(m >> 2) + 2 * h], c[m], 0, 0, 0);
    }
    t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  float sum = 0.0f;
  for (int m = 0; m < 8; ++m)
    for (int q = 0; q < 16; ++q) sum += c[m][q];
  sink[blockIdx.x * kThreads + tid] = sum;   // keeps every MFMA live
  if (tid == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

#define CHECK(x)                                                           \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));         \
      std::exit(1);                                                        \
    }                                                                      \
  } while (0)

template <bool kFp8, bool kRandom>
void run(int iters, float* sink, unsigned long long* clk) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  // a short launch first, so clocks and caches are settled
  hipLaunchKernelGGL((mfma_loop<kFp8, kRandom>), dim3(kBlocks), dim3(kThreads), 0, 0,
                     iters / 10, sink, clk);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL((mfma_loop<kFp8, kRandom>), dim3(kBlocks), dim3(kThreads), 0, 0,
                     iters, sink, clk);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.0f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long h[2 * kBlocks];
  CHECK(hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost));
  double ghz = 0.0;
  for (int i = 0; i < kBlocks; ++i)
    ghz += static_cast<double>(h[2 * i]) / (static_cast<double>(h[2 * i + 1]) * 10.0);
  ghz /= kBlocks;
  const double k = kFp8 ? 64.0 : 16.0;
  const double flops = 2.0 * 32 * 32 * k * 8.0 * iters * (kThreads / 64) * kBlocks;
  std::printf("%s %s %d %.3f %.1f %.3f\n", kFp8 ? "fp8" : "bf16",
              kRandom ? "random" : "constant", iters, ms,
              flops / (ms * 1e-3) / 1e12, ghz);
  std::fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

}  // namespace

int main() {
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&sink, sizeof(float) * kBlocks * kThreads));
  CHECK(hipMalloc(&clk, sizeof(unsigned long long) * 2 * kBlocks));
  // about 50 ms (bf16) and 100 ms (fp8) a launch
  run<false, false>(200000, sink, clk);
  run<false, true>(200000, sink, clk);
  run<true, false>(200000, sink, clk);
  run<true, true>(200000, sink, clk);
  CHECK(hipFree(sink));
  CHECK(hipFree(clk));
  return 0;
}
