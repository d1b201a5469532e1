// Sustained dense MFMA rate of the whole chip, as a measured ceiling beside
// the published peaks: every CU runs two workgroups of four waves (two waves
// per SIMD, the fused kernels' occupancy) issuing back-to-back
// v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x64_f8f6f4 on register
// operands, with no memory traffic inside the timed loop.  The chip's clock
// under such load depends on how much the operand bits toggle, so the
// operands are either one constant pair per lane or eight pairs of random
// values (random signs and mantissas, as attention inputs have) used in
// rotation.  Prints one JSON line per case: TFLOP/s from HIP events and the
// shader clock from the cycle and real-time counters of one wave.  Two more
// cases give the vector unit's rates at the same occupancy, in lane
// operations per second: v_exp_f32 (the exponential every attention score
// needs) and v_fma_f32, each on eight independent dependency chains.
//
// Standalone measurement program (not part of libiofa.so).  Every lane
// writes only out[blockIdx.x * blockDim.x + threadIdx.x]; lane 0 of block 0
// writes the two counters.  All loops have fixed trip counts.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                    \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                 \
    }                                                                               \
  } while (0)

__device__ inline unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
// bf16 with random sign and mantissa, magnitude in [2^-3, 2^3)
__device__ inline unsigned short rand_bf16(unsigned h) {
  return static_cast<unsigned short>(((h >> 31) << 15) | ((124u + h % 6u) << 7) | ((h >> 8) & 0x7Fu));
}
// E4M3 code with random sign and mantissa, exponent field 4..10 (finite)
__device__ inline unsigned rand_e4m3(unsigned h) {
  return ((h >> 31) << 7) | ((4u + h % 7u) << 3) | ((h >> 8) & 7u);
}

constexpr int kAcc = 4;

template <int NOP>
__global__ __launch_bounds__(256, 2) void bf16_kernel(float* out, int iters,
                                                      unsigned long long* clk) {
  const unsigned id = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[NOP], b[NOP];
  for (int i = 0; i < NOP; ++i) {
    u16x8 ua, ub;
    for (int e = 0; e < 8; ++e) {
      ua[e] = rand_bf16(mix(id * 131u + i * 17u + e));
      ub[e] = rand_bf16(mix(id * 977u + i * 29u + e + 7u));
    }
    a[i] = __builtin_bit_cast(bf16x8, ua);
    b[i] = __builtin_bit_cast(bf16x8, ub);
  }
  f32x16 acc[kAcc];
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x16{};
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NOP; ++i)
#pragma unroll
      for (int j = 0; j < kAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + j) % NOP], acc[j], 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < kAcc; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[id] = s;
  if (id == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
}

template <int NOP>
__global__ __launch_bounds__(256, 2) void fp8_kernel(float* out, int iters,
                                                     unsigned long long* clk) {
  const unsigned id = blockIdx.x * blockDim.x + threadIdx.x;
  i32x8 a[NOP], b[NOP];
  for (int i = 0; i < NOP; ++i)
    for (int w = 0; w < 8; ++w) {
      unsigned wa = 0, wb = 0;
      for (int e = 0; e < 4; ++e) {
        wa |= rand_e4m3(mix(id * 131u + i * 37u + w * 4u + e)) << (8 * e);
        wb |= rand_e4m3(mix(id * 977u + i * 41u + w * 4u + e + 5u)) << (8 * e);
      }
      a[i][w] = static_cast<int>(wa);
      b[i][w] = static_cast<int>(wb);
    }
  f32x16 acc[kAcc];
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x16{};
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NOP; ++i)
#pragma unroll
      for (int j = 0; j < kAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[(i + j) % NOP], acc[j], 0,
                                                                 0, 0, 0, 0, 0);
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < kAcc; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[id] = s;
  if (id == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
}

// NCH independent chains of v_exp_f32 (x <- -exp2(x) stays in [-1, -0.5])
// or v_fma_f32 (x <- 0.999 x + 0.001 stays near 1).
template <bool EXP>
__global__ __launch_bounds__(256, 2) void valu_kernel(float* out, int iters,
                                                      unsigned long long* clk) {
  constexpr int NCH = 8;
  const unsigned id = blockIdx.x * blockDim.x + threadIdx.x;
  float x[NCH];
  for (int j = 0; j < NCH; ++j) x[j] = -0.6f - 0.01f * j - 1e-7f * (id & 1023);
  const unsigned long long c0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
      x[j] = EXP ? -__builtin_amdgcn_exp2f(x[j]) : __builtin_fmaf(x[j], 0.999f, 0.001f);
  }
  const unsigned long long c1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int j = 0; j < NCH; ++j) s += x[j];
  out[id] = s;
  if (id == 0) {
    clk[0] = c1 - c0;
    clk[1] = r1 - r0;
  }
}

typedef void (*KernelFn)(float*, int, unsigned long long*);

void run(const char* name, KernelFn fn, double flops_per_mfma, int mfma_per_iter,
         double peak_tflops, float* out, unsigned long long* clk, int blocks, int iters) {
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, 0, out, 2, clk);   // warm-up
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, 0, out, iters, clk);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipGetLastError());
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long h[2];
  CHECK(hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost));
  const double waves = 4.0 * blocks;
  const double tflops = flops_per_mfma * mfma_per_iter * iters * waves / (ms * 1e-3) / 1e12;
  // s_memrealtime counts at 100 MHz
  const double mhz = h[1] ? 100.0 * static_cast<double>(h[0]) / static_cast<double>(h[1]) : 0.0;
  std::printf("{\"case\": \"%s\", \"ms\": %.3f, \"tflops\": %.1f, \"frac_of_published_peak\": %.4f, "
              "\"shader_clock_mhz\": %.0f}\n",
              name, ms, tflops, tflops / peak_tflops, mhz);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

void run_valu(const char* name, KernelFn fn, float* out, unsigned long long* clk, int blocks,
              int iters) {
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, 0, out, 2, clk);   // warm-up
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, 0, out, iters, clk);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  CHECK(hipGetLastError());
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long h[2];
  CHECK(hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost));
  const double lane_ops = 8.0 * iters * 256.0 * blocks;
  const double mhz = h[1] ? 100.0 * static_cast<double>(h[0]) / static_cast<double>(h[1]) : 0.0;
  std::printf("{\"case\": \"%s\", \"ms\": %.3f, \"lane_ops_per_s\": %.4e, "
              "\"lanes_per_clock_per_simd\": %.2f, \"shader_clock_mhz\": %.0f}\n",
              name, ms, lane_ops / (ms * 1e-3),
              mhz > 0 ? lane_ops / (ms * 1e-3) / (1024.0 * mhz * 1e6) : 0.0, mhz);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

}  // namespace

int main() {
  const int blocks = 512;   // two workgroups per CU on 256 CUs
  {
    // what the runtime reports for device 0: its name and its peak clocks
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    printf("{\"device\": \"%s\", \"arch\": \"%s\", \"compute_units\": %d, "
           "\"max_shader_clock_mhz\": %d, \"memory_clock_mhz\": %d, \"memory_bus_bits\": %d}\n",
           prop.name, prop.gcnArchName, prop.multiProcessorCount, prop.clockRate / 1000,
           prop.memoryClockRate / 1000, prop.memoryBusWidth);
    fflush(stdout);
  }
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&out, blocks * 256 * sizeof(float)));
  CHECK(hipMalloc(&clk, 2 * sizeof(unsigned long long)));
  const double bf16_mfma = 2.0 * 32 * 32 * 16, fp8_mfma = 2.0 * 32 * 32 * 64;
  run("bf16 32x32x16, constant operands", bf16_kernel<1>, bf16_mfma, kAcc, 2516.6, out, clk,
      blocks, 20000);
  run("bf16 32x32x16, 8 random operand pairs", bf16_kernel<8>, bf16_mfma, 8 * kAcc, 2516.6, out,
      clk, blocks, 2500);
  run("fp8 e4m3 32x32x64, 8 random operand pairs", fp8_kernel<8>, fp8_mfma, 8 * kAcc, 5033.2, out,
      clk, blocks, 1250);
  run_valu("v_exp_f32, 8 chains per lane", valu_kernel<true>, out, clk, blocks, 20000);
  run_valu("v_fma_f32, 8 chains per lane", valu_kernel<false>, out, clk, blocks, 40000);
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}
