// Issue rates of the three pipes the FAVOR+ kernels lean on, measured on the device:
// the transcendental v_exp_f32 (one per token-feature for the positive features), the fp32
// FMA on the vector ALU, and the bf16 16x16x32 MFMA. Each test runs independent dependency
// chains in every lane (enough of them to cover the pipe latency) on two (or more) waves per
// SIMD of 256 CUs, times itself with the shader clock (clock64) per wave and with HIP
// events, and prints instructions per SIMD per clock and per second. A mixed test issues
// exp and MFMA chains together to show whether the two pipes overlap.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         random_feature_amd/tools/rates.hip -o rates && ./rates
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef RATES_CHAINS
#define RATES_CHAINS 8
#endif
#ifndef RATES_WAVES_PER_SIMD
#define RATES_WAVES_PER_SIMD 2
#endif
constexpr int kChains = RATES_CHAINS;  // independent chains per lane
constexpr int kIters = 4096;           // loop iterations (each issues kChains instructions per chain kind)
constexpr int kWps = RATES_WAVES_PER_SIMD;
constexpr int kWaves = 1024 * kWps;    // on 256 CUs x 4 SIMDs
constexpr int kBlock = 256;

// every kernel writes one value per lane (so nothing is optimised away) and its wave's clock span
__global__ void __launch_bounds__(kBlock) exp_chain(float* out, long long* cyc, float seed) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = seed + 0.01f * c + 1e-6f * threadIdx.x;
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);  // stays in [1/2, 1]
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kBlock + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[(blockIdx.x * kBlock + threadIdx.x) >> 6] = t1 - t0;
}

__global__ void __launch_bounds__(kBlock) fma_chain(float* out, long long* cyc, float seed) {
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = seed + 0.01f * c + 1e-6f * threadIdx.x;
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_fmaf(x[c], 0.999f, 0.0001f);
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kBlock + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[(blockIdx.x * kBlock + threadIdx.x) >> 6] = t1 - t0;
}

#ifndef RATES_ACC
#define RATES_ACC 4
#endif
constexpr int kAcc = RATES_ACC;  // independent MFMA accumulators per wave
__global__ void __launch_bounds__(kBlock) mfma_chain(float* out, long long* cyc, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed + 0.001f * j);
    b[j] = (__bf16)(0.5f - 0.001f * j);
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int c = 0; c < kAcc; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < kAcc; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kAcc; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * kBlock + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[(blockIdx.x * kBlock + threadIdx.x) >> 6] = t1 - t0;
}

// kAcc MFMAs and kChains exps per iteration, independent of each other
__global__ void __launch_bounds__(kBlock) mixed_chain(float* out, long long* cyc, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed + 0.001f * j);
    b[j] = (__bf16)(0.5f - 0.001f * j);
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int c = 0; c < kAcc; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = seed + 0.01f * c + 1e-6f * threadIdx.x;
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < kAcc; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kAcc; ++c) s += acc[c][0];
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kBlock + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[(blockIdx.x * kBlock + threadIdx.x) >> 6] = t1 - t0;
}

// kAcc MFMAs and 2*kChains FMAs per iteration, independent of each other
__global__ void __launch_bounds__(kBlock) mixed_fma_chain(float* out, long long* cyc, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed + 0.001f * j);
    b[j] = (__bf16)(0.5f - 0.001f * j);
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int c = 0; c < kAcc; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) x[c] = seed + 0.01f * c + 1e-6f * threadIdx.x;
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < kAcc; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_fmaf(x[c], 0.999f, 0.0001f);
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = __builtin_fmaf(x[c], 0.999f, 0.0001f);
  }
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kAcc; ++c) s += acc[c][0];
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += x[c];
  out[blockIdx.x * kBlock + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[(blockIdx.x * kBlock + threadIdx.x) >> 6] = t1 - t0;
}

typedef void (*Kern)(float*, long long*, float);

static int run(const char* name, Kern k, double instr_per_wave, const char* unit) {
  float* out = nullptr;
  long long* cyc = nullptr;
  if (hipMalloc(&out, sizeof(float) * kWaves * 64) != hipSuccess) return 1;
  if (hipMalloc(&cyc, sizeof(long long) * kWaves) != hipSuccess) return 1;
  const int grid = kWaves * 64 / kBlock;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  k<<<grid, kBlock>>>(out, cyc, 0.3f);  // warm-up
  if (hipEventRecord(e0) != hipSuccess) return 1;
  k<<<grid, kBlock>>>(out, cyc, 0.4f);
  if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
  std::vector<long long> c(kWaves);
  if (hipMemcpy(c.data(), cyc, sizeof(long long) * kWaves, hipMemcpyDeviceToHost) != hipSuccess) return 1;
  double mean = 0.0;
  for (long long x : c) mean += (double)x;
  mean /= kWaves;
  // kWps waves share each SIMD for the whole run: per-SIMD issue rate = kWps * per-wave instructions / cycles
  const double per_simd_clk = kWps * instr_per_wave / mean;
  const double per_s = kWaves * instr_per_wave / (ms * 1e-3);
  printf("%-6s %8.3f ms  %8.0f cycles/wave  %.3f %s per SIMD per clock  %.3e %s/s (device)  clock %.2f GHz\n", name, ms,
         mean, per_simd_clk, unit, per_s, unit, mean / (ms * 1e-3) / 1e9);
  (void)hipFree(out);
  (void)hipFree(cyc);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

int main() {
  int rc = 0;
  rc |= run("exp", exp_chain, (double)kIters * kChains, "v_exp_f32 wave-instr");
  rc |= run("fma", fma_chain, (double)kIters * kChains, "v_fma_f32 wave-instr");
  rc |= run("mfma", mfma_chain, (double)kIters * kAcc, "mfma_16x16x32_bf16");
  rc |= run("mixed", mixed_chain, (double)kIters * kAcc, "mfma_16x16x32_bf16 (+2 exp each)");
  rc |= run("mixfma", mixed_fma_chain, (double)kIters * kAcc, "mfma_16x16x32_bf16 (+4 fma each)");
  printf("status %s\n", rc ? "error" : "ok");
  return rc;
}
