// Feature-map kinds and the Omega fragment kernel, shared by the bidirectional and causal
// paths.
#pragma once
#include "favor_device.hpp"

namespace favor {

constexpr int kPrf = 0;
constexpr int kRelu = 1;
constexpr int kTrig = 2;

// Trigonometric feature of a projection in revolutions (the Omega' fragments carry the
// 1/(2 pi)): the first half of the m features are sines, the second half cosines, written
// as one cosine with a quarter-turn phase so that every lane issues one transcendental.
// The hardware cosine takes |a| <= 256 revolutions.
__device__ __forceinline__ float trig_feature(float a, int feature, int m) {
  return __builtin_amdgcn_cosf(a - (feature < (m >> 1) ? 0.25f : 0.f));
}

// Scale folded into the Omega' fragments: d^-1/4, times log2(e) for the exponential map (the
// hardware exp2) or 1/(2 pi) for the trigonometric map (the hardware cosine takes revolutions).
inline float omega_scale(int kind, float sc) {
  return kind == kPrf ? sc * kLog2e : (kind == kTrig ? sc * 0.15915494309189535f : sc);
}

// ---------------------------------------------------------------- omega fragments
// frag[h][fb][dc][lane][j] = scale * omega[h][fb*16 + c][dc*32 + 8g + j] (0 beyond d),
// which is both the B operand (k = d, n = feature) of the key projection and the
// A operand (row = feature, k = d) of the transposed query projection.
// residual != 0 writes instead what rounding to T left out, x - (float)(T)x rounded to T: a
// projection through both fragment sets (two MFMAs) sees the fp32 value to about 2^-22.
// mk >= m (a multiple of 16) is the feature count of the kernels that read the fragments: rows
// m..mk-1 are zero.
template <typename T>
__global__ void omega_frag_kernel(const float* __restrict__ omega, int H, int m, int mk, int d, float scale,
                                  T* __restrict__ frag, int residual) {
  const int dc_n = (d + 31) / 32;
  const long long total = (long long)H * (mk / 16) * dc_n * 64;
  for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(id & 63);
    unsigned rest = (unsigned)(id >> 6);  // (h, fb, dc): at most 2^31 for the shapes the ABI accepts
    const int dc = (int)(rest % (unsigned)dc_n);
    rest /= (unsigned)dc_n;
    const int fb = (int)(rest % (unsigned)(mk / 16));
    const int h = (int)(rest / (unsigned)(mk / 16));
    const int c = lane & 15, g = lane >> 4;
    const int r = fb * 16 + c;
    const float* row = omega + ((size_t)h * m + (r < m ? r : 0)) * d;
    vec8<T> x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = dc * 32 + 8 * g + j;
      const float v = (col < d && r < m) ? row[col] * scale : 0.f;
      x[j] = residual ? to_t<T>(v - to_f(to_t<T>(v))) : to_t<T>(v);
    }
    st8<T>(frag + (size_t)id * 8, x);
  }
}

}  // namespace favor
