// Kernels shared by the bidirectional and causal paths: Omega fragments and the
// per-segment reduction S_aug = Phi_K^T [V 1] (Performer paper, Algorithm 1, Buf1).
#pragma once
#include "favor_device.hpp"

namespace favor {

constexpr int kPrf = 0;
constexpr int kRelu = 1;

// ---------------------------------------------------------------- omega fragments
// frag[h][fb][dc][lane][j] = scale * omega[h][fb*16 + c][dc*32 + 8g + j] (0 beyond d),
// which is both the B operand (k = d, n = feature) of the key projection and the
// A operand (row = feature, k = d) of the transposed query projection.
template <typename T>
__global__ void omega_frag_kernel(const float* __restrict__ omega, int H, int m, int d, float scale,
                                  T* __restrict__ frag) {
  const int dc_n = (d + 31) / 32;
  const long long total = (long long)H * (m / 16) * dc_n * 64;
  for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(id & 63);
    long long rest = id >> 6;
    const int dc = (int)(rest % dc_n);
    rest /= dc_n;
    const int fb = (int)(rest % (m / 16));
    const int h = (int)(rest / (m / 16));
    const int c = lane & 15, g = lane >> 4;
    const float* row = omega + ((size_t)h * m + fb * 16 + c) * d;
    vec8<T> x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = dc * 32 + 8 * g + j;
      x[j] = to_t<T>(col < d ? row[col] * scale : 0.f);
    }
    st8<T>(frag + id * 8, x);
  }
}

// ---------------------------------------------------------------- reduce
// Workgroup (segment, b*h): NW waves, wave w owns features [w*FB*16, (w+1)*FB*16)
// and all tokens of the segment. Per 32-token tile the workgroup stages K (row
// major) and V (transposed, token pairs packed) in LDS; each wave then
//   projects its features        A = K tile (rows = tokens), B = Omega'  -> a'[token][feature]
//   applies the feature map      PRF: exp2(a' - n'_t - M_w) with n'_t = log2e |x_t|^2 / 2 and
//                                M_w the wave's running max of a' - n' (accumulators are
//                                rescaled when it grows); ReLU: max(a,0)/sqrt(m) + eps
//   accumulates S_aug            A = Phi^T (paired slot map, straight from the accumulators),
//                                B = [V 1] (paired slot map, read from the transposed tile)
// and finally writes its FB*16 rows of S_aug plus M_w.
template <typename T, int D, int DV, int M, int FB>
__global__ void __launch_bounds__(64 * (M / (16 * FB)))
reduce_kernel(const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ omf, int H, int L,
              int seg_len, int nseg, int kind, float eps, float inv_sqrt_m, float nscale,
              float* __restrict__ part, float* __restrict__ pmax) {
  constexpr int NW = M / (16 * FB);
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;
  constexpr int KROW = D + 8;
  constexpr int VROW = 32 + 8;
  __shared__ __attribute__((aligned(16))) T ks[32 * KROW];
  __shared__ __attribute__((aligned(16))) T vts[DV * VROW];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
  const int tbeg = seg * seg_len, tend = min(L, tbeg + seg_len);
  const T* Kb = K + (size_t)bh * L * D;
  const T* Vb = V + (size_t)bh * L * DV;

  vec8<T> om[FB][DC];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      om[fb][dc] = ld8<T>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);

  f32x4 sacc[FB][NB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float runmax = -INFINITY;

  vec8<T> ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = to_t<T>(c == 0 ? 1.f : 0.f);

  for (int t0 = tbeg; t0 < tend; t0 += 32) {
    __syncthreads();
    constexpr int KCH = 32 * D / 8;
    for (int q = threadIdx.x; q < KCH; q += NW * 64) {
      const int row = q / (D / 8), col = (q % (D / 8)) * 8;
      const vec8<T> x = (t0 + row < tend) ? ld8<T>(Kb + (size_t)(t0 + row) * D + col) : zero8<T>();
      st8<T>(ks + row * KROW + col, x);
    }
    constexpr int VCH = 16 * (DV / 8);
    for (int q = threadIdx.x; q < VCH; q += NW * 64) {
      const int tp = q / (DV / 8), col = (q % (DV / 8)) * 8;
      const int t = t0 + 2 * tp;
      const vec8<T> a = (t < tend) ? ld8<T>(Vb + (size_t)t * DV + col) : zero8<T>();
      const vec8<T> b = (t + 1 < tend) ? ld8<T>(Vb + (size_t)(t + 1) * DV + col) : zero8<T>();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vec2<T> pr;
        pr[0] = a[e];
        pr[1] = b[e];
        *reinterpret_cast<vec2<T>*>(vts + (col + e) * VROW + 2 * tp) = pr;
      }
    }
    __syncthreads();

    // key fragments and squared norms
    vec8<T> kf[2][DC];
    float nrm[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float s2 = 0.f;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[tb][dc] = (col < D) ? ld8<T>(ks + (tb * 16 + c) * KROW + col) : zero8<T>();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = to_f(kf[tb][dc][j]);
          s2 += x * x;
        }
      }
      nrm[tb] = group_sum(s2) * nscale;
    }

    f32x4 pacc[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pacc[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(pacc[tb][fb], kf[tb][dc], om[fb][dc]);
      }

    // pacc[tb][fb][i] is a' for token t0 + tb*16 + 4g + i, feature (w*FB + fb)*16 + c
    if (kind == kPrf) {
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float nt = __shfl(nrm[tb], 4 * g + i, 64);
          const bool ok = t0 + tb * 16 + 4 * g + i < tend;
#pragma unroll
          for (int fb = 0; fb < FB; ++fb) {
            const float e = ok ? pacc[tb][fb][i] - nt : -INFINITY;
            pacc[tb][fb][i] = e;
            tmax = fmaxf(tmax, e);
          }
        }
      tmax = wave_max(tmax);
      if (tmax > runmax) {
        const float sc = fast_exp2(runmax - tmax);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] *= sc;
        runmax = tmax;
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = fast_exp2(pacc[tb][fb][i] - runmax);
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = t0 + tb * 16 + 4 * g + i < tend;
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
            pacc[tb][fb][i] = ok ? fmaxf(pacc[tb][fb][i], 0.f) * inv_sqrt_m + eps : 0.f;
        }
    }

    vec8<T> af[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int j = 0; j < 8; ++j) af[fb][j] = to_t<T>(pacc[j >> 2][fb][j & 3]);

    vec8<T> vf[NB];
#pragma unroll
    for (int nb = 0; nb < NB - 1; ++nb) {
      const T* row = vts + (nb * 16 + c) * VROW;
      const vec4<T> lo = *reinterpret_cast<const vec4<T>*>(row + 4 * g);
      const vec4<T> hi = *reinterpret_cast<const vec4<T>*>(row + 16 + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[nb][j] = lo[j];
        vf[nb][j + 4] = hi[j];
      }
    }
    vf[NB - 1] = ones;

#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma16(sacc[fb][nb], af[fb], vf[nb]);
  }

  // sacc[fb][nb][i] = S_aug[feature (w*FB+fb)*16 + 4g + i][column nb*16 + c]
  float* P = part + ((size_t)bh * nseg + seg) * M * (DV + 1);
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (w * FB + fb) * 16 + 4 * g + i;
#pragma unroll
      for (int nb = 0; nb < NB - 1; ++nb) P[(size_t)r * (DV + 1) + nb * 16 + c] = sacc[fb][nb][i];
      if (c == 0) P[(size_t)r * (DV + 1) + DV] = sacc[fb][NB - 1][i];
    }
  if (lane == 0) pmax[((size_t)bh * nseg + seg) * NW + w] = (kind == kPrf) ? runmax : 0.f;
}

}  // namespace favor
