// One recurrent decode step of causal FAVOR+ for N sequences x H heads.
//
// The causal sums advanced by one token (linear-attention blog, "Autoregressive
// Generation"; RFA summary page, appendix A.3):
//   S <- S + phi(k) v^T,  z <- z + phi(k),  out = phi(q).S / phi(q).z
// with the updated state (token t's output includes token t).
//
// The state S [N,H,m,dv] fp32 dominates the traffic: each step reads and writes it
// once, so the kernel is an HBM stream. Work split: one workgroup per (head, group
// of G sequences).
//   phase 1  thread r holds omega_r of its head in registers and computes
//            a = omega_r . x for the group's q and k (fp32 FMA). Keys use the
//            canonical feature exp(a - |x|^2/2)/sqrt(m) because the state is kept
//            unstabilised; queries use exp(a - max_r a), a per-row constant that
//            cancels in the ratio. phi is staged in LDS.
//   phase 2  per sequence, the state block is streamed with 16-byte loads and
//            stores: consecutive threads cover consecutive columns of one row, so
//            a wave touches whole rows; the numerator is accumulated on the fly
//            from the updated rows and reduced across row groups through LDS.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

constexpr int kDecodeThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
              const float* __restrict__ omega, float* __restrict__ S, float* __restrict__ z, int N, int H,
              int dv, int m, int G, int n_groups, int kind, float eps, float inv_sqrt_m, float wscale,
              float nscale, float log2_sqrt_m, float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  // layout: aq[G][m], ak[G][m] (features after phase 1), xs[2][G][D] (q, k as fp32),
  //         red[256][4] (numerator partials), scal[G][4]
  float* aq = sm;
  float* ak = aq + G * m;
  float* xs = ak + G * m;
  float* red = xs + 2 * G * D;
  float* scal = red + kDecodeThreads * 4;
  __shared__ float dsum[kDecodeThreads / 64];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int h = logical / n_groups, grp = logical % n_groups;
  const int s0 = grp * G;
  const int ng = min(G, N - s0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  // stage q and k of the group as fp32
  for (int i = tid; i < 2 * G * D; i += kDecodeThreads) {
    const int which = i / (G * D), rem = i % (G * D), s = rem / D, dd = rem % D;
    float x = 0.f;
    if (s < ng) {
      const T* src = which == 0 ? q : k;
      x = to_f(src[((size_t)(s0 + s) * H + h) * D + dd]);
    }
    xs[i] = x;
  }
  __syncthreads();

  // phase 1: projections a = omega' . x
  for (int r = tid; r < m; r += kDecodeThreads) {
    float w[D];
    const f32x4* wr = reinterpret_cast<const f32x4*>(omega + ((size_t)h * m + r) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const f32x4 t = wr[i];
      w[4 * i] = t[0] * wscale;
      w[4 * i + 1] = t[1] * wscale;
      w[4 * i + 2] = t[2] * wscale;
      w[4 * i + 3] = t[3] * wscale;
    }
    for (int s = 0; s < G; ++s) {
      const float* xq = xs + s * D;
      const float* xk = xs + (G + s) * D;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int dd = 0; dd < D; ++dd) {
        a0 += w[dd] * xq[dd];
        a1 += w[dd] * xk[dd];
      }
      aq[s * m + r] = a0;
      ak[s * m + r] = a1;
    }
  }
  __syncthreads();

  // per-sequence scalars: query row max (PRF) and the key's log2 normaliser
  if (kind == 0) {
    for (int s = wv; s < G; s += kDecodeThreads / 64) {
      float mx = -INFINITY;
      for (int r = lane; r < m; r += 64) mx = fmaxf(mx, aq[s * m + r]);
      mx = wave_max(mx);
      float k2 = 0.f;
      for (int dd = lane; dd < D; dd += 64) {
        const float x = xs[(G + s) * D + dd];
        k2 += x * x;
      }
      k2 = wave_sum(k2);
      if (lane == 0) {
        scal[s * 4 + 0] = mx;
        scal[s * 4 + 1] = k2 * nscale + log2_sqrt_m;
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < G * m; i += kDecodeThreads) {
    const int s = i / m;
    if (kind == 0) {
      aq[i] = fast_exp2(aq[i] - scal[s * 4 + 0]);
      ak[i] = fast_exp2(ak[i] - scal[s * 4 + 1]);
    } else {
      aq[i] = fmaxf(aq[i], 0.f) * inv_sqrt_m + eps;
      ak[i] = fmaxf(ak[i], 0.f) * inv_sqrt_m + eps;
    }
  }
  __syncthreads();

  // phase 2: stream the state
  const int tpr = dv / 4;                 // threads per row (power of two, <= 64)
  const int rpp = kDecodeThreads / tpr;   // rows per pass
  const int col4 = tid % tpr, row0 = tid / tpr;
  for (int s = 0; s < ng; ++s) {
    const size_t pair = (size_t)(s0 + s) * H + h;
    float* Sp = S + pair * m * dv;
    float* zp = z + pair * m;
    const float* pq = aq + s * m;
    const float* pk = ak + s * m;
    f32x4 vv;
    {
      const T* vs = v + pair * dv + col4 * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = to_f(vs[i]);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < m; r0 += 8 * rpp) {
      f32x4 st[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + u * rpp + row0;
        if (r < m) st[u] = *reinterpret_cast<const f32x4*>(Sp + (size_t)r * dv + col4 * 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + u * rpp + row0;
        if (r < m) {
          const float fk = pk[r], fq = pq[r];
          st[u] += fk * vv;
          acc += fq * st[u];
          *reinterpret_cast<f32x4*>(Sp + (size_t)r * dv + col4 * 4) = st[u];
        }
      }
    }
    float dpart = 0.f;
    for (int r = tid; r < m; r += kDecodeThreads) {
      const float zn = zp[r] + pk[r];
      zp[r] = zn;
      dpart += pq[r] * zn;
    }
    dpart = wave_sum(dpart);
    *reinterpret_cast<f32x4*>(red + tid * 4) = acc;
    if (lane == 0) dsum[wv] = dpart;
    __syncthreads();
    if (tid < dv) {
      const int cc = tid / 4, ii = tid % 4;
      float num = 0.f;
      for (int rg = 0; rg < rpp; ++rg) num += red[(rg * tpr + cc) * 4 + ii];
      float den = 0.f;
#pragma unroll
      for (int i = 0; i < kDecodeThreads / 64; ++i) den += dsum[i];
      out[pair * dv + tid] = num / den;
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t run_decode(const T* q, const T* k, const T* v, const float* omega, float* S, float* z, int N, int H,
                             int dv, int m, int kind, float eps, float* out, hipStream_t st) {
  const int G = 4;
  const int n_groups = (N + G - 1) / G;
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = (kind == 0) ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float log2_sqrt_m = 0.5f * std::log2((float)m);
  const float inv_sqrt_m = 1.0f / std::sqrt((float)m);
  const size_t lds = (size_t)(2 * G * m + 2 * G * D + kDecodeThreads * 4 + G * 4) * sizeof(float);
  {
    FAVOR_TIMED("decode", st);
    decode_kernel<T, D><<<(unsigned)(H * n_groups), kDecodeThreads, lds, st>>>(
        q, k, v, omega, S, z, N, H, dv, m, G, n_groups, kind, eps, inv_sqrt_m, wscale, nscale, log2_sqrt_m, out);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* omega, float* S, float* z,
                         int N, int H, int d, int dv, int m, int dtype, int kind, float eps, float* out,
                         hipStream_t st) {
#define DEC(D_)                                                                                                 \
  if (d == D_) {                                                                                                \
    if (dtype == 0)                                                                                             \
      return run_decode<float, D_>(static_cast<const float*>(q), static_cast<const float*>(k),                  \
                                   static_cast<const float*>(v), omega, S, z, N, H, dv, m, kind, eps, out, st); \
    return run_decode<bf16, D_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),                       \
                                static_cast<const bf16*>(v), omega, S, z, N, H, dv, m, kind, eps, out, st);     \
  }
  DEC(16)
  DEC(32)
  DEC(64)
#undef DEC
  return hipErrorInvalidValue;
}

}  // namespace favor
