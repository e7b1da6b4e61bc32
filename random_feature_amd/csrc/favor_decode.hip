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

constexpr int kDecodeGroup = 4;  // sequences per workgroup
constexpr int kDecodeRows = 8;   // state rows per thread per batch (loads in flight)

template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
              const float* __restrict__ omega, float* __restrict__ S, float* __restrict__ z, int N, int H,
              int dv, int m, int n_groups, int kind, float eps, float inv_sqrt_m, float wscale,
              float nscale, float log2_sqrt_m, float* __restrict__ out) {
  constexpr int G = kDecodeGroup, U = kDecodeRows;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  // layout: aq[G][m], ak[G][m] (features after phase 1), xs[2][G][D] (q, k as fp32),
  //         red[G][256][4] (numerator partials), scal[G][4]
  float* aq = sm;
  float* ak = aq + G * m;
  float* xs = ak + G * m;
  float* red = xs + 2 * G * D;
  float* scal = red + G * kDecodeThreads * 4;
  __shared__ float dsum[G][kDecodeThreads / 64];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int h = logical / n_groups, grp = logical % n_groups;
  const int s0 = grp * G;
  const int ng = min(G, N - s0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  // the state stream: batch i covers rows [b*U*rpp, (b+1)*U*rpp) of sequence i / nbat;
  // thread (row0, col4) moves U rows, 16 bytes each. The first batch is requested now,
  // so its loads are in flight while the features are computed.
  const int tpr = dv / 4;                 // threads per row (power of two, <= 64)
  const int rpp = kDecodeThreads / tpr;   // rows per pass
  const int col4 = tid % tpr, row0 = tid / tpr;
  const int rows_per_batch = U * rpp;
  const int nbat = (m + rows_per_batch - 1) / rows_per_batch;
  const int total = ng * nbat;
  auto load_batch = [&](int i, f32x4 (&buf)[U]) {
    const int sq = i / nbat, b = i % nbat;
    const float* Sp = S + ((size_t)(s0 + sq) * H + h) * m * dv;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = b * rows_per_batch + u * rpp + row0;
      if (r < m) buf[u] = *reinterpret_cast<const f32x4*>(Sp + (size_t)r * dv + col4 * 4);
    }
  };
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
  // this thread's first Omega row, then the first state batch: every load the features
  // wait for is older than the state loads, so those stay in flight meanwhile
  f32x4 w0[D / 4];
  if (tid < m) {
    const f32x4* wr = reinterpret_cast<const f32x4*>(omega + ((size_t)h * m + tid) * D);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) w0[i] = wr[i];
  }
  f32x4 bufA[U], bufB[U];
  if (total > 0) load_batch(0, bufA);
  __syncthreads();

  // phase 1: projections a = omega' . x
  for (int r = tid; r < m; r += kDecodeThreads) {
    float w[D];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      const f32x4 t = (r == tid) ? w0[i] : reinterpret_cast<const f32x4*>(omega + ((size_t)h * m + r) * D)[i];
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

  // z rows and the denominators (small: m floats per sequence)
  for (int sq = 0; sq < ng; ++sq) {
    const size_t pair = (size_t)(s0 + sq) * H + h;
    float* zp = z + pair * m;
    float dpart = 0.f;
    for (int r = tid; r < m; r += kDecodeThreads) {
      const float zn = zp[r] + ak[sq * m + r];
      zp[r] = zn;
      dpart += aq[sq * m + r] * zn;
    }
    dpart = wave_sum(dpart);
    if (lane == 0) dsum[sq][wv] = dpart;
  }

  // phase 2: stream the state, two batches in flight
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto process = [&](int i, const f32x4 (&buf)[U]) {
    const int sq = i / nbat, b = i % nbat;
    const size_t pair = (size_t)(s0 + sq) * H + h;
    float* Sp = S + pair * m * dv;
    const float* pq = aq + sq * m;
    const float* pk = ak + sq * m;
    f32x4 vv;
    const T* vs = v + pair * dv + col4 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = to_f(vs[j]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = b * rows_per_batch + u * rpp + row0;
      if (r < m) {
        const f32x4 st = buf[u] + pk[r] * vv;
        acc += pq[r] * st;
        *reinterpret_cast<f32x4*>(Sp + (size_t)r * dv + col4 * 4) = st;
      }
    }
    if (b == nbat - 1) {  // the sequence is complete: park its numerator partial
      *reinterpret_cast<f32x4*>(red + ((size_t)sq * kDecodeThreads + tid) * 4) = acc;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  int i = 0;
  for (; i + 1 < total; i += 2) {
    load_batch(i + 1, bufB);
    process(i, bufA);
    if (i + 2 < total) load_batch(i + 2, bufA);
    process(i + 1, bufB);
  }
  if (i < total) process(i, bufA);
  __syncthreads();
  for (int o = tid; o < ng * dv; o += kDecodeThreads) {
    const int sq = o / dv, col = o % dv;
    const int cc = col / 4, ii = col % 4;
    float num = 0.f;
    for (int rg = 0; rg < rpp; ++rg) num += red[((size_t)sq * kDecodeThreads + rg * tpr + cc) * 4 + ii];
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeThreads / 64; ++w) den += dsum[sq][w];
    out[((size_t)(s0 + sq) * H + h) * dv + col] = num / den;
  }
}

template <typename T, int D>
static hipError_t run_decode(const T* q, const T* k, const T* v, const float* omega, float* S, float* z, int N, int H,
                             int dv, int m, int kind, float eps, float* out, hipStream_t st) {
  const int G = kDecodeGroup;
  const int n_groups = (N + G - 1) / G;
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = (kind == 0) ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float log2_sqrt_m = 0.5f * std::log2((float)m);
  const float inv_sqrt_m = 1.0f / std::sqrt((float)m);
  const size_t lds = (size_t)(2 * G * m + 2 * G * D + G * kDecodeThreads * 4 + G * 4) * sizeof(float);
  {
    FAVOR_TIMED("decode", st);
    decode_kernel<T, D><<<(unsigned)(H * n_groups), kDecodeThreads, lds, st>>>(
        q, k, v, omega, S, z, N, H, dv, m, n_groups, kind, eps, inv_sqrt_m, wscale, nscale, log2_sqrt_m, out);
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
