// One recurrent decode step of causal FAVOR+ for N sequences x H heads.
//
// The causal sums advanced by one token (linear-attention blog, "Autoregressive
// Generation"; RFA summary page, appendix A.3):
//   S <- S + phi(k) v^T,  z <- z + phi(k),  out = phi(q).S / phi(q).z
// with the updated state (token t's output includes token t).
//
// The state S [N,H,m,dv] fp32 dominates the traffic: each step reads and writes it
// once, so the kernel is an HBM stream. Work split: one workgroup per (sequence, head).
//   every thread first requests the loads the features need (q, k, its v columns, the
//   Omega row of its feature), then its state rows (16-byte loads, consecutive threads
//   on consecutive columns of a row), so the state streams in during the projections;
//   thread r computes a = omega_r . x for q and k (fp32 FMA). Keys use the canonical
//   feature exp(a - |x|^2/2)/sqrt(m) because the state is kept unstabilised; queries
//   use exp(a - max_r a), a per-row constant that cancels in the ratio.
//   Each thread then updates its rows in place, accumulates its share of the numerator
//   and the workgroup reduces the shares through LDS.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

#ifndef FAVOR_DECODE_THREADS
#define FAVOR_DECODE_THREADS 256
#endif
#ifndef FAVOR_DECODE_ROWS
#define FAVOR_DECODE_ROWS 16
#endif
constexpr int kDecodeThreads = FAVOR_DECODE_THREADS;
#ifndef FAVOR_DECODE_NT
#define FAVOR_DECODE_NT 1
#endif
constexpr int kDecodeRows = FAVOR_DECODE_ROWS;  // state rows (16 bytes each) a thread moves per sequence and batch
// the state is streamed once per step: bit 0 marks its loads, bit 1 its stores non-temporal
__device__ __forceinline__ f32x4 ld_state(const float* p) {
  if constexpr (FAVOR_DECODE_NT & 1) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  else return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ void st_state(float* p, const f32x4& x) {
  if constexpr (FAVOR_DECODE_NT & 2) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
  else *reinterpret_cast<f32x4*>(p) = x;
}
#ifndef FAVOR_DECODE_AHEAD
#define FAVOR_DECODE_AHEAD 128
#endif
constexpr int kDecodeAhead = FAVOR_DECODE_AHEAD;  // input prefetch distance, in workgroups of one XCD
#ifndef FAVOR_DECODE_PREFETCH
#define FAVOR_DECODE_PREFETCH 4
#endif
constexpr int kDecodePrefetch = FAVOR_DECODE_PREFETCH;  // later workgroups whose inputs each one requests
static_assert(kDecodePrefetch <= kDecodeThreads / 64, "one wave per prefetched workgroup");
constexpr int kDecodeSeqs = 1;                  // sequences of one head per workgroup (they share Omega's rows)

// One workgroup per (head, group of kDecodeSeqs sequences); every thread owns 4 columns of
// runs of kDecodeRows consecutive state rows of each sequence. The first batch of state
// rows is requested right after the (older) loads the features need, so the state streams
// in while the projections are computed. Two threads share each feature's projection (one
// half of d each). Measured on the 256-sequence, 16-head, m = 256, dv = 64 step: 256
// threads with 16 rows each (the whole state in one batch) beat 8 or 4 rows and 512
// threads.
// Gated form (RFA page, section 3.2): with `gate` non-null the old state decays by the
// pair's scalar gate[pair] and the new token enters with weight inw[pair] (1 if inw is
// null): S = g S + w phi(k) v^T, z = g z + w phi(k); with gate null g = w = 1.
template <typename T, int D>
__global__ void __launch_bounds__(kDecodeThreads)
decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
              const float* __restrict__ omega, float* __restrict__ S, float* __restrict__ z, int N, int H,
              int dv, int m, int kind, float eps, float inv_sqrt_m, float wscale, float nscale, float log2_sqrt_m,
              const float* __restrict__ gate, const float* __restrict__ inw, float* __restrict__ out, int ahead,
              int sink) {
  constexpr int U = kDecodeRows, G = kDecodeSeqs;
  constexpr int NWV = kDecodeThreads / 64;
  constexpr int DH = D / 2;  // the d-half of a feature this thread projects
  extern __shared__ __attribute__((aligned(16))) float sm[];
  // layout: fq[G][m], fk[G][m] (features), xs[G][2][D] (q, k as fp32), red[G][threads][4]
  float* fq = sm;
  float* fk = fq + G * m;
  float* xs = fk + G * m;
  float* red = xs + G * 2 * D;
  __shared__ float wred[G][2][NWV];

  const int n_grp = (N + G - 1) / G;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int h = logical / n_grp, s0 = (logical % n_grp) * G;
  const int ng = min(G, N - s0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int tpr = dv / 4;                 // threads per row (4..64)
  const int rgs = kDecodeThreads / tpr;   // row groups of U consecutive rows per batch
  const int col4 = tid % tpr, rg0 = tid / tpr;
  // when tpr does not divide the threads, the last few (rg0 == rgs) own no rows: they load clamped rows
  // like the others but never store or contribute
  const bool owns_rows = rg0 < rgs;
  const int rows_per_batch = U * rgs;
  const int nbat = (m + rows_per_batch - 1) / rows_per_batch;
  // this thread's rows in batch b: b*rows_per_batch + rg0*U + u, u < U (consecutive rows,
  // so one base address and immediate offsets); a wave covers whole rows
  // the pair (sequence, head) of slot g; a missing sequence of the last group reuses
  // the first one's data for its loads and writes nothing
  auto pair_of = [&](int g) -> size_t { return (size_t)(s0 + (g < ng ? g : 0)) * H + h; };

  // the q, k and v rows of the workgroups that this XCD starts ahead, 2*ahead, ...,
  // kDecodePrefetch*ahead workgroups later are requested now (16 bytes per lane), so that
  // they are cache-resident when those start instead of queued behind the state stream in
  // HBM; the values are kept only under the flag `sink`, which the host passes as 0
  f32x4 pf = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const int per = gridDim.x >> 3;  // xcd_remap: workgroups of one XCD take consecutive logical ids
    constexpr int RB = D * (int)sizeof(T);
    const int rbv = dv * (int)sizeof(T);
    const int jpf = wv + 1;  // wave w requests the workgroup (w + 1) * ahead later
    if (ahead > 0 && (gridDim.x & 7) == 0 && jpf <= kDecodePrefetch && logical % per + ahead * jpf < per) {
      const int l2 = logical + ahead * jpf;
      const size_t pair2 = (size_t)((l2 % n_grp) * G) * H + l2 / n_grp;
      const int which = lane >> 4, off = (lane & 15) * 16;  // lanes 0-15 q, 16-31 k, 32-47 v, then the gates
      if (which < 3) {
        const char* base = which == 0   ? reinterpret_cast<const char*>(q + pair2 * D)
                           : which == 1 ? reinterpret_cast<const char*>(k + pair2 * D)
                                        : reinterpret_cast<const char*>(v + pair2 * dv);
        if (off < (which < 2 ? RB : rbv)) pf = *reinterpret_cast<const f32x4*>(base + off);
      } else if (lane == 48 && gate) {
        pf[0] = gate[pair2];
      } else if (lane == 49 && gate && inw) {
        pf[0] = inw[pair2];
      }
    }
  }
  // loads the features wait for: q, k (raw, into registers: their copy to LDS waits until
  // every load below is in flight), this thread's v columns, its Omega half-row
  constexpr int XPT = (G * 2 * D + kDecodeThreads - 1) / kDecodeThreads;
  T xraw[XPT];
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = tid + u * kDecodeThreads;
    const int ii = i < G * 2 * D ? i : 0;
    const int g = ii / (2 * D), w2 = (ii / D) & 1, dd = ii % D;
    xraw[u] = (w2 == 0 ? q : k)[pair_of(g) * D + dd];
  }
  f32x4 vv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const T* vs = v + pair_of(g) * dv + col4 * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[g][j] = to_f(vs[j]);
  }
  float gv[G], iw[G];  // decay of the old state and weight of the new token
#pragma unroll
  for (int g = 0; g < G; ++g) {
    gv[g] = gate ? gate[pair_of(g)] : 1.f;
    iw[g] = gate && inw ? inw[pair_of(g)] : 1.f;
  }
  const int half = tid & 1, f0 = tid >> 1;
  // (loads are unconditional, from clamped rows, so they issue back to back with no
  // waits in between; results for rows past m are never used)
  f32x4 w0[DH / 4];
  {
    const f32x4* wr =
        reinterpret_cast<const f32x4*>(omega + ((size_t)h * m + (f0 < m ? f0 : m - 1)) * D + half * DH);
#pragma unroll
    for (int i = 0; i < DH / 4; ++i) w0[i] = wr[i];
  }
  // then the first state batch of every sequence; a row past m is read as row m-1 and its
  // value never used
  auto row_ptr = [&](int g, int r) -> float* {
    return S + pair_of(g) * m * dv + (size_t)(r < m ? r : m - 1) * dv + col4 * 4;
  };
  f32x4 buf[G][U];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int r0 = rg0 * U;
    if (r0 + U <= m) {
      const float* p0 = row_ptr(g, r0);
#pragma unroll
      for (int u = 0; u < U; ++u) buf[g][u] = ld_state(p0 + u * dv);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) buf[g][u] = ld_state(row_ptr(g, r0 + u));
    }
  }
#pragma unroll
  for (int u = 0; u < XPT; ++u) {
    const int i = tid + u * kDecodeThreads;
    if (i < G * 2 * D) xs[i] = to_f(xraw[u]);
  }
  __syncthreads();

  // projections a = omega' . x of q and k, stored raw; the key norms meanwhile
  if (wv < G) {
    float k2 = 0.f;
    for (int dd = lane; dd < D; dd += 64) k2 += xs[(wv * 2 + 1) * D + dd] * xs[(wv * 2 + 1) * D + dd];
    k2 = wave_sum(k2);
    // log2 of the key's normaliser exp(|k'|^2/2) sqrt(m) (exponential map: divides), or of its scale
    // exp(|k'|^2/2) / sqrt(m/2) (trigonometric map, log2_sqrt_m then taken of m/2: multiplies)
    if (lane == 0) wred[wv][1][0] = kind == kTrig ? k2 * nscale - log2_sqrt_m : k2 * nscale + log2_sqrt_m;
  }
  // feature r's projection from this thread's half of omega_r (w), completed across the
  // lane pair by DPP; every thread runs the same iterations
  auto feature = [&](int r, const f32x4 (&w)[DH / 4]) {
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
      const f32x4* xq = reinterpret_cast<const f32x4*>(xs + (g * 2) * D + half * DH);
      const f32x4* xk = reinterpret_cast<const f32x4*>(xs + (g * 2 + 1) * D + half * DH);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < DH / 4; ++i) {
        const f32x4 tq = xq[i], tk = xk[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a0 += w[i][j] * tq[j];
          a1 += w[i][j] * tk[j];
        }
      }
      a0 = (a0 + dpp<kDppXor1>(a0)) * wscale;
      a1 = (a1 + dpp<kDppXor1>(a1)) * wscale;
      if (r < m && half == 0) {
        fq[g * m + r] = a0;
        fk[g * m + r] = a1;
      }
    }
  };
  feature(f0, w0);
  for (int r = f0 + kDecodeThreads / 2; r - f0 < m; r += kDecodeThreads / 2) {  // m > 256 only
    f32x4 w[DH / 4];
    const int rr = r < m ? r : m - 1;
#pragma unroll
    for (int i = 0; i < DH / 4; ++i)
      w[i] = reinterpret_cast<const f32x4*>(omega + ((size_t)h * m + rr) * D + half * DH)[i];
    feature(r, w);
  }
  __syncthreads();
  // feature maps: keys the canonical exp(a - |k|^2/2)/sqrt(m) (the state is kept
  // unstabilised), queries exp(a - max_r a), a per-row constant that cancels in the ratio
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    if (kind == 0) {
      float mx = -INFINITY;
      for (int r = tid; r < m; r += kDecodeThreads) mx = fmaxf(mx, fq[g * m + r]);
      mx = wave_max(mx);
      if (lane == 0) wred[g][0][wv] = mx;
    }
  }
  __syncthreads();
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    float mx = 0.f;
    if (kind == 0) {
      mx = wred[g][0][0];
#pragma unroll
      for (int i = 1; i < NWV; ++i) mx = fmaxf(mx, wred[g][0][i]);
    }
    const float kbg = wred[g][1][0];
    for (int r = tid; r < m; r += kDecodeThreads) {
      if (kind == 0) {
        fq[g * m + r] = fast_exp2(fq[g * m + r] - mx);
        fk[g * m + r] = fast_exp2(fk[g * m + r] - kbg);
      } else if (kind == kTrig) {
        // the m/2 sines, then the m/2 cosines; the query's scale cancels in the ratio
        fq[g * m + r] = trig_feature(fq[g * m + r], r, m);
        fk[g * m + r] = trig_feature(fk[g * m + r], r, m) * fast_exp2(kbg);
      } else {
        fq[g * m + r] = fmaxf(fq[g * m + r], 0.f) * inv_sqrt_m + eps;
        fk[g * m + r] = fmaxf(fk[g * m + r], 0.f) * inv_sqrt_m + eps;
      }
    }
  }
  __syncthreads();

  // z and the denominators
  float dpart[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    dpart[g] = 0.f;
    float* zp = z + pair_of(g) * m;
    for (int r = tid; r < m; r += kDecodeThreads) {
      const float zn = zp[r] * gv[g] + fk[g * m + r] * iw[g];
      if (g < ng) zp[r] = zn;
      dpart[g] += fq[g * m + r] * zn;
    }
  }
  // the state: S += phi(k) v^T, numerator += phi(q) . S
  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < nbat; ++b) {
    const int r0 = b * rows_per_batch + rg0 * U;
    if (b > 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < U; ++u) buf[g][u] = ld_state(row_ptr(g, r0 + u));
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* const p0 = row_ptr(g, r0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u;
        if (r < m && owns_rows) {
          const f32x4 st = buf[g][u] * gv[g] + (fk[g * m + r] * iw[g]) * vv[g];
          acc[g] += fq[g * m + r] * st;
          if (g < ng) st_state(p0 + u * dv, st);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    *reinterpret_cast<f32x4*>(red + ((size_t)g * kDecodeThreads + tid) * 4) = acc[g];
    const float dp = wave_sum(dpart[g]);
    if (lane == 0) wred[g][1][wv] = dp;
  }
  __syncthreads();
  for (int o = tid; o < ng * dv; o += kDecodeThreads) {
    const int g = o / dv, col = o % dv;
    const int cc = col / 4, ii = col % 4;
    float num = 0.f;
    for (int rg = 0; rg < rgs; ++rg) num += red[((size_t)g * kDecodeThreads + rg * tpr + cc) * 4 + ii];
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) den += wred[g][1][i];
    out[pair_of(g) * dv + col] = num / den;
  }
  if (sink) out[tid] = pf[0] + pf[1] + pf[2] + pf[3];
}

// ---------------------------------------------------------------- host side
template <typename T, int D>
static hipError_t run_decode(const T* q, const T* k, const T* v, const float* omega, float* S, float* z, int N, int H,
                             int dv, int m, int kind, float eps, const float* gate, const float* inw, float* out,
                             hipStream_t st) {
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = omega_scale(kind, sc);
  const float nscale = sc * sc * kLog2e * 0.5f;
  // the features' normaliser: sqrt(m), or sqrt(m/2) for the trigonometric map (m/2 vectors, two features each)
  const float log2_sqrt_m = 0.5f * std::log2((float)(kind == kTrig ? m / 2 : m));
  const float inv_sqrt_m = 1.0f / std::sqrt((float)m);
  const size_t lds =
      (size_t)(2 * kDecodeSeqs * m + kDecodeSeqs * 2 * D + kDecodeSeqs * kDecodeThreads * 4) * sizeof(float);
  if (N == 0) return hipSuccess;
  const size_t n_grp = ((size_t)N + kDecodeSeqs - 1) / kDecodeSeqs;
  {
    launch("decode", decode_kernel<T, D>, (unsigned)(n_grp * H), kDecodeThreads, lds, st, q, k, v, omega, S, z, N, H,
        dv, m, kind, eps, inv_sqrt_m, wscale, nscale, log2_sqrt_m, gate, inw, out, kDecodeAhead, 0);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* omega, float* S, float* z,
                         int N, int H, int d, int dv, int m, int dtype, int kind, float eps, const float* gate,
                         const float* inw, float* out, hipStream_t st) {
#define DEC(D_)                                                                                                 \
  if (d == D_) {                                                                                                \
    if (dtype == 0)                                                                                             \
      return run_decode<float, D_>(static_cast<const float*>(q), static_cast<const float*>(k),                  \
                                   static_cast<const float*>(v), omega, S, z, N, H, dv, m, kind, eps, gate,     \
                                   inw, out, st);                                                               \
    return run_decode<bf16, D_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),                       \
                                static_cast<const bf16*>(v), omega, S, z, N, H, dv, m, kind, eps, gate, inw,    \
                                out, st);                                                                       \
  }
  DEC(16)
  DEC(32)
  DEC(64)
#undef DEC
  return hipErrorInvalidValue;
}

}  // namespace favor
