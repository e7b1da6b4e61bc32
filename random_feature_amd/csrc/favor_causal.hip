// Causal (unidirectional) FAVOR+ on gfx950 as a segmented, chunked prefix scan.
//
// Performer paper, appendix B.1 (equation 11, Figure 8): row i of the output is
// G^PS_i Q'_i with G^PS_i = sum_{j <= i} K'_j [v_j 1]^T, i.e. prefix sums of S and z
// including the diagonal. Appendix B.3 notes that storing G^PS costs O(mLd) and that
// a sequential aggregation avoids it; the prefix sum itself is parallel (O(log L) depth).
// This file keeps both properties: L is cut into P segments that run in parallel, the
// segments are joined by a scan over their totals, and inside a segment the state is
// carried sequentially from one 32-token chunk to the next, never materialising G^PS.
//   1. omega_frag_kernel + reduce_kernel (shared with the bidirectional path):
//      per-segment totals of S_aug = Phi_K^T [V 1] with the segment's key maxima.
//   2. scan_kernel: prefix maxima M*_p over segments and the exclusive prefix sums
//      carry_p = sum_{q<p} total_q * 2^(M_q - M*_p); optionally the final state in
//      canonical (unstabilised) scale.
//   3. sweep_kernel, one workgroup per (segment, b*h), wave w owning FB*16 features:
//      per chunk of 32 tokens
//        * Q and K projections transposed (lane = token): Phi_Q with the row max
//          taken across all waves, Phi_K = 2^(a' - n' - M*_p);
//        * A^T = Phi_K Phi_Q^T over the wave's features (the intra-chunk scores) and
//          the inter-chunk term out^T = S_carry^T Phi_Q^T over the wave's features;
//          the partial tiles of all waves are summed through LDS;
//        * the intra-chunk term out^T += [V 1]^T tril(A)^T (keys <= queries);
//        * the wave's carried rows: S_carry += Phi_K^T [V 1], where Phi_K^T in the
//          row = feature layout comes from an exact MFMA product with an identity;
//        * division by the z row and a coalesced store of the chunk.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_timing.hpp"
#include "favor_reduce.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

// ---------------------------------------------------------------- scan over segments
// Grid (element chunks of 256, b*h): every thread scans one element of S_aug over the
// segments; the prefix maxima (a few values per segment) are recomputed per workgroup.
template <int DV, int M, int NW>
__global__ void __launch_bounds__(256)
scan_kernel(const float* __restrict__ part, const float* __restrict__ pmax, int nseg, int kind, float log2_sqrt_m,
            float* __restrict__ carry, float* __restrict__ cmax, float* __restrict__ S_final,
            float* __restrict__ z_final) {
  constexpr int FPW = M / NW;
  constexpr int W = DV + 1;
  extern __shared__ float pre[];  // [nseg] prefix maxima
  const int bh = blockIdx.y;
  if (threadIdx.x == 0) {
    float run = -INFINITY;
    for (int p = 0; p < nseg; ++p) {
      float mx = -INFINITY;
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, pmax[((size_t)bh * nseg + p) * NW + w]);
      run = fmaxf(run, mx);
      pre[p] = (kind == kPrf) ? run : 0.f;
      if (blockIdx.x == 0) cmax[(size_t)bh * nseg + p] = pre[p];
    }
  }
  __syncthreads();
  const size_t base = (size_t)bh * nseg * M * W;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= M * W) return;
  const int wv = (e / W) / FPW;
  float acc = 0.f, prev = 0.f;
  for (int p = 0; p < nseg; ++p) {
    const float mp = pre[p];
    if (p > 0) acc *= fast_exp2(prev - mp);
    carry[base + (size_t)p * M * W + e] = acc;
    const float sc = (kind == kPrf) ? fast_exp2(pmax[((size_t)bh * nseg + p) * NW + wv] - mp) : 1.f;
    acc += part[base + (size_t)p * M * W + e] * sc;
    prev = mp;
  }
  if (S_final) {
    const float canon = (kind == kPrf) ? acc * fast_exp2(prev - log2_sqrt_m) : acc;
    const int r = e / W, n = e % W;
    if (n < DV)
      S_final[((size_t)bh * M + r) * DV + n] = canon;
    else
      z_final[(size_t)bh * M + r] = canon;
  }
}

// ---------------------------------------------------------------- chunk sweep
template <typename T, int D, int DV, int M, int FB>
__global__ void __launch_bounds__(64 * (M / (16 * FB)))
sweep_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ omf,
             const float* __restrict__ carry, const float* __restrict__ cmax, int H, int L, int seg_len, int nseg,
             int kind, float eps, float inv_sqrt_m, float nscale, int out_f32, void* __restrict__ out) {
  constexpr int NW = M / (16 * FB);
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (FB + 1) / 2;
  constexpr int KROW = D + 8, VROW = 40;
  constexpr int NT = 4 + 2 * NB;
  constexpr int OROW = DV + 4;
  constexpr int W = DV + 1;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* qs = reinterpret_cast<T*>(smem);
  T* ks = qs + 32 * KROW;
  T* vts = ks + 32 * KROW;
  constexpr size_t TILE_BYTES = ((2 * 32 * KROW + DV * VROW) * sizeof(T) + 15) & ~(size_t)15;
  float* qmx = reinterpret_cast<float*>(smem + TILE_BYTES);
  float* xch = qmx + NW * 32;
  float* outs = xch + NW * NT * 256;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int seg = blockIdx.x, bh = blockIdx.y, h = bh % H;
  const int tbeg = seg * seg_len, tend = min(L, tbeg + seg_len);
  const size_t rowbase = (size_t)bh * L;
  const T* Qb = Q + rowbase * D;
  const T* Kb = K + rowbase * D;
  const T* Vb = V + rowbase * DV;

  vec8<T> om[FB][DC];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      om[fb][dc] = ld8<T>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);

  // carried state for this wave's rows, C layout: sacc[fb][nb][i] = S_aug[row 4g+i of block][col nb*16+c]
  f32x4 sacc[FB][NB];
  {
    const float* cp = carry + ((size_t)bh * nseg + seg) * M * W;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (w * FB + fb) * 16 + 4 * g + i;
#pragma unroll
        for (int nb = 0; nb < NB - 1; ++nb) sacc[fb][nb][i] = cp[(size_t)r * W + nb * 16 + c];
        sacc[fb][NB - 1][i] = (c == 0) ? cp[(size_t)r * W + DV] : 0.f;
      }
  }
  const float mstar = cmax[(size_t)bh * nseg + seg];

  vec8<T> ones, idb[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ones[j] = to_t<T>(c == 0 ? 1.f : 0.f);
    const int kslot = 16 * (j >> 2) + 4 * g + (j & 3);
    idb[0][j] = to_t<T>(kslot == c ? 1.f : 0.f);
    idb[1][j] = to_t<T>(kslot == 16 + c ? 1.f : 0.f);
  }

  for (int t0 = tbeg; t0 < tend; t0 += 32) {
    // ---- stage Q, K (row major) and V (transposed, token pairs) in LDS
    constexpr int XCH8 = 32 * D / 8;
    for (int q = threadIdx.x; q < 2 * XCH8; q += NW * 64) {
      const int which = q / XCH8, qq = q % XCH8;
      const int row = qq / (D / 8), col = (qq % (D / 8)) * 8;
      const T* src = which == 0 ? Qb : Kb;
      const vec8<T> x = (t0 + row < tend) ? ld8<T>(src + (size_t)(t0 + row) * D + col) : zero8<T>();
      st8<T>((which == 0 ? qs : ks) + row * KROW + col, x);
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

    // ---- projections (transposed: A = Omega' rows, B = X^T) -> [feature 4g+i][token c]
    f32x4 pq[2][FB], pk[2][FB];
    float knorm[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<T> qf[DC], kf[DC];
      float s2 = 0.f;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        qf[dc] = (col < D) ? ld8<T>(qs + (tb * 16 + c) * KROW + col) : zero8<T>();
        kf[dc] = (col < D) ? ld8<T>(ks + (tb * 16 + c) * KROW + col) : zero8<T>();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = to_f(kf[dc][j]);
          s2 += x * x;
        }
      }
      knorm[tb] = group_sum(s2) * nscale;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pq[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
        pk[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          mma16(pq[tb][fb], om[fb][dc], qf[dc]);
          mma16(pk[tb][fb], om[fb][dc], kf[dc]);
        }
      }
    }
    // ---- feature maps
    if (kind == kPrf) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = -INFINITY;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pq[tb][fb][i]);
        mx = group_max(mx);
        if (g == 0) qmx[w * 32 + tb * 16 + c] = mx;
        const bool ok = t0 + tb * 16 + c < tend;
        const float sub = knorm[tb] + mstar;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[tb][fb][i] = ok ? fast_exp2(pk[tb][fb][i] - sub) : 0.f;
      }
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bool ok = t0 + tb * 16 + c < tend;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pk[tb][fb][i] = ok ? fmaxf(pk[tb][fb][i], 0.f) * inv_sqrt_m + eps : 0.f;
            pq[tb][fb][i] = fmaxf(pq[tb][fb][i], 0.f) * inv_sqrt_m + eps;
          }
      }
    }
    __syncthreads();
    if (kind == kPrf) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) mx = fmaxf(mx, qmx[ww * 32 + tb * 16 + c]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pq[tb][fb][i] = fast_exp2(pq[tb][fb][i] - mx);
      }
    }
    // operand fragments with paired feature slots: lane = token c
    vec8<T> fq[2][NFC], fk[2][NFC];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int fb = 2 * fc + (j >> 2);
          const int fbs = fb < FB ? fb : 0;
          fq[tb][fc][j] = to_t<T>(fb < FB ? pq[tb][fbs][j & 3] : 0.f);
          fk[tb][fc][j] = to_t<T>(fb < FB ? pk[tb][fbs][j & 3] : 0.f);
        }

    // ---- partial tiles over this wave's features -> LDS
    float* xw = xch + (size_t)w * NT * 256;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc) mma16(a, fk[kt][fc], fq[qt][fc]);
        *reinterpret_cast<f32x4*>(xw + (kt * 2 + qt) * 256 + lane * 4) = a;
      }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      vec8<T> sf[NFC];
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int fb = 2 * fc + (j >> 2);
          sf[fc][j] = to_t<T>(fb < FB ? sacc[fb < FB ? fb : 0][nb][j & 3] : 0.f);
        }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc) mma16(o, sf[fc], fq[qt][fc]);
        *reinterpret_cast<f32x4*>(xw + (4 + qt * NB + nb) * 256 + lane * 4) = o;
      }
    }

    // ---- value fragments (paired token slots), shared by the update and the intra term
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

    // ---- carried rows: S_carry += Phi_K^T [V 1]; Phi_K^T (row = feature) via identity products
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      f32x4 tr[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        tr[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma16(tr[tb], fk[tb][fb >> 1], idb[fb & 1]);
      }
      vec8<T> afk;
#pragma unroll
      for (int j = 0; j < 8; ++j) afk[j] = to_t<T>(tr[j >> 2][j & 3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma16(sacc[fb][nb], afk, vf[nb]);
    }
    __syncthreads();

    // ---- sum the intra scores over waves, mask keys > query: B fragments (k = key, n = query)
    vec8<T> atf[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) a += *reinterpret_cast<const f32x4*>(xch + ((size_t)ww * NT + kt * 2 + qt) * 256 + lane * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt * 16 + 4 * g + i, qry = qt * 16 + c;
          atf[qt][kt * 4 + i] = to_t<T>(key <= qry ? a[i] : 0.f);
        }
      }
    }
    // ---- output tiles owned by this wave: sum of inter partials + intra product
    for (int t = w; t < 2 * NB; t += NW) {
      const int qt = t / NB, nb = t % NB;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) o += *reinterpret_cast<const f32x4*>(xch + ((size_t)ww * NT + 4 + qt * NB + nb) * 256 + lane * 4);
      mma16(o, vf[nb], atf[qt]);
      // o[i] = out^T[col nb*16 + 4g + i][query qt*16 + c]
      if (nb < NB - 1) {
        *reinterpret_cast<f32x4*>(outs + (qt * 16 + c) * OROW + nb * 16 + 4 * g) = o;
      } else if (g == 0) {
        outs[(qt * 16 + c) * OROW + DV] = o[0];
      }
    }
    __syncthreads();

    // ---- normalise and store the chunk (coalesced rows)
    constexpr int C4 = DV / 4;
    for (int e = threadIdx.x; e < 32 * C4; e += NW * 64) {
      const int qrow = e / C4, c4 = e % C4;
      const int tok = t0 + qrow;
      if (tok < tend) {
        const float rden = 1.0f / outs[qrow * OROW + DV];
        const f32x4 o = *reinterpret_cast<const f32x4*>(outs + qrow * OROW + c4 * 4);
        const size_t off = (rowbase + tok) * DV + c4 * 4;
        if (out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = o * rden;
        } else {
          vec4<T> r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = to_t<T>(o[i] * rden);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(out) + off) = r;
        }
      }
    }
  }
}

template <typename T, int D, int DV, int M>
static hipError_t run_causal(const T* q, const T* k, const T* v, const float* omega, const Shape& s, int kind,
                             float eps, int out_f32, void* out, float* S_final, float* z_final, void* ws,
                             hipStream_t st) {
  constexpr int FB = (M / 16) < 4 ? (M / 16) : 4;
  constexpr int NW = M / (16 * FB);
  constexpr int DC = (D + 31) / 32, NB = DV / 16 + 1;
  const CausalPlan p = plan_causal(s, sizeof(T) == 4 ? 0 : 1);
  char* base = static_cast<char*>(ws);
  T* omf = reinterpret_cast<T*>(base + p.off_omf);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* pmax = reinterpret_cast<float*>(base + p.off_pmax);
  float* carry = reinterpret_cast<float*>(base + p.off_carry);
  float* cmax = reinterpret_cast<float*>(base + p.off_cmax);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = (kind == kPrf) ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)M);
  const float log2_sqrt_m = 0.5f * std::log2((float)M);

  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  {
    FAVOR_TIMED("omega_frag", st);
    omega_frag_kernel<T><<<(unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st>>>(
        omega, s.H, M, D, wscale, omf);
  }
  {
    FAVOR_TIMED("reduce", st);
    reduce_kernel<T, D, DV, M, FB><<<dim3(p.nseg, (unsigned)s.bh()), 64 * NW, 0, st>>>(
        k, v, omf, s.H, s.L, p.seg_len, p.nseg, kind, eps, inv_sqrt_m, nscale, part, pmax);
  }
  {
    FAVOR_TIMED("scan", st);
    scan_kernel<DV, M, NW><<<dim3((unsigned)((M * (DV + 1) + 255) / 256), (unsigned)s.bh()), 256,
                             p.nseg * sizeof(float), st>>>(
        part, pmax, p.nseg, kind, log2_sqrt_m, carry, cmax, S_final, z_final);
  }
  constexpr int KROW = D + 8, VROW = 40, NT = 4 + 2 * NB, OROW = DV + 4;
  const size_t lds = (((2 * 32 * KROW + DV * VROW) * sizeof(T) + 15) & ~(size_t)15) +
                     (size_t)(NW * 32 + NW * NT * 256 + 32 * OROW) * sizeof(float);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sweep_kernel<T, D, DV, M, FB>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  {
    FAVOR_TIMED("sweep", st);
    sweep_kernel<T, D, DV, M, FB><<<dim3(p.nseg, (unsigned)s.bh()), 64 * NW, lds, st>>>(
        q, k, v, omf, carry, cmax, s.H, s.L, p.seg_len, p.nseg, kind, eps, inv_sqrt_m, nscale, out_f32, out);
  }
  return hipGetLastError();
}

hipError_t launch_causal(const void* q, const void* k, const void* v, const float* omega, const Shape& s,
                         int dtype, int kind, float eps, int out_f32, void* out, float* S_final, float* z_final,
                         void* ws, hipStream_t st) {
#define X(D_, DV_, M_)                                                                                          \
  if (s.d == D_ && s.dv == DV_ && s.m == M_) {                                                                  \
    if (dtype == 0)                                                                                             \
      return run_causal<float, D_, DV_, M_>(static_cast<const float*>(q), static_cast<const float*>(k),        \
                                            static_cast<const float*>(v), omega, s, kind, eps, out_f32, out,    \
                                            S_final, z_final, ws, st);                                          \
    return run_causal<bf16, D_, DV_, M_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),             \
                                         static_cast<const bf16*>(v), omega, s, kind, eps, out_f32, out,        \
                                         S_final, z_final, ws, st);                                             \
  }
  FAVOR_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace favor
