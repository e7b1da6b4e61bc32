// Gradients of causal FAVOR+ on gfx950.
//
// Performer paper, appendix B.1 (equation 11): out_i = N_i / D_i with the prefix sums
// S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j), N_i = phi(q_i) S_i, D_i = phi(q_i) z_i.
// With W_i = [g_i, -gamma_i] / D_i (gamma_i = g_i . out_i, g = dL/dout) the chain rule gives
//   dPhi_Q,i = [S_i z_i] W_i                       (a prefix state, as in the forward)
//   dPhi_K,j = R_j [v_j 1],  dv_j = R_j^T phi(k_j)  with the suffix sums R_j = sum_{i>=j} phi(q_i) W_i^T
// and through the positive feature map dx = d^-1/4 (Omega^T (phi * dphi) - xs (phi . dphi)), whose
// second term vanishes for the queries. The segments and chunks of the forward sweep carry over:
// L is cut into segments that run in parallel; inside a segment the state moves from one 32-token
// chunk to the next, forwards for the queries and backwards for the keys; the chunk's own
// interactions are masked products. Every stabiliser constant is the forward's: the keys of segment
// p are taken against its prefix key maximum M_p (so phi'_K = 2^(a' - n' - M_p) <= 2^-8) and a
// query's features against its own bias b_i, which cancels in phi_Q * dPhi_Q. Then
//   phi~_i = phi'_Q,i / D'_i = 2^(a'_i - l_i),  l_i = b_i + log2 D'_i   (D' = phi'_Q . z' in the
//                                                                        segment's scale)
//   R''_j = sum_{i>=j} phi~_i [g_i, -gamma_i]^T 2^(M_p - M_p(i))        (segment p of key j)
//   phi_K * dPhi_K = phi'_K,j * (R''_j [v_j 1]),   dv_j = R''_j^T phi'_K,j
// which are the true gradients: the 1/sqrt(m) factors and the scales of both sides cancel.
// KIND = kRelu (the ReLU map of appendix A.4, phi = max(a, 0)/sqrt(m) + eps) has no stabiliser: the
// keys' features are phi_K itself, l_i = log2 D_i, phi~_i = phi_Q,i 2^-l_i, and the derivative factors
// phi' of P become the masks 1[a > 0]/sqrt(m) (times 2^-l_i on the query side), with no norm term.
// Kernels, in launch order (after the forward's Omega fragments, segment reduction and scan):
//   omegaT_pair_kernel  Omega'^T as hi + lo fragments for the back-projections
//   cbwd_fwd_kernel     per segment, forwards: the forward output of every chunk (carried term and
//                       masked intra term); gamma and l per query to HBM
//   cbwd_q_kernel       per segment, forwards: dPhi_Q from the prefix state and the chunk's masked
//                       scores, dq
//   cbwd_t_kernel       per segment: T_p = sum over its queries of phi~_i [g_i, -gamma_i]^T
//   cbwd_rscan_kernel   suffix carries over segments: C_p = sum_{q>p} T_q 2^(M_p - M_q)
//   cbwd_k_kernel       per segment, backwards: dPhi_K from the suffix state and the chunk's masked
//                       scores, dk
//   cbwd_v_kernel       per segment, backwards: dv from the suffix state and the masked score matrix
// Each kernel holds one layout of its state in registers ([feature][column] where it contracts over
// features, [column][feature] where over columns): a kernel holding both would need more than the
// 256 registers of two waves per SIMD. Inputs enter the products exactly (bf16 values); the
// features, states and scores enter as hi + lo bf16 pairs (two or three MFMAs), since the sums
// over tokens and over features cancel.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_segments.hpp"
#include "favor_tiles.hpp"
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>
#include <type_traits>

namespace favor {

template <typename T> struct CbwdOps;  // hi + lo pairs for 16-bit contraction types
template <> struct CbwdOps<bf16> { static constexpr int NSPL = 2; };
template <> struct CbwdOps<float> { static constexpr int NSPL = 1; };

// x as a rounded part and its remainder, into slot j of two operands
template <typename V>
__device__ __forceinline__ void split2(float x, V& h, V& l, int j) {
  using C = std::remove_cv_t<std::remove_reference_t<decltype(h[0])>>;
  const C hv = to_t<C>(x);
  h[j] = hv;
  l[j] = to_t<C>(x - to_f(hv));
}

// acc += ah bh (+ ah bl + al bh for split operands)
template <int NSPL, typename V>
__device__ __forceinline__ void mma_split(f32x4& acc, const V& ah, const V& al, const V& bh, const V& bl) {
  mma16(acc, ah, bh);
  if constexpr (NSPL == 2) {
    mma16(acc, ah, bl);
    mma16(acc, al, bh);
  }
}

// Feature of a key from its projection accumulator: PRF 2^a (the bias -(n'_k + M) is already in a);
// ReLU max(a, 0)/sqrt(m) + eps (the accumulator starts at zero).
template <int KIND>
__device__ __forceinline__ float key_feature(float a, float inv_sqrt_m, float eps) {
  if constexpr (KIND == kPrf) return fast_exp2(a);
  return fmaxf(a, 0.f) * inv_sqrt_m + eps;
}

// phi~ of a query (its feature over its denominator) from its projection accumulator: PRF 2^a (the
// accumulator starts at -l); ReLU (max(a, 0)/sqrt(m) + eps) 2^-l (it starts at zero). l = +inf (queries
// outside the segment) gives 0 either way.
template <int KIND>
__device__ __forceinline__ float query_feature(float a, float l, float inv_sqrt_m, float eps) {
  if constexpr (KIND == kPrf) return fast_exp2(a);
  return (fmaxf(a, 0.f) * inv_sqrt_m + eps) * fast_exp2(-l);
}

// Accumulator start of a projection: the PRF bias, zero for ReLU.
template <int KIND>
__device__ __forceinline__ float proj_start(float prf_bias) {
  return KIND == kPrf ? prf_bias : 0.f;
}

// Operand of 8 paired slots from a [k][n] array in LDS (row stride `stride`): lane (c, g) gets
// base[(row0 + 16(j>>2) + 4g + (j&3)) * stride + col0 + c], j = 0..7 (the transposing read for
// 16-bit types).
template <typename C>
__device__ __forceinline__ vec8<C> tr_read8(const C* base, int stride, int row0, int col0, int c, int g) {
  vec8<C> r;
  if constexpr (sizeof(C) == 2) {
    const bf16x4 lo = lds_read_tr4(reinterpret_cast<const bf16*>(base + (row0 + 4 * g + (c >> 2)) * stride + col0 + 4 * (c & 3)));
    const bf16x4 hi =
        lds_read_tr4(reinterpret_cast<const bf16*>(base + (row0 + 16 + 4 * g + (c >> 2)) * stride + col0 + 4 * (c & 3)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = lo[i];
      r[i + 4] = hi[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = base[(row0 + 16 * (j >> 2) + 4 * g + (j & 3)) * stride + col0 + c];
  }
  return r;
}

// 8 paired slots of one row: row[k0 + 16(j>>2) + 4g + (j&3)]
template <typename X>
__device__ __forceinline__ vec8<X> pair_read8(const X* row, int k0, int g) {
  const vec4<X> a = *reinterpret_cast<const vec4<X>*>(row + k0 + 4 * g);
  const vec4<X> b = *reinterpret_cast<const vec4<X>*>(row + k0 + 16 + 4 * g);
  vec8<X> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = a[i];
    r[i + 4] = b[i];
  }
  return r;
}

template <typename C, typename T>
__device__ __forceinline__ vec8<C> cvt8(const vec8<T>& x) {
  vec8<C> r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = to_t<C>(to_f(x[j]));
  return r;
}

// A head's Omega'^T fragments (hi and lo, BYTES each) copied into LDS with asynchronous 16-byte
// copies, whole waves per round; the caller waits (vmcnt) and synchronises before the first read.
template <int NT, int BYTES, typename C>
__device__ __forceinline__ void stage_omT(const C* hi, const C* lo, C* dst_hi, C* dst_lo) {
  static_assert(BYTES % (16 * NT) == 0, "whole rounds of 16-byte copies");
  const int tid = threadIdx.x, w = tid >> 6;
#pragma unroll
  for (int u = 0; u < BYTES / (16 * NT); ++u) {
    const size_t off = (size_t)(u * NT + tid) * 16;
    const uint32_t dst = (uint32_t)(u * NT + w * 64) * 16u;
    lds_dma16(reinterpret_cast<const unsigned char*>(hi) + off, lds_addr(dst_hi) + dst);
    if (lo != nullptr) lds_dma16(reinterpret_cast<const unsigned char*>(lo) + off, lds_addr(dst_lo) + dst);
  }
}

// Omega'^T as the A operand of the back-projections with paired feature slots, split into a
// rounded part and its remainder: hi[h][db][fc][lane][j] = rnd(scale * omega[h][f][db*16 + c]),
// f = fc*32 + 16(j>>2) + 4g + (j&3) (0 past m or d), lo the rounding remainder (0 for fp32).
template <typename C>
__global__ void omegaT_pair_kernel(const float* __restrict__ omega, int H, int m, int d, float scale,
                                   C* __restrict__ hi, C* __restrict__ lo) {
  const int nfc = (m + 31) / 32, ndb = (d + 15) / 16;
  const long long total = (long long)H * ndb * nfc * 64;
  for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(id & 63);
    unsigned rest = (unsigned)(id >> 6);
    const int fc = (int)(rest % (unsigned)nfc);
    rest /= (unsigned)nfc;
    const int db = (int)(rest % (unsigned)ndb);
    const int h = (int)(rest / (unsigned)ndb);
    const int c = lane & 15, g = lane >> 4;
    const int dd = db * 16 + c;
    vec8<C> xh, xl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = fc * 32 + 16 * (j >> 2) + 4 * g + (j & 3);
      const float x = (f < m && dd < d) ? omega[((size_t)h * m + f) * d + dd] * scale : 0.f;
      split2(x, xh, xl, j);
    }
    st8<C>(hi + (size_t)id * 8, xh);
    st8<C>(lo + (size_t)id * 8, xl);
  }
}

// ---------------------------------------------------------------- forward recomputed
// Workgroup = NW waves on segment sp of (b,h) (piece pc = bh * nseg + sp), wave w owning the 32
// features [32w, 32w + 32). The segment's carry S' (from the scan, in the scale of its key maximum
// M) is held as Sc[fb][nb] = C[feature][column]. Per chunk of 32 tokens (Q, K, V and dOut rows
// through a two-slot DMA ring):
//   X   projections as in the forward sweep (keys against M, queries against the norm bound or,
//       rarely, their exact maximum: the bias b_i); Phi'_K and Phi'_Q as hi + lo operands;
//       o^T = S'^T Phi'_Q^T (A = Sc) + [V 1]^T masked (Phi'_K Phi'_Q^T), the wave's partial to its
//       LDS buffer (fp32 inputs: LDS atomics into one sum, for want of LDS); Sc takes the chunk
//   Y   per query: D' = o_z, out = o / D', gamma = g . out; l = b + log2 D' and gamma to HBM
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
cbwd_fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                const T* __restrict__ dOut, const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo,
                const float* __restrict__ cpart, const float* __restrict__ cz, const float* __restrict__ cmax, int H,
                int L, int seg_len, int nseg, float nscale, float* __restrict__ lg, float* __restrict__ gam,
                float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB == 2, "one 32-feature chunk per wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NVB = DV / 16, NB = NVB + 1;
  constexpr int NFC = M / 32;
  constexpr int NSPL = CbwdOps<T>::NSPL;
  constexpr int CPR = DV / 8;  // 8-column items of a row
  static_assert(32 * CPR <= NT && (32 * CPR) % 64 == 0, "one (row, 8 columns) item per thread, whole waves");
  constexpr int KPROW = 36;    // a wave's Phi'_K transpose [feature][key]
  constexpr int OROW = NB * 16 + 4;
  constexpr bool XOW = sizeof(T) == 2;      // per-wave partial outputs (else LDS atomics)
  constexpr int XO = 2 * NVB * 256 + 32;    // floats of one wave's partial output
  using Rg = SweepRing<T, D, DV, NT, true>;
  using VR = Ring<T, D, DV, NT, true>;  // V and G rows share its layout
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) C ubuf[NSPL][NW * 32 * KPROW];  // the waves' Phi'_K transposes (hi, lo)
  __shared__ __attribute__((aligned(16))) float osum[XOW ? 1 : 2][XOW ? 4 : 32 * OROW];
  __shared__ __attribute__((aligned(16))) float xo[XOW ? NW : 1][XOW ? XO : 4];
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  __shared__ __attribute__((aligned(16))) float qn[2][32];
  __shared__ __attribute__((aligned(16))) float qmx[NW][32];
  __shared__ float qbias[32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  Rg::issue(Q, K, V, L, rowbase, t0, ring0, dOut);
  if constexpr (!XOW)
    for (int e = threadIdx.x; e < 2 * 32 * OROW; e += NT) (&osum[0][0])[e] = 0.f;

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
  // the carry at the segment's start: this wave's 32-feature chunk of the scan's fragments
  f32x4 Sc[FB][NB];
  {
    const size_t fcb = (size_t)pc * NFC + w;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
      if (nb < NVB) {
        const float* src = cpart + ((fcb * NVB + nb) * 64 + lane) * 8;
        lo = reinterpret_cast<const f32x4*>(src)[0];
        hi = reinterpret_cast<const f32x4*>(src)[1];
      } else if (c == 0) {
        const float* src = cz + (fcb * 4 + g) * 8;
        lo = reinterpret_cast<const f32x4*>(src)[0];
        hi = reinterpret_cast<const f32x4*>(src)[1];
      }
      Sc[0][nb] = lo;
      Sc[1][nb] = hi;
    }
  }
  const float mk = cmax[pc];
  const float omax = omega_norm_max<NW>(om, &qmx[0][0], 32);
  wait_vmcnt<0>();
  Rg::template convert<P>(ring[0], qn[0], kn[0], nscale, tend - t0);

  for (int t = 0; t < n; ++t) {
    const int buf = t & 1;
    const unsigned char* sl = ring[buf];
    const unsigned char* vbase = sl + Rg::XC * 16;
    const unsigned char* gbase = sl + (Rg::XC + Rg::VC) * 16;
    const int tok0 = t0 + 32 * t;
    float* os = osum[XOW ? 0 : buf];
    lds_barrier();  // X: chunk t converted; the previous chunk's reads of the other slot and of osum done
    if (t + 1 < n) Rg::issue(Q, K, V, L, rowbase, tok0 + 32, ring0 + (buf ^ 1) * Rg::SLOT, dOut);

    // ---- projections: keys [key][feature] from -(n'_k + M), queries [feature][query] from -b
    f32x4 pk[2][FB], pq[2][FB];
    bool exact = false;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 kbias;
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) kbias[i] = proj_start<KIND>(-(n4[i] + mk));
      const float b = KIND == kPrf ? qn[buf][tb * 16 + c] * omax : 0.f;
      exact |= b > kQueryBoundLimit;
      vec8<P> kf[DC], qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 1, tb * 16 + c, col) : zero8<P>();
        qf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 0, tb * 16 + c, col) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pk[tb][fb] = kbias;
        pq[tb][fb] = f32x4{-b, -b, -b, -b};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          mma16_split_b<PSO>(pk[tb][fb], kf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
          mma16_split_a<PSO>(pq[tb][fb], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0], qf[dc]);
        }
      }
    }
    float qsh[2] = {0.f, 0.f};
    if (__builtin_amdgcn_ballot_w64(exact) != 0) {  // the same in every wave
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = -INFINITY;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pq[tb][fb][i]);
        mx = group_max(mx);
        if (g == 0) qmx[w][tb * 16 + c] = mx;
      }
      lds_barrier();
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = qmx[0][tb * 16 + c];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, qmx[ww][tb * 16 + c]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) pq[tb][fb] -= mx;
        qsh[tb] = mx;
      }
    }
    if (w == 0 && g == 0)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) qbias[tb * 16 + c] = KIND == kPrf ? qn[buf][tb * 16 + c] * omax + qsh[tb] : 0.f;

    // ---- features: Phi'_K^T (A [feature][key], paired key slots), Phi'_Q (B [feature][query],
    // paired feature slots), each as hi + lo
    vec8<C> afh[FB], afl[FB], bqh[2], bql[2];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
      split_all<8>(afh[fb], afl[fb], [&](int j) { return key_feature<KIND>(pk[j >> 2][fb][j & 3], inv_sqrt_m, eps); });
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
      split_all<8>(bqh[tb], bql[tb], [&](int j) { return key_feature<KIND>(pq[tb][j >> 2][j & 3], inv_sqrt_m, eps); });

    // ---- forward, carried term: o^T[col][q] = S'^T (A: Sc, paired feature slots) x Phi'_Q
    f32x4 o[NB][2];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      vec8<C> sh, slo;
      split_all<8>(sh, slo, [&](int j) { return Sc[j >> 2][cb][j & 3]; });
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        o[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma_split<NSPL>(o[cb][tb], sh, slo, bqh[tb], bql[tb]);
      }
    }
    // ---- forward, intra-chunk scores over this wave's features: A^T[key][q] = Phi'_K Phi'_Q^T, hi + lo
    // (for peaked attention a few features carry a score, so their roundings do not average out)
    f32x4 sc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb][0] = sc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int sp = 0; sp < NSPL; ++sp) {
        C* ph = &ubuf[sp][w * 32 * KPROW];  // wave-private: [feature][key]
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          vec4<C> lo4, hi4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lo4[i] = sp == 0 ? afh[hh][i] : afl[hh][i];
            hi4[i] = sp == 0 ? afh[hh][i + 4] : afl[hh][i + 4];
          }
          *reinterpret_cast<vec4<C>*>(ph + (16 * hh + c) * KPROW + 4 * g) = lo4;
          *reinterpret_cast<vec4<C>*>(ph + (16 * hh + c) * KPROW + 16 + 4 * g) = hi4;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const vec8<C> kah = tr_read8<C>(&ubuf[0][w * 32 * KPROW], KPROW, 0, kb * 16, c, g);  // A [key][feature]
        const vec8<C> kal = NSPL == 2 ? tr_read8<C>(&ubuf[NSPL - 1][w * 32 * KPROW], KPROW, 0, kb * 16, c, g) : kah;
        mma_split<NSPL>(sc[kb][0], kah, kal, bqh[0], bql[0]);
        mma_split<NSPL>(sc[kb][1], kah, kal, bqh[1], bql[1]);
      }
    }
    // ---- forward, intra term: o^T += [V 1]^T (A: value fragments) x masked A^T (B, hi + lo)
    vec8<C> vf[NB];
    value_frags<T, D, DV, NT>(vbase, vf, c, g);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<C> sbh, sbl;
      split_all<8>(sbh, sbl, [&](int jj) {
        const int kb = jj >> 2, i = jj & 3;
        const int key = kb * 16 + 4 * g + i, qry = tb * 16 + c;
        return key <= qry ? sc[kb][tb][i] : 0.f;
      });
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        mma16(o[cb][tb], vf[cb], sbh);
        if constexpr (NSPL == 2) mma16(o[cb][tb], vf[cb], sbl);
      }
    }
    // the wave's partial outputs (value columns and the denominator)
    if constexpr (XOW) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int cb = 0; cb < NVB; ++cb)
          *reinterpret_cast<f32x4*>(&xo[w][((tb * NVB + cb) * 64 + lane) * 4]) = o[cb][tb];
        if (g == 0) xo[w][2 * NVB * 256 + tb * 16 + c] = o[NB - 1][tb][0];
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = cb * 16 + 4 * g + i;
            if (col <= DV) atomicAdd(&os[(tb * 16 + c) * OROW + col], o[cb][tb][i]);
          }
    }
    // ---- Sc takes the chunk
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        mma16(Sc[fb][nb], afh[fb], vf[nb]);
        if constexpr (NSPL == 2) mma16(Sc[fb][nb], afl[fb], vf[nb]);
      }
    lds_barrier();  // Y: the chunk's summed outputs

    // ---- per query: D' and gamma = g . out; l = b + log2 D' and gamma to HBM
    if (threadIdx.x < 32 * CPR) {
      const int row = threadIdx.x / CPR, c8 = threadIdx.x % CPR;
      float den = 0.f;
      f32x4 o0 = f32x4{0.f, 0.f, 0.f, 0.f}, o1 = o0;
      if constexpr (XOW) {
        const int tb = row >> 4, cq = row & 15, cb = (c8 * 8) >> 4, g0 = ((c8 * 8) & 15) >> 2;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float* base = &xo[ww][((tb * NVB + cb) * 64 + cq + 16 * g0) * 4];
          o0 += *reinterpret_cast<const f32x4*>(base);
          o1 += *reinterpret_cast<const f32x4*>(base + 64);
          den += xo[ww][2 * NVB * 256 + tb * 16 + cq];
        }
      } else {
        const float* orow = &os[row * OROW];
        den = orow[DV];
        o0 = *reinterpret_cast<const f32x4*>(orow + c8 * 8);
        o1 = *reinterpret_cast<const f32x4*>(orow + c8 * 8 + 4);
      }
      const vec8<T> g8 = ld8<T>(reinterpret_cast<const T*>(gbase + VR::v_off(row, c8 * 8)));
      float ga = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) ga += to_f(g8[j]) * o0[j] + to_f(g8[j + 4]) * o1[j];
      ga = lanes_sum<CPR>(ga);
      if (c8 == 0) {
        const float gm = ga * __builtin_amdgcn_rcpf(den);  // hardware reciprocal (1 ulp)
        const int tok = tok0 + row;
        if (tok < tend) {
          lg[rowbase + tok] = qbias[row] + log2f(den);
          gam[rowbase + tok] = gm;
        }
      }
    }
    if constexpr (!XOW)
      for (int e = threadIdx.x; e < 32 * OROW; e += NT) osum[buf ^ 1][e] = 0.f;  // for chunk t+1
    // ---- chunk t+1 lands and is converted
    if (t + 1 < n) {
      wait_vmcnt<0>();
      Rg::template convert<P>(ring[buf ^ 1], qn[buf ^ 1], kn[buf ^ 1], nscale, tend - tok0 - 32);
    }
  }
}

// ---------------------------------------------------------------- query gradient
// Workgroup = NW waves on segment sp of (b,h), wave w owning features [32w, 32w + 32). The carry
// S' is held as St[nb][fb] = C[column][feature]. Per chunk (Q, K, V and dOut rows through a
// two-slot DMA ring; l and gamma per query prefetched a chunk ahead):
//   X   projections: keys [key][feature] against M (Phi'_K, hi + lo A operand), queries
//       [feature][query] against l (phi~ = Phi'_Q / D')
//       dPhi~^T[f][q] = S'[f][col] (A: St, hi + lo) x [g_q, -gamma_q] (B) + Phi'_K^T (A) x B with
//       the masked scores B[key][q] = g_q . v_key - gamma_q (key <= q, hi + lo); then
//       P = phi~ * dPhi~ = phi_Q * dPhi_Q as rows [query][feature] (hi + lo); St takes the chunk
//   P   dq^T blocks = Omega'^T P / log2(e), every wave its share over all features (the head's
//       Omega'^T hi/lo fragments staged in LDS once per workgroup)
// KIND = kRelu: pq holds the derivative factor 1[a > 0] 2^-l / sqrt(m) in place of phi~, and dq takes no
// 1/log2(e).
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
cbwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dOut,
              const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo, const typename Ops<T>::C* __restrict__ omTh,
              const typename Ops<T>::C* __restrict__ omTl, const float* __restrict__ cpart,
              const float* __restrict__ cz, const float* __restrict__ cmax, const float* __restrict__ lg,
              const float* __restrict__ gam, int H, int L, int seg_len, int nseg, float nscale, int grad_f32,
              void* __restrict__ dq, float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB == 2, "one 32-feature chunk per wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NDB = D / 16, NVB = DV / 16, NB = NVB + 1;
  constexpr int NFC = M / 32;
  constexpr int KC = (NB + 1) / 2;     // 32-column chunks of [value columns, z]
  constexpr int KCV = (DV + 31) / 32;  // 32-column chunks of the value columns
  constexpr int BPW = 2 * NDB / NW;    // dq^T blocks (dims db, queries tb) per wave
  static_assert(BPW >= 1 && (2 * NDB) % NW == 0, "dq blocks split evenly over the waves");
  constexpr int NSPL = CbwdOps<T>::NSPL;
  constexpr int PROW = M + 8;  // P rows [query][feature]
  using Rg = SweepRing<T, D, DV, NT, true>;
  using VR = Ring<T, D, DV, NT, true>;
  constexpr int OMT = NDB * NFC * 512;  // elements of one head's Omega'^T fragments
  constexpr bool STAGE = sizeof(C) == 2;  // those fragments in LDS (fp32: read from the cache, for want of LDS)
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) C omts[NSPL][STAGE ? OMT : 8];
  __shared__ __attribute__((aligned(16))) C prow[NSPL][32 * PROW];
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  __shared__ __attribute__((aligned(16))) float qn[2][32];
  __shared__ __attribute__((aligned(16))) float rl[2][32];
  __shared__ __attribute__((aligned(16))) float rgm[2][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  float pl = INFINITY, pg = 0.f;  // l and gamma of a chunk, threads < 32
  auto fetch = [&](int tok0) {
    if (threadIdx.x < 32) {
      const int tok = tok0 + threadIdx.x;
      pl = tok < tend ? lg[rowbase + tok] : INFINITY;
      pg = tok < tend ? gam[rowbase + tok] : 0.f;
    }
  };
  Rg::issue(Q, K, V, L, rowbase, t0, ring0, dOut);
  if constexpr (STAGE)
    stage_omT<NT, OMT * (int)sizeof(C), C>(omTh + (size_t)h * OMT, NSPL == 2 ? omTl + (size_t)h * OMT : nullptr,
                                           omts[0], omts[NSPL - 1]);
  fetch(t0);

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
  // St[nb][fb][i] = S'[feature 16fb + c][column 16nb + 4g + i]: lane (4g + i) + 16(c >> 2), slot 4fb + (c & 3)
  // of the scan's fragments of this wave's 32-feature chunk
  f32x4 St[NB][FB];
  {
    const size_t fcb = (size_t)pc * NFC + w;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int col = nb * 16 + 4 * g + i, j = 4 * fb + (c & 3);
          float x = 0.f;
          if (nb < NVB)
            x = cpart[((fcb * NVB + nb) * 64 + (4 * g + i) + 16 * (c >> 2)) * 8 + j];
          else if (col == DV)
            x = cz[(fcb * 4 + (c >> 2)) * 8 + j];
          St[nb][fb][i] = x;
        }
  }
  const float mk = cmax[pc];
  wait_vmcnt<0>();
  Rg::template convert<P>(ring[0], qn[0], kn[0], nscale, tend - t0);
  if (threadIdx.x < 32) {
    rl[0][threadIdx.x] = pl;
    rgm[0][threadIdx.x] = pg;
  }

  for (int t = 0; t < n; ++t) {
    const int buf = t & 1;
    const unsigned char* sl = ring[buf];
    const unsigned char* vbase = sl + Rg::XC * 16;
    const unsigned char* gbase = sl + (Rg::XC + Rg::VC) * 16;
    const int tok0 = t0 + 32 * t;
    lds_barrier();  // X: chunk t converted; the previous chunk's reads of the other slot and of the P rows done
    if (t + 1 < n) {
      Rg::issue(Q, K, V, L, rowbase, tok0 + 32, ring0 + (buf ^ 1) * Rg::SLOT, dOut);
      fetch(tok0 + 32);
    }
    // ---- projections: keys [key][feature] from -(n'_k + M), queries [feature][query] from -l
    vec8<C> afh[FB], afl[FB];  // Phi'_K^T: A [feature][key], paired key slots
    f32x4 pq[2][FB];           // phi~ [feature][query]
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 kbias;
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) kbias[i] = proj_start<KIND>(-(n4[i] + mk));
      const float ql = rl[buf][tb * 16 + c];
      const float qb = proj_start<KIND>(-ql);
      vec8<P> kf[DC], qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 1, tb * 16 + c, col) : zero8<P>();
        qf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 0, tb * 16 + c, col) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        f32x4 pk = kbias;
        pq[tb][fb] = f32x4{qb, qb, qb, qb};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          mma16_split_b<PSO>(pk, kf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
          mma16_split_a<PSO>(pq[tb][fb], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0], qf[dc]);
        }
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          split_pair(key_feature<KIND>(pk[i], inv_sqrt_m, eps), key_feature<KIND>(pk[i + 1], inv_sqrt_m, eps), afh[fb],
                     afl[fb], 4 * tb + i);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (KIND == kPrf)
            pq[tb][fb][i] = fast_exp2(pq[tb][fb][i]);
          else
            pq[tb][fb][i] = pq[tb][fb][i] > 0.f ? inv_sqrt_m * fast_exp2(-ql) : 0.f;
        }
      }
    }
    // ---- carried part: dPhi~^T[f][q] = S'[f][col] (A: St, paired column slots, hi + lo) x
    // [g_q, -gamma_q] (B, paired column slots)
    f32x4 dph[FB][2];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) dph[fb][0] = dph[fb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      vec8<C> sth[FB], stl[FB];
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
        split_all<8>(sth[fb], stl[fb], [&](int j) {
          const int nb = 2 * kc + (j >> 2);
          return nb < NB ? St[nb][fb][j & 3] : 0.f;
        });
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int qr = tb * 16 + c;
        vec8<C> gh, gl;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int col0 = kc * 32 + 16 * hf + 4 * g;
          if (col0 < DV) {
            const vec4<T> g4 = *reinterpret_cast<const vec4<T>*>(gbase + VR::v_off(qr, col0));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              gh[4 * hf + i] = to_t<C>(to_f(g4[i]));
              gl[4 * hf + i] = to_t<C>(0.f);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; i += 2)
              split_pair(col0 + i == DV ? -rgm[buf][qr] : 0.f, col0 + i + 1 == DV ? -rgm[buf][qr] : 0.f, gh, gl,
                         4 * hf + i);
          }
        }
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          mma16(dph[fb][tb], sth[fb], gh);
          if constexpr (NSPL == 2) {
            mma16(dph[fb][tb], stl[fb], gh);
            if (kc == DV / 32) mma16(dph[fb][tb], sth[fb], gl);  // the chunk that holds the gamma column
          }
        }
      }
    }
    // ---- intra part: B[key][q] = g_q . v_key - gamma_q for key <= q (A: V rows, B: g rows, linear
    // column slots), dPhi~^T += Phi'_K^T (A, hi + lo) x B (hi + lo)
    {
      f32x4 bs[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) bs[kb][0] = bs[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kcv = 0; kcv < KCV; ++kcv) {
        const int col = kcv * 32 + 8 * g;
        vec8<C> va[2], gb[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          va[x] = col < DV ? cvt8<C, T>(ld8<T>(reinterpret_cast<const T*>(vbase + VR::v_off(x * 16 + c, col))))
                           : zero8<C>();
          gb[x] = col < DV ? cvt8<C, T>(ld8<T>(reinterpret_cast<const T*>(gbase + VR::v_off(x * 16 + c, col))))
                           : zero8<C>();
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) mma16(bs[kb][tb], va[kb], gb[tb]);
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int qr = tb * 16 + c;
        const float gq = rgm[buf][qr];
        vec8<C> bh, bl;
        split_all<8>(bh, bl, [&](int jj) {
          const int kb = jj >> 2, i = jj & 3;
          const int key = kb * 16 + 4 * g + i;
          return key <= qr ? bs[kb][tb][i] - gq : 0.f;
        });
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) mma_split<NSPL>(dph[fb][tb], afh[fb], afl[fb], bh, bl);
      }
    }
    // ---- P = phi~ * dPhi~, rows [query][feature] as hi + lo
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        vec4<C> h4, l4;
        split_all<4>(h4, l4, [&](int i) { return pq[tb][fb][i] * dph[fb][tb][i]; });
        const int off = (tb * 16 + c) * PROW + w * 32 + fb * 16 + 4 * g;
        *reinterpret_cast<vec4<C>*>(&prow[0][off]) = h4;
        if constexpr (NSPL == 2) *reinterpret_cast<vec4<C>*>(&prow[NSPL - 1][off]) = l4;
      }
    // ---- St takes the chunk: St[col][f] += [V 1]^T (A) x Phi'_K (B)
    {
      vec8<C> vf[NB];
      value_frags<T, D, DV, NT>(vbase, vf, c, g);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          mma16(St[nb][fb], vf[nb], afh[fb]);
          if constexpr (NSPL == 2) mma16(St[nb][fb], vf[nb], afl[fb]);
        }
    }
    lds_barrier();  // P rows of every wave

    // ---- dq: this wave's blocks of dq^T over all features: A = Omega'^T (hi + lo), B = P rows
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = w * BPW + bi, db = blk >> 1, tb = blk & 1;
      const int qr = tb * 16 + c;
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc) {
        const int fo = ((db * NFC + fc) * 64 + lane) * 8;
        const C* oth = STAGE ? &omts[0][0] : omTh + (size_t)h * OMT;
        const C* otl = STAGE ? &omts[NSPL - 1][0] : omTl + (size_t)h * OMT;
        const vec8<C> oh = ld8<C>(oth + fo);
        const vec8<C> ol = NSPL == 2 ? ld8<C>(otl + fo) : oh;
        const vec8<C> p8h = pair_read8<C>(&prow[0][qr * PROW], fc * 32, g);
        const vec8<C> p8l = NSPL == 2 ? pair_read8<C>(&prow[NSPL - 1][qr * PROW], fc * 32, g) : p8h;
        mma_split<NSPL>(a, oh, ol, p8h, p8l);
      }
      const int tok = tok0 + qr;
      if (tok < tend) {
        const size_t off = (rowbase + tok) * D + db * 16 + 4 * g;
        if constexpr (KIND == kPrf) a = a * (1.f / kLog2e);
        if (grad_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dq) + off) = a;
        } else {
          vec4<T> o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = to_t<T>(a[i]);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(dq) + off) = o4;
        }
      }
    }
    // ---- chunk t+1 lands and is converted
    // (the wait on every path: otherwise the compiler, which does not see the ring's copies, takes the next
    // iteration's fetch() loads as possibly outstanding and waits for every copy right after issuing them)
    wait_vmcnt<0>();
    if (t + 1 < n) {
      Rg::template convert<P>(ring[buf ^ 1], qn[buf ^ 1], kn[buf ^ 1], nscale, tend - tok0 - 32);
      if (threadIdx.x < 32) {
        rl[buf ^ 1][threadIdx.x] = pl;
        rgm[buf ^ 1][threadIdx.x] = pg;
      }
    }
  }
}

// ---------------------------------------------------------------- segment totals of the key side
// Workgroup = NW waves on segment sp of (b,h), wave w owning features [32w, 32w + 32). Per chunk
// (Q and dOut rows through a two-slot DMA ring, l and gamma per query prefetched a chunk ahead):
//   projection [query][feature] from -l_q: phi~ = 2^(a' - l) (0 for queries outside the segment)
//   T[f][col] += phi~^T (A, paired query slots, hi + lo) x [g, -gamma] (B: value fragments of the
//   g rows, exact; the gamma block built in registers, hi + lo)
// The total goes to trow[pc] as fp32 rows [feature][NB*16].
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
cbwd_t_kernel(const T* __restrict__ Q, const T* __restrict__ dOut, const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo,
              const float* __restrict__ lg, const float* __restrict__ gam, int H, int L, int seg_len, int nseg,
              float* __restrict__ trow, float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB == 2, "one 32-feature chunk per wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NVB = DV / 16, NB = NVB + 1, NBC = NB * 16;
  constexpr int KROW = D + 8;
  constexpr int NSPL = CbwdOps<T>::NSPL;
  using Rg = Ring<T, D, DV, NT, true>;  // Q rows and dOut rows
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P qs[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float rl[2][32];
  __shared__ __attribute__((aligned(16))) float rgm[2][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  float pl = INFINITY, pg = 0.f;  // l and gamma of a chunk, threads < 32
  auto fetch = [&](int tok0) {
    if (threadIdx.x < 32) {
      const int tok = tok0 + threadIdx.x;
      pl = tok < tend ? lg[rowbase + tok] : INFINITY;
      pg = tok < tend ? gam[rowbase + tok] : 0.f;
    }
  };
  Rg::issue(Q, dOut, L, bh, t0, true, ring0);
  fetch(t0);
  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
  f32x4 Ta[FB][NB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) Ta[fb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  wait_vmcnt<0>();
  Rg::template convert<P, KROW, kNormNone>(ring[0], qs[0], nullptr, 0.f, L);
  if (threadIdx.x < 32) {
    rl[0][threadIdx.x] = pl;
    rgm[0][threadIdx.x] = pg;
  }

  for (int t = 0; t < n; ++t) {
    const int buf = t & 1;
    const int tok0 = t0 + 32 * t;
    lds_barrier();
    if (t + 1 < n) {
      Rg::issue(Q, dOut, L, bh, tok0 + 32, true, ring0 + (buf ^ 1) * Rg::SLOT);
      fetch(tok0 + 32);
    }
    f32x4 pq[2][FB];
    f32x4 lq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x4 bias;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rl[buf][qb * 16 + 4 * g]);
      lq[qb] = l4;
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = proj_start<KIND>(-l4[i]);
      vec8<P> qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        qf[dc] = (col < D) ? ld8<P>(&qs[buf][(qb * 16 + c) * KROW + col]) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pq[qb][fb] = bias;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16_split_b<PSO>(pq[qb][fb], qf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
      }
    }
    vec8<C> ah[FB], al[FB];  // phi~^T: A [feature][query], paired query slots
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
      split_all<8>(ah[fb], al[fb],
                   [&](int j) { return query_feature<KIND>(pq[j >> 2][fb][j & 3], lq[j >> 2][j & 3], inv_sqrt_m, eps); });
    vec8<C> wv[NB];
    value_frags<T, D, DV, NT>(ring[buf], wv, c, g);
    vec8<C> zh, zl;  // the -gamma column (c == 0 of the last block)
    split_all<8>(zh, zl, [&](int j) {
      const int q = 16 * (j >> 2) + 4 * g + (j & 3);
      return c == 0 ? -rgm[buf][q] : 0.f;
    });
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
      for (int nb = 0; nb < NVB; ++nb) {
        mma16(Ta[fb][nb], ah[fb], wv[nb]);
        if constexpr (NSPL == 2) mma16(Ta[fb][nb], al[fb], wv[nb]);
      }
      mma_split<NSPL>(Ta[fb][NVB], ah[fb], al[fb], zh, zl);
    }
    wait_vmcnt<0>();  // on every path (see cbwd_q_kernel)
    if (t + 1 < n) {
      Rg::template convert<P, KROW, kNormNone>(ring[buf ^ 1], qs[buf ^ 1], nullptr, 0.f, L);
      if (threadIdx.x < 32) {
        rl[buf ^ 1][threadIdx.x] = pl;
        rgm[buf ^ 1][threadIdx.x] = pg;
      }
    }
  }
  float* dst = trow + (size_t)pc * M * NBC;
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(size_t)(w * 32 + fb * 16 + 4 * g + i) * NBC + nb * 16 + c] = Ta[fb][nb][i];
}

// ---------------------------------------------------------------- suffix carries over segments
// In place, per (b,h) and element of the [M][NB*16] rows: C_p = (C_{p+1} + T_{p+1}) 2^(M_p - M_{p+1}),
// C_last = 0 (the prefix key maxima M_p do not decrease, so every factor is at most 1).
__global__ void __launch_bounds__(256)
cbwd_rscan_kernel(float* __restrict__ trow, const float* __restrict__ cmax, int nseg, int per, int nblk) {
  const int bh = blockIdx.x / nblk;
  const int e = (blockIdx.x % nblk) * 256 + threadIdx.x;
  if (e >= per) return;
  float acc = 0.f;
  for (int p = nseg - 1; p >= 0; --p) {
    const size_t slot = (size_t)bh * nseg + p;
    float* x = trow + slot * per + e;
    const float tv = *x;
    *x = acc;
    if (p > 0) acc = (acc + tv) * fast_exp2(cmax[slot - 1] - cmax[slot]);
  }
}

// ---------------------------------------------------------------- key gradient
// Workgroup = NW waves on segment sp of (b,h), wave w owning features [32w, 32w + 32); the chunks
// run backwards from the segment's end. The suffix state R'' (the later segments' carry, then the
// chunks already passed) is held as Rc[nb][fb] = C[column][feature]. Per chunk:
//   X   projections [token][feature]: keys against M (phi'_K), queries against l (phi~)
//       Bt[q][key] = g_q . v_key (A = g rows, B = V rows), B = Bt - gamma_q for q >= key
//       dPhi''_K[key][f] = [V 1] (A, exact) x Rc (B, hi + lo) + B (A, hi + lo) x phi~ (B, hi + lo)
//       P = phi'_K * dPhi''_K as rows [feature][key] (hi + lo), rho = its sum over the wave's
//       features; Rc takes the chunk's queries
//   B1  dk^T blocks = Omega'^T P / log2(e) - d^-1/2 k rho over all features (Omega'^T staged in
//       LDS once per workgroup)
// KIND = kRelu: pk holds the key's derivative factor 1[a > 0]/sqrt(m) in place of phi'_K; dk has no
// 1/log2(e) and no norm term.
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
cbwd_k_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dOut,
              const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo, const typename Ops<T>::C* __restrict__ omTh,
              const typename Ops<T>::C* __restrict__ omTl, const float* __restrict__ rcar,
              const float* __restrict__ cmax, const float* __restrict__ lg, const float* __restrict__ gam, int H,
              int L, int seg_len, int nseg, float nscale, float s2, int grad_f32, void* __restrict__ dk,
              float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB == 2, "one 32-feature chunk per wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NDB = D / 16, NVB = DV / 16, NB = NVB + 1, NBC = NB * 16;
  constexpr int NFC = M / 32;
  constexpr int KC = (NB + 1) / 2;
  constexpr int KCV = (DV + 31) / 32;
  constexpr int BPWK = 2 * NDB / NW;
  static_assert(BPWK >= 1 && (2 * NDB) % NW == 0, "dk blocks split evenly over the waves");
  constexpr int NSPL = CbwdOps<T>::NSPL;
  constexpr int FROW = 36;  // [feature][token] rows
  using Rg = SweepRing<T, D, DV, NT, true>;
  using VR = Ring<T, D, DV, NT, true>;
  constexpr int OMT = NDB * NFC * 512;  // elements of one head's Omega'^T fragments
  constexpr bool STAGE = sizeof(C) == 2;  // those fragments in LDS (fp32: read from the cache, for want of LDS)
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) C omts[NSPL][STAGE ? OMT : 8];
  __shared__ __attribute__((aligned(16))) C ft[NSPL][M * FROW];  // P: [feature][key]
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  __shared__ __attribute__((aligned(16))) float qn[2][32];
  __shared__ __attribute__((aligned(16))) float rl[2][32];
  __shared__ __attribute__((aligned(16))) float rgm[2][32];
  __shared__ __attribute__((aligned(16))) float rho[32][NW];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  float pl = INFINITY, pg = 0.f;
  auto fetch = [&](int tok0) {
    if (threadIdx.x < 32) {
      const int tok = tok0 + threadIdx.x;
      pl = tok < tend ? lg[rowbase + tok] : INFINITY;
      pg = tok < tend ? gam[rowbase + tok] : 0.f;
    }
  };
  const int last0 = t0 + 32 * (n - 1);
  Rg::issue(Q, K, V, L, rowbase, last0, ring0, dOut);
  if constexpr (STAGE)
    stage_omT<NT, OMT * (int)sizeof(C), C>(omTh + (size_t)h * OMT, NSPL == 2 ? omTl + (size_t)h * OMT : nullptr,
                                           omts[0], omts[NSPL - 1]);
  fetch(last0);

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
  f32x4 Rc[NB][FB];
  {
    const float* src = rcar + (size_t)pc * M * NBC;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
        Rc[nb][fb] = *reinterpret_cast<const f32x4*>(src + (size_t)(w * 32 + fb * 16 + c) * NBC + nb * 16 + 4 * g);
  }
  const float mk = cmax[pc];
  wait_vmcnt<0>();
  Rg::template convert<P>(ring[0], qn[0], kn[0], nscale, tend - last0);
  if (threadIdx.x < 32) {
    rl[0][threadIdx.x] = pl;
    rgm[0][threadIdx.x] = pg;
  }

  for (int it = 0; it < n; ++it) {
    const int t = n - 1 - it;
    const int buf = it & 1;
    const unsigned char* sl = ring[buf];
    const unsigned char* vbase = sl + Rg::XC * 16;
    const unsigned char* gbase = sl + (Rg::XC + Rg::VC) * 16;
    const int tok0 = t0 + 32 * t;
    lds_barrier();  // X: chunk t converted; the previous chunk's reads done
    if (t > 0) {
      Rg::issue(Q, K, V, L, rowbase, tok0 - 32, ring0 + (buf ^ 1) * Rg::SLOT, dOut);
      fetch(tok0 - 32);
    }
    // ---- projections [token][feature]: keys from -(n'_k + M), queries from -l_q; then the features
    f32x4 pk[2][FB], pq[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 kbias, qbias;
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rl[buf][tb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kbias[i] = proj_start<KIND>(-(n4[i] + mk));
        qbias[i] = proj_start<KIND>(-l4[i]);
      }
      vec8<P> kf[DC], qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 1, tb * 16 + c, col) : zero8<P>();
        qf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 0, tb * 16 + c, col) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pk[tb][fb] = kbias;
        pq[tb][fb] = qbias;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          mma16_split_b<PSO>(pk[tb][fb], kf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
          mma16_split_b<PSO>(pq[tb][fb], qf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (KIND == kPrf)
            pk[tb][fb][i] = fast_exp2(pk[tb][fb][i]);
          else
            pk[tb][fb][i] = pk[tb][fb][i] > 0.f ? inv_sqrt_m : 0.f;  // the derivative factor
          pq[tb][fb][i] = query_feature<KIND>(pq[tb][fb][i], l4[i], inv_sqrt_m, eps);
        }
      }
    }
    // phi~ as B [query][feature] (paired query slots), hi + lo
    vec8<C> qbh[FB], qbl[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) split_all<8>(qbh[fb], qbl[fb], [&](int j) { return pq[j >> 2][fb][j & 3]; });
    // ---- scores Bt[q][key] = g_q . v_key; A operand [key][query] of B = Bt - gamma_q, q >= key
    vec8<C> bah[2], bal[2];
    {
      f32x4 bt[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) bt[qb][0] = bt[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kcv = 0; kcv < KCV; ++kcv) {
        const int col = kcv * 32 + 8 * g;
        vec8<C> ga[2], va[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          ga[x] = col < DV ? cvt8<C, T>(ld8<T>(reinterpret_cast<const T*>(gbase + VR::v_off(x * 16 + c, col))))
                           : zero8<C>();
          va[x] = col < DV ? cvt8<C, T>(ld8<T>(reinterpret_cast<const T*>(vbase + VR::v_off(x * 16 + c, col))))
                           : zero8<C>();
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma16(bt[qb][kb], ga[qb], va[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        split_all<8>(bah[kb], bal[kb], [&](int jj) {
          const int qb = jj >> 2, i = jj & 3;
          const int q = qb * 16 + 4 * g + i, key = kb * 16 + c;
          return q >= key ? bt[qb][kb][i] - rgm[buf][q] : 0.f;
        });
    }
    // ---- dPhi''_K[key][f]: [V 1] (A, paired column slots) x Rc (B, hi + lo), + B x phi~
    f32x4 dpk[2][FB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dpk[kb][0] = dpk[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      vec8<C> rh[FB], rlo[FB];
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
        split_all<8>(rh[fb], rlo[fb], [&](int j) {
          const int nb = 2 * kc + (j >> 2);
          return nb < NB ? Rc[nb][fb][j & 3] : 0.f;
        });
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 16 + c;
        vec8<C> va8;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int col0 = kc * 32 + 16 * hf + 4 * g;
          if (col0 < DV) {
            const vec4<T> v4 = *reinterpret_cast<const vec4<T>*>(vbase + VR::v_off(key, col0));
#pragma unroll
            for (int i = 0; i < 4; ++i) va8[4 * hf + i] = to_t<C>(to_f(v4[i]));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) va8[4 * hf + i] = to_t<C>(col0 + i == DV ? 1.f : 0.f);
          }
        }
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          mma16(dpk[kb][fb], va8, rh[fb]);
          if constexpr (NSPL == 2) mma16(dpk[kb][fb], va8, rlo[fb]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) mma_split<NSPL>(dpk[kb][fb], bah[kb], bal[kb], qbh[fb], qbl[fb]);
    // ---- P = phi'_K * dPhi''_K and its sum over this wave's features per key
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 r4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        dpk[kb][fb] = pk[kb][fb] * dpk[kb][fb];
        r4 += dpk[kb][fb];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r = lanes_sum<16>(r4[i]);
        if (c == 0) rho[kb * 16 + 4 * g + i][w] = r;
      }
    }
    // ---- P rows [feature][key] (hi + lo)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        vec4<C> h4, l4;
        split_all<4>(h4, l4, [&](int i) { return dpk[kb][fb][i]; });
        const int off = (w * 32 + fb * 16 + c) * FROW + kb * 16 + 4 * g;
        *reinterpret_cast<vec4<C>*>(&ft[0][off]) = h4;
        if constexpr (NSPL == 2) *reinterpret_cast<vec4<C>*>(&ft[NSPL - 1][off]) = l4;
      }
    // ---- the suffix state takes the chunk's queries: Rc[col][f] += [g, -gamma]^T (A, paired query
    // slots) x phi~ (B)
    vec8<C> gv[NB];
    value_frags<T, D, DV, NT>(gbase, gv, c, g);
    {
      vec8<C> zh, zl;
      split_all<8>(zh, zl, [&](int j) {
        const int q = 16 * (j >> 2) + 4 * g + (j & 3);
        return c == 0 ? -rgm[buf][q] : 0.f;
      });
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
        for (int nb = 0; nb < NVB; ++nb) {
          mma16(Rc[nb][fb], gv[nb], qbh[fb]);
          if constexpr (NSPL == 2) mma16(Rc[nb][fb], gv[nb], qbl[fb]);
        }
        mma_split<NSPL>(Rc[NVB][fb], zh, zl, qbh[fb], qbl[fb]);
      }
    }
    lds_barrier();  // B1: P rows and rho of every wave

    // ---- dk: blocks of dk^T over all features: A = Omega'^T (hi + lo), B = P (transposing reads)
#pragma unroll
    for (int bi = 0; bi < BPWK; ++bi) {
      const int blk = w * BPWK + bi, db = blk >> 1, kb = blk & 1;
      const int key = kb * 16 + c;
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc) {
        const int fo = ((db * NFC + fc) * 64 + lane) * 8;
        const C* oth = STAGE ? &omts[0][0] : omTh + (size_t)h * OMT;
        const C* otl = STAGE ? &omts[NSPL - 1][0] : omTl + (size_t)h * OMT;
        const vec8<C> oh = ld8<C>(oth + fo);
        const vec8<C> ol = NSPL == 2 ? ld8<C>(otl + fo) : oh;
        const vec8<C> p8h = tr_read8<C>(ft[0], FROW, fc * 32, kb * 16, c, g);
        const vec8<C> p8l = NSPL == 2 ? tr_read8<C>(ft[NSPL - 1], FROW, fc * 32, kb * 16, c, g) : p8h;
        mma_split<NSPL>(a, oh, ol, p8h, p8l);
      }
      const int tok = tok0 + key;
      if (tok < tend) {
        float rs = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) rs += rho[key][ww];
        const int d0 = db * 16 + 4 * g;
        const vec4<P> k4 = *reinterpret_cast<const vec4<P>*>(sl + Rg::x_off(1, key, d0 / Rg::EPC) +
                                                             (d0 % Rg::EPC) * (int)sizeof(P));
        if constexpr (KIND == kPrf) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = a[i] * (1.f / kLog2e) - s2 * to_f(k4[i]) * rs;
        }
        const size_t off = (rowbase + tok) * D + d0;
        if (grad_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dk) + off) = a;
        } else {
          vec4<T> o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = to_t<T>(a[i]);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(dk) + off) = o4;
        }
      }
    }
    // ---- chunk t-1 lands and is converted
    wait_vmcnt<0>();  // on every path (see cbwd_q_kernel)
    if (t > 0) {
      Rg::template convert<P>(ring[buf ^ 1], qn[buf ^ 1], kn[buf ^ 1], nscale, tend - (tok0 - 32));
      if (threadIdx.x < 32) {
        rl[buf ^ 1][threadIdx.x] = pl;
        rgm[buf ^ 1][threadIdx.x] = pg;
      }
    }
  }
}

// ---------------------------------------------------------------- value gradient
// Workgroup = NW waves on segment sp of (b,h), wave w owning features [32w, 32w + 32); the chunks
// run backwards. The suffix state's value columns are held as Rt[fb][nb] = C[feature][column].
// Per chunk:
//   X   projections [token][feature]: keys against M (phi'_K), queries against l (phi~), written
//       as the wave's rows [feature][token] (hi + lo)
//       dv^T partial [col][key] = Rt (A, hi + lo) x phi'_K (B, transposing reads of those rows)
//                  + g^T (A: value fragments of the g rows) x masked (phi~ phi'_K^T, q >= key) (B),
//       written over the wave's rows once they are read; Rt takes the chunk's queries
//   B1  the waves' partials summed, dv stored
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
cbwd_v_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dOut,
              const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo, const float* __restrict__ rcar,
              const float* __restrict__ cmax, const float* __restrict__ lg, int H, int L, int seg_len, int nseg,
              float nscale, int grad_f32, void* __restrict__ dv, float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB == 2, "one 32-feature chunk per wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NVB = DV / 16, NB = NVB + 1, NBC = NB * 16;
  constexpr int NSPL = CbwdOps<T>::NSPL;
  constexpr int CPR = DV / 8;
  static_assert(32 * CPR <= NT, "one (row, 8 columns) item per thread");
  constexpr int FROW = 36;  // [feature][token] rows
  constexpr int FQ = 2 * NSPL * 32 * FROW;  // a wave's rows: phi'_K (hi, lo), phi~ (hi, lo)
  static_assert(FQ * (int)sizeof(C) >= 2 * NVB * 256 * 4, "a wave's partial dv fits over its rows");
  using Rg = SweepRing<T, D, DV, NT, true>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) C fq[NW][FQ];  // per wave: phi'_K and phi~ rows, then its dv partial
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  __shared__ __attribute__((aligned(16))) float qn[2][32];
  __shared__ __attribute__((aligned(16))) float rl[2][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  float pl = INFINITY;
  auto fetch = [&](int tok0) {
    if (threadIdx.x < 32) {
      const int tok = tok0 + threadIdx.x;
      pl = tok < tend ? lg[rowbase + tok] : INFINITY;
    }
  };
  const int last0 = t0 + 32 * (n - 1);
  Rg::issue(Q, K, V, L, rowbase, last0, ring0, dOut);
  fetch(last0);
  C* const fth = &fq[w][0];
  C* const ftl = &fq[w][(NSPL - 1) * 32 * FROW];
  C* const qth = &fq[w][NSPL * 32 * FROW];
  C* const qtl = &fq[w][(2 * NSPL - 1) * 32 * FROW];

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
  f32x4 Rt[FB][NVB];
  {
    const float* src = rcar + (size_t)pc * M * NBC;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NVB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) Rt[fb][nb][i] = src[(size_t)(w * 32 + fb * 16 + 4 * g + i) * NBC + nb * 16 + c];
  }
  const float mk = cmax[pc];
  wait_vmcnt<0>();
  Rg::template convert<P>(ring[0], qn[0], kn[0], nscale, tend - last0);
  if (threadIdx.x < 32) rl[0][threadIdx.x] = pl;

  for (int it = 0; it < n; ++it) {
    const int t = n - 1 - it;
    const int buf = it & 1;
    const unsigned char* sl = ring[buf];
    const unsigned char* gbase = sl + (Rg::XC + Rg::VC) * 16;
    const int tok0 = t0 + 32 * t;
    lds_barrier();  // X: chunk t converted; the previous chunk's reads done
    if (t > 0) {
      Rg::issue(Q, K, V, L, rowbase, tok0 - 32, ring0 + (buf ^ 1) * Rg::SLOT, dOut);
      fetch(tok0 - 32);
    }
    // ---- projections [token][feature]: keys from -(n'_k + M), queries from -l_q; then the features
    f32x4 pk[2][FB], pq[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 kbias, qbias;
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&rl[buf][tb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kbias[i] = proj_start<KIND>(-(n4[i] + mk));
        qbias[i] = proj_start<KIND>(-l4[i]);
      }
      vec8<P> kf[DC], qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 1, tb * 16 + c, col) : zero8<P>();
        qf[dc] = (col < D) ? Rg::template ld_x8<P>(sl, 0, tb * 16 + c, col) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pk[tb][fb] = kbias;
        pq[tb][fb] = qbias;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          mma16_split_b<PSO>(pk[tb][fb], kf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
          mma16_split_b<PSO>(pq[tb][fb], qf[dc], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[tb][fb][i] = key_feature<KIND>(pk[tb][fb][i], inv_sqrt_m, eps);
          pq[tb][fb][i] = query_feature<KIND>(pq[tb][fb][i], l4[i], inv_sqrt_m, eps);
        }
      }
    }
    // phi~ as B [query][feature] (paired query slots), hi + lo; phi'_K and phi~ rows [feature][token]
    vec8<C> qbh[FB], qbl[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) split_all<8>(qbh[fb], qbl[fb], [&](int j) { return pq[j >> 2][fb][j & 3]; });
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        vec4<C> kh4, kl4, qh4, ql4;
        split_all<4>(kh4, kl4, [&](int i) { return pk[tb][fb][i]; });
        split_all<4>(qh4, ql4, [&](int i) { return pq[tb][fb][i]; });
        const int off = (fb * 16 + c) * FROW + tb * 16 + 4 * g;
        *reinterpret_cast<vec4<C>*>(fth + off) = kh4;
        *reinterpret_cast<vec4<C>*>(qth + off) = qh4;
        if constexpr (NSPL == 2) {
          *reinterpret_cast<vec4<C>*>(ftl + off) = kl4;
          *reinterpret_cast<vec4<C>*>(qtl + off) = ql4;
        }
      }
    // ---- dv partial over this wave's features
    f32x4 dvt[NVB][2];  // dv^T [col][key]
#pragma unroll
    for (int nb = 0; nb < NVB; ++nb) dvt[nb][0] = dvt[nb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    vec8<C> gv[NB];  // g rows as value fragments: [query][col], paired query slots
    value_frags<T, D, DV, NT>(gbase, gv, c, g);
    {
      vec8<C> fah[2], fal[2];  // phi'_K: A [key][feature] / B [feature][key], paired feature slots
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        fah[kb] = tr_read8<C>(fth, FROW, 0, kb * 16, c, g);
        fal[kb] = NSPL == 2 ? tr_read8<C>(ftl, FROW, 0, kb * 16, c, g) : fah[kb];
      }
#pragma unroll
      for (int nb = 0; nb < NVB; ++nb) {
        vec8<C> rth, rtl;
        split_all<8>(rth, rtl, [&](int j) { return Rt[j >> 2][nb][j & 3]; });
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma_split<NSPL>(dvt[nb][kb], rth, rtl, fah[kb], fal[kb]);
      }
      // A^T[q][key] = phi~ (A [query][feature]) x phi'_K (B), over this wave's features
      f32x4 at[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const vec8<C> qah = tr_read8<C>(qth, FROW, 0, qb * 16, c, g);
        const vec8<C> qal = NSPL == 2 ? tr_read8<C>(qtl, FROW, 0, qb * 16, c, g) : qah;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          at[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
          mma_split<NSPL>(at[qb][kb], qah, qal, fah[kb], fal[kb]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        vec8<C> aah, aal;  // B [query][key], paired query slots, q >= key
        split_all<8>(aah, aal, [&](int jj) {
          const int qb = jj >> 2, i = jj & 3;
          const int q = qb * 16 + 4 * g + i, key = kb * 16 + c;
          return q >= key ? at[qb][kb][i] : 0.f;
        });
#pragma unroll
        for (int nb = 0; nb < NVB; ++nb) {
          mma16(dvt[nb][kb], gv[nb], aah);
          if constexpr (NSPL == 2) mma16(dvt[nb][kb], gv[nb], aal);
        }
      }
    }
    // the wave's partial over its own rows (read above by this wave only): [kb][nb][lane] f32x4
    {
      float* part = reinterpret_cast<float*>(&fq[w][0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nb = 0; nb < NVB; ++nb) *reinterpret_cast<f32x4*>(&part[((kb * NVB + nb) * 64 + lane) * 4]) = dvt[nb][kb];
    }
    // ---- the suffix state takes the chunk's queries: Rt[f][col] += phi~^T (A) x g (B)
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NVB; ++nb) {
        mma16(Rt[fb][nb], qbh[fb], gv[nb]);
        if constexpr (NSPL == 2) mma16(Rt[fb][nb], qbl[fb], gv[nb]);
      }
    lds_barrier();  // B1: the dv sums of every wave

    // ---- dv of the chunk: the waves' partials summed, stored
    if (threadIdx.x < 32 * CPR) {
      const int row = threadIdx.x / CPR, c8 = threadIdx.x % CPR;
      const int kb = row >> 4, ck = row & 15, nb = (c8 * 8) >> 4, g0 = ((c8 * 8) & 15) >> 2;
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* base = reinterpret_cast<const float*>(&fq[ww][0]) + ((kb * NVB + nb) * 64 + ck + 16 * g0) * 4;
        a += *reinterpret_cast<const f32x4*>(base);
        b += *reinterpret_cast<const f32x4*>(base + 64);
      }
      const int tok = tok0 + row;
      if (tok < tend) {
        const size_t off = (rowbase + tok) * DV + c8 * 8;
        if (grad_f32) {
          f32x4* o4 = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dv) + off);
          o4[0] = a;
          o4[1] = b;
        } else {
          vec8<T> r;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r[i] = to_t<T>(a[i]);
            r[i + 4] = to_t<T>(b[i]);
          }
          st8<T>(reinterpret_cast<T*>(dv) + off, r);
        }
      }
    }
    // ---- chunk t-1 lands and is converted
    wait_vmcnt<0>();  // on every path (see cbwd_q_kernel)
    if (t > 0) {
      Rg::template convert<P>(ring[buf ^ 1], qn[buf ^ 1], kn[buf ^ 1], nscale, tend - (tok0 - 32));
      if (threadIdx.x < 32) rl[buf ^ 1][threadIdx.x] = pl;
    }
  }
}

// ---------------------------------------------------------------- host side
CausalBackwardPlan plan_causal_backward(const Shape& s, int dtype) {
  CausalBackwardPlan p;
  p.f = plan_causal(s, dtype);
  const size_t ndb = s.d / 16, nfc = (s.m + 31) / 32, nbc = (s.dv / 16 + 1) * 16;
  const size_t omt = (size_t)s.H * ndb * nfc * 512 * elt(dtype);
  size_t off = p.f.total;
  p.off_omlo = off;
  off = align256(off + (size_t)s.H * (s.m / 16) * ((s.d + 31) / 32) * 512 * elt(dtype));
  p.off_omth = off;
  off = align256(off + omt);
  p.off_omtl = off;
  off = align256(off + omt);
  p.off_lg = off;
  off = align256(off + (size_t)s.bh() * s.L * 4);
  p.off_gam = off;
  off = align256(off + (size_t)s.bh() * s.L * 4);
  p.off_trow = off;
  off = align256(off + (size_t)p.f.G * s.m * nbc * 4);
  p.total = off;
  return p;
}

template <typename T, int D, int DV, int M, int KIND>
static hipError_t run_causal_backward(const T* q, const T* k, const T* v, const float* omega, const T* dout,
                                      const Shape& s, float eps, int grad_f32, void* dq, void* dk, void* dv, void* ws,
                                      hipStream_t st) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int DC = (D + 31) / 32;
  constexpr int NWR = RedSplit<M, D>::NW;
  constexpr int NWB = BwdSplit<M>::NW;
  constexpr int NBC = (DV / 16 + 1) * 16;
  const CausalBackwardPlan p = plan_causal_backward(s, sizeof(T) == 4 ? 0 : 1);
  const CausalPlan& f = p.f;
  char* base = static_cast<char*>(ws);
  P* omf = reinterpret_cast<P*>(base + f.off_omf);
  P* omlo = reinterpret_cast<P*>(base + p.off_omlo);
  float* part = reinterpret_cast<float*>(base + f.off_part);
  float* zpart = reinterpret_cast<float*>(base + f.off_zpart);
  float* pmax = reinterpret_cast<float*>(base + f.off_pmax);
  float* cpart = reinterpret_cast<float*>(base + f.off_cpart);
  float* cz = reinterpret_cast<float*>(base + f.off_cz);
  float* cmax = reinterpret_cast<float*>(base + f.off_cmax);
  C* omth = reinterpret_cast<C*>(base + p.off_omth);
  C* omtl = reinterpret_cast<C*>(base + p.off_omtl);
  float* lg = reinterpret_cast<float*>(base + p.off_lg);
  float* gam = reinterpret_cast<float*>(base + p.off_gam);
  float* trow = reinterpret_cast<float*>(base + p.off_trow);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = KIND == kPrf ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)M);
  const float log2_sqrt_m = 0.5f * std::log2((float)M);
  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  const long long nfragT = (long long)s.H * (D / 16) * ((M + 31) / 32) * 64;
  {
    launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st,
        omega, s.H, M, M, D, wscale, omf, 0);
    if constexpr (sizeof(P) == 2)
      launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0,
          st, omega, s.H, M, M, D, wscale, omlo, 1);
    launch("omega_frag", omegaT_pair_kernel<C>, (unsigned)std::min<long long>((nfragT + 255) / 256, 4096), 256, 0, st,
        omega, s.H, M, D, wscale, omth, omtl);
  }
  {
    launch("reduce", kv_reduce_kernel<T, D, DV, M, 4, KIND, true, true>, f.G, 64 * NWR, 0, st, k, v, omf,
        omlo, s.H,
        s.L, f.tpb, f.T_all, f.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, f.seg_len / 32, f.nseg, s.m, DV, DV);
  }
  {
    constexpr int NQ = ((M + 31) / 32) * ((DV / 16) * 512 + 32) / 4;
    launch("scan", scan_kernel<D, DV, M>, (unsigned)(s.bh() * ((NQ + 255) / 256)), 256, f.nseg * sizeof(float), st, part,
        zpart, pmax, f.nseg, KIND, log2_sqrt_m, cpart, cz, cmax, nullptr, nullptr, s.m, DV, DV);
  }
  {
    launch("cbwd_fwd", cbwd_fwd_kernel<T, D, DV, M, KIND>, f.G, 64 * NWB, 0, st, q, k, v, dout, omf, omlo, cpart, cz, cmax,
        s.H, s.L, f.seg_len, f.nseg, nscale, lg, gam, inv_sqrt_m, eps);
  }
  {
    launch("cbwd_q", cbwd_q_kernel<T, D, DV, M, KIND>, f.G, 64 * NWB, 0, st, q, k, v, dout, omf, omlo, omth, omtl, cpart,
        cz, cmax, lg, gam, s.H, s.L, f.seg_len, f.nseg, nscale, grad_f32, dq, inv_sqrt_m, eps);
  }
  {
    launch("cbwd_t", cbwd_t_kernel<T, D, DV, M, KIND>, f.G, 64 * NWB, 0, st, q, dout, omf, omlo, lg, gam, s.H, s.L,
        f.seg_len, f.nseg, trow, inv_sqrt_m, eps);
  }
  {
    const int per = M * NBC, nblk = (per + 255) / 256;
    launch("rscan", cbwd_rscan_kernel, (unsigned)(s.bh() * nblk), 256, 0, st, trow, cmax, f.nseg, per, nblk);
  }
  {
    launch("cbwd_k", cbwd_k_kernel<T, D, DV, M, KIND>, f.G, 64 * NWB, 0, st, q, k, v, dout, omf, omlo, omth, omtl, trow,
        cmax, lg, gam, s.H, s.L, f.seg_len, f.nseg, nscale, sc * sc, grad_f32, dk, inv_sqrt_m, eps);
  }
  {
    launch("cbwd_v", cbwd_v_kernel<T, D, DV, M, KIND>, f.G, 64 * NWB, 0, st, q, k, v, dout, omf, omlo, trow, cmax, lg, s.H,
        s.L, f.seg_len, f.nseg, nscale, grad_f32, dv, inv_sqrt_m, eps);
  }
  return hipGetLastError();
}

template <typename T, int D, int DV, int M>
static hipError_t run_causal_backward_kind(const void* q, const void* k, const void* v, const float* omega,
                                           const void* dout, const Shape& s, int kind, float eps, int grad_f32,
                                           void* dq, void* dk, void* dv, void* ws, hipStream_t st) {
  const T* q_ = static_cast<const T*>(q);
  const T* k_ = static_cast<const T*>(k);
  const T* v_ = static_cast<const T*>(v);
  const T* o_ = static_cast<const T*>(dout);
  if (kind == kPrf)
    return run_causal_backward<T, D, DV, M, kPrf>(q_, k_, v_, omega, o_, s, eps, grad_f32, dq, dk, dv, ws, st);
  if (kind == kRelu)
    return run_causal_backward<T, D, DV, M, kRelu>(q_, k_, v_, omega, o_, s, eps, grad_f32, dq, dk, dv, ws, st);
  return hipErrorInvalidValue;
}

hipError_t launch_causal_backward(const void* q, const void* k, const void* v, const float* omega, const void* dout,
                                  const Shape& s, int dtype, int kind, float eps, int grad_f32, void* dq, void* dk,
                                  void* dv, void* ws, hipStream_t st) {
#define X(D_, DV_, M_)                                                                                           \
  if (s.d == D_ && s.dv == DV_ && s.m == M_) {                                                                   \
    if (dtype == 0) return run_causal_backward_kind<float, D_, DV_, M_>(q, k, v, omega, dout, s, kind, eps,       \
                                                                        grad_f32, dq, dk, dv, ws, st);            \
    return run_causal_backward_kind<bf16, D_, DV_, M_>(q, k, v, omega, dout, s, kind, eps, grad_f32, dq, dk, dv,  \
                                                       ws, st);                                                   \
  }
  FAVOR_BWD_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace favor
