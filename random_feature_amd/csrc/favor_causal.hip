// Causal (unidirectional) FAVOR+ on gfx950 as a segmented, chunked prefix scan.
//
// Performer paper, appendix B.1 (equation 11, Figure 8): row i of the output is
// G^PS_i Q'_i with G^PS_i = sum_{j <= i} K'_j [v_j 1]^T, i.e. prefix sums of S and z
// including the diagonal. Appendix B.3 notes that storing G^PS costs O(mLd) and that
// a sequential aggregation avoids it; the prefix sum itself is parallel (O(log L) depth).
// This file keeps both properties: L is cut into P segments that run in parallel, the
// segments are joined by a scan over their totals, and inside a segment the state is
// carried sequentially from one 32-token chunk to the next, never materialising G^PS.
//   1. omega_frag_kernel, then kv_reduce_kernel (the bidirectional reduction) with one
//      piece per (b*h, segment): the segment totals of S_aug = Phi_K^T [V 1] in MFMA
//      fragment layout, with the waves' key maxima.
//   2. scan_kernel: prefix maxima M*_p over segments and the exclusive prefix sums
//      carry_p = sum_{q<p} total_q * 2^(M_q - M*_p) in the same layout; optionally the
//      final state in canonical (unstabilised) scale.
//   3. sweep_kernel, one workgroup per (b*h, segment), wave w owning a block of features
//      with its rows of the carried state in registers; per chunk of 32 tokens
//        * the key and query projections on MFMA (fp16 for bf16 inputs), keys against
//          the fixed key maximum M*_p of the segment, queries against the per-row bound;
//        * the carried term out^T = S_carry^T Phi_Q^T over the wave's features;
//        * the state update S_carry += Phi_K^T [V 1];
//        * the intra-chunk scores A^T = Phi_K Phi_Q^T over the wave's features (Phi_K
//          transposed through LDS), masked to keys <= queries, and out^T += [V 1]^T A^T;
//        * the waves' partial outputs summed through LDS, divided by the z row, stored.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_segments.hpp"
#include "favor_tiles.hpp"
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

// ---------------------------------------------------------------- sweep
// Workgroup = NW waves on segment sp of (b,h) (piece pc = bh * nseg + sp); wave w owns the
// FB*16 features [w*FB*16, (w+1)*FB*16), the same split as the reduction, so its rows of
// the carried state arrive from the scan in its own fragment layout. The segment's keys
// use the fixed maximum M*_sp of the scan (every key exponent of the segment is below it),
// so the carry never needs rescaling. Per chunk t (ring slot t mod 3):
//   barrier X (chunk t converted by every thread; the partial outputs of chunk t-1 written)
//   the output of chunk t-1: the NW partials summed, divided by the z row, stored
//   phase A (all in registers but the Phi_K transpose):
//     K projection  A = K rows, B = Omega'         -> [token][feature] (start -(n'_k + M*))
//     Q projection  A = Omega', B = Q rows         -> [feature][token] (start -b_q)
//     features      Phi_K as A operand (paired token slots), Phi_Q as B operand (paired
//                   feature slots), straight from the accumulators
//     carried term  o^T[col][q]  = S^T (A, the state rows as they stand) x Phi_Q^T
//     update        S_aug       += Phi_K^T (A) x [V 1] (B, transposing reads of V)
//     scores        A^T[key][q]  = Phi_K (A, through LDS, per 32-feature chunk) x Phi_Q^T
//     intra term    o^T         += [V 1]^T (A: the value fragments) x masked A^T (B)
//   chunk t+1 lands and is converted in place by the threads that copied it
//   barrier Y; the wave's partial o^T goes to LDS; chunk t+2 is copied into slot (t+2) mod 3
// Shapes as kv_reduce_kernel (GEN): m_valid <= M features (the query features past it are zero, which
// keeps the rest of those features out of every output), a column group of vcols <= DV columns of V
// and out whose rows are ld elements apart.
// CT: the type of the stored carries (see scan_kernel).
template <typename T, int D, int DV, int M, int KIND, bool GEN, typename CT>
__global__ void __launch_bounds__(64 * (RedSplit<M, D>::NW), (RedSplit<M, D>::WPE))
sweep_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
             const typename Ops<T>::P* __restrict__ omf, const CT* __restrict__ cpart,
             const CT* __restrict__ cz, const float* __restrict__ cmax, int H, int L, int seg_len, int nseg,
             float eps, float inv_sqrt_m, float nscale, int out_f32, void* __restrict__ out, int m_valid_, int ld_,
             int vcols_) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = RedSplit<M, D>::NW, FB = RedSplit<M, D>::FB;
  const int m_valid = GEN ? m_valid_ : M, ld = GEN ? ld_ : DV, vcols = GEN ? vcols_ : DV;
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;  // value-column blocks + the ones column
  constexpr int NVB = DV / 16;
  constexpr int NFC = (M + 31) / 32;
  constexpr int NFCW = (FB + 1) / 2;  // 32-feature chunks of a wave
  constexpr int R = 3;
  constexpr int PROW = 36;              // row stride (elements) of the Phi_K transpose buffer
  constexpr int XO = 2 * NVB * 256 + 32;  // floats of one wave's partial output
  static_assert(FB % 2 == 0 || NW == 1, "an odd block count per wave only with a single wave");
  using Rg = SweepRing<T, D, DV, NT>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[R][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) float xo[NW][XO];
  __shared__ __attribute__((aligned(16))) C phk[NW][32 * PROW];
  __shared__ __attribute__((aligned(16))) float kn[R][32];
  __shared__ __attribute__((aligned(16))) float qn[R][32];
  __shared__ __attribute__((aligned(16))) float qmx[NW][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int pc = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = pc / nseg, sp = pc % nseg, h = bh % H;
  const int t0 = sp * seg_len, tend = min(t0 + seg_len, L);
  const int n = (tend - t0 + 31) / 32;
  const size_t rowbase = (size_t)bh * L;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  // chunks 0 and 1 in flight
  Rg::issue(Q, K, V, L, rowbase, t0, ring0, nullptr, ld, vcols);
  if (n > 1) Rg::issue(Q, K, V, L, rowbase, t0 + 32, ring0 + Rg::SLOT, nullptr, ld, vcols);

  vec8<P> om[FB][DC];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      om[fb][dc] = ld8<P>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);
  // the wave's rows of the carry (fragment layout of the reduction's partials)
  f32x4 sacc[FB][NB];
#pragma unroll
  for (int p = 0; p < NFCW; ++p) {
    const int fc = (w * FB) / 2 + p;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
      if (nb < NB - 1)
        ld8_f32(cpart + ((((size_t)pc * NFC + fc) * NVB + nb) * 64 + lane) * 8, lo, hi);
      else if (c == 0)
        ld8_f32(cz + (((size_t)pc * NFC + fc) * 4 + g) * 8, lo, hi);
      sacc[2 * p][nb] = lo;
      if (2 * p + 1 < FB) sacc[2 * p + 1][nb] = hi;
    }
  }
  // the keys' fixed maximum of the segment: of their exponents (exponential map) or of their norms n'
  // (trigonometric map, whose keys carry the scale 2^(n'_k))
  const float mk = (KIND != kRelu) ? cmax[pc] : 0.f;
  float omax = 0.f;
  if constexpr (KIND == kPrf) omax = omega_norm_max<NW>(om, &qmx[0][0], 32);
  wait_vmcnt<0>();
  Rg::template convert<P>(ring[0], qn[0], kn[0], nscale, tend - t0);

  // the summed partial outputs of chunk tc: divided by the z row and stored
  auto store_chunk = [&](int tc) {
    constexpr int C8 = DV / 8;
    const int tok0 = t0 + 32 * tc;
    // item e: query row (e >> 4 ... ) taken 16 rows at a time, so the 16 threads of a quarter-wave read one column
    // chunk of 16 rows: 16 different 4-bank groups of the partial outputs (row-major items put a row's 8 chunks,
    // all in the same banks, on consecutive threads)
    for (int e = threadIdx.x; e < 32 * C8; e += NT) {
      const int cq = e & 15, rest = e >> 4;
      const int tb = rest / C8, c8 = rest % C8;
      const int qrow = tb * 16 + cq;
      const int tok = tok0 + qrow;
      if (tok >= tend || c8 * 8 >= vcols) continue;
      const int cb = (c8 * 8) >> 4, g0 = ((c8 * 8) & 15) >> 2;
      const int xoff = ((tb * NVB + cb) * 64 + cq + 16 * g0) * 4, doff = 2 * NVB * 256 + tb * 16 + cq;
      f32x4 lo = *reinterpret_cast<const f32x4*>(&xo[0][xoff]);
      f32x4 hi = *reinterpret_cast<const f32x4*>(&xo[0][xoff + 64]);
      float den = xo[0][doff];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        lo += *reinterpret_cast<const f32x4*>(&xo[ww][xoff]);
        hi += *reinterpret_cast<const f32x4*>(&xo[ww][xoff + 64]);
        den += xo[ww][doff];
      }
      const float rden = __builtin_amdgcn_rcpf(den);  // hardware reciprocal (1 ulp)
      const size_t off = (rowbase + tok) * ld + c8 * 8;
      if (out_f32) {
        f32x4* o4 = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off);
        o4[0] = lo * rden;
        o4[1] = hi * rden;
      } else {
        vec8<T> r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r[i] = to_t<T>(lo[i] * rden);
          r[i + 4] = to_t<T>(hi[i] * rden);
        }
        st8<T>(reinterpret_cast<T*>(out) + off, r);
      }
    }
  };

  int s_cur = 0;
  for (int t = 0; t < n; ++t) {
    const int s_nx = s_cur + 1 == R ? 0 : s_cur + 1;
    const int s_is = s_nx + 1 == R ? 0 : s_nx + 1;
    lds_barrier();  // X
    if (t > 0) store_chunk(t - 1);

    const unsigned char* sl = ring[s_cur];
    const int tok0 = t0 + 32 * t;
    // ---- projections
    f32x4 pk[2][FB], pq[2][FB];
    bool exact = false;
    float tw[2][4];  // trigonometric map: the keys' scale 2^(n'_k - M*) (0 past the segment)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 kbias = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KIND == kPrf) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[s_cur][tb * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) kbias[i] = -(n4[i] + mk);
      } else if constexpr (KIND == kTrig) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[s_cur][tb * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) tw[tb][i] = n4[i] < INFINITY ? fast_exp2(n4[i] - mk) : 0.f;
      }
      const float b = (KIND == kPrf) ? qn[s_cur][tb * 16 + c] * omax : 0.f;
      if constexpr (KIND == kPrf) exact |= b > kQueryBoundLimit;
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
          mma16(pk[tb][fb], kf[dc], om[fb][dc]);
          mma16(pq[tb][fb], om[fb][dc], qf[dc]);
        }
      }
    }
    if constexpr (KIND == kPrf) {
      if (__builtin_amdgcn_ballot_w64(exact) != 0) {  // the same in every wave
        // rare: shift every query row by its exact maximum (over the m_valid real features), taken across
        // the waves
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float mx = -INFINITY;
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((w * FB + fb) * 16 + 4 * g + i < m_valid) mx = fmaxf(mx, pq[tb][fb][i]);
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
        }
      }
    }
    // ---- feature maps
    vec8<C> af[FB];        // Phi_K^T: A operand [feature][token], paired token slots
    vec8<C> bq[2][NFCW];   // Phi_Q^T: B operand [feature][query], paired feature slots
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = pk[j >> 2][fb][j & 3];
        float f;
        if constexpr (KIND == kPrf) {
          f = fast_exp2(a);  // rows past the segment carry an infinite norm: exp2(-inf) = 0
        } else if constexpr (KIND == kTrig) {
          f = trig_feature(a, (w * FB + fb) * 16 + c, M) * tw[j >> 2][j & 3];
        } else {
          const bool ok = tok0 + 16 * (j >> 2) + 4 * g + (j & 3) < tend;
          f = ok ? fmaxf(a, 0.f) * inv_sqrt_m + eps : 0.f;
        }
        af[fb][j] = to_t<C>(f);
      }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int fb = 2 * fcw + (j >> 2);
          float f = 0.f;
          // features past m_valid: zero query features, so the state rows and scores they would feed (the
          // keys' features there are not masked) never reach an output
          if (fb < FB && (!GEN || (w * FB + fb) * 16 + 4 * g + (j & 3) < m_valid)) {  // exact shapes: all valid
            const float a = pq[tb][fb][j & 3];
            if constexpr (KIND == kPrf)
              f = fast_exp2(a);
            else if constexpr (KIND == kTrig)
              f = trig_feature(a, (w * FB + fb) * 16 + 4 * g + (j & 3), M);  // the query's scale cancels
            else
              f = fmaxf(a, 0.f) * inv_sqrt_m + eps;
          }
          bq[tb][fcw][j] = to_t<C>(f);
        }
    // ---- carried term, before the state takes this chunk
    f32x4 o[NB][2];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      o[cb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      o[cb][1] = o[cb][0];
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw) {
        vec8<C> sa;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sa[j] = to_t<C>(sacc[2 * fcw][cb][j]);
          sa[j + 4] = (2 * fcw + 1 < FB) ? to_t<C>(sacc[2 * fcw + 1][cb][j]) : to_t<C>(0.f);
        }
        mma16(o[cb][0], sa, bq[0][fcw]);
        mma16(o[cb][1], sa, bq[1][fcw]);
      }
    }
    // ---- state update
    vec8<C> vf[NB];
    value_frags<T, D, DV, NT>(sl + Rg::XC * 16, vf, c, g, vcols);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma16(sacc[fb][nb], af[fb], vf[nb]);
    // ---- intra-chunk scores A^T[key][query] over this wave's features
    f32x4 sc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb][0] = sc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    C* ph = &phk[w][0];
#pragma unroll
    for (int fcw = 0; fcw < NFCW; ++fcw) {
      // Phi_K rows (features) of this 32-feature chunk, [feature][token] (wave-private: the
      // wave's own LDS operations complete in order)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int fb = 2 * fcw + hh;
        vec4<C> lo4, hi4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo4[i] = fb < FB ? af[fb][i] : to_t<C>(0.f);
          hi4[i] = fb < FB ? af[fb][i + 4] : to_t<C>(0.f);
        }
        *reinterpret_cast<vec4<C>*>(ph + (16 * hh + c) * PROW + 4 * g) = lo4;
        *reinterpret_cast<vec4<C>*>(ph + (16 * hh + c) * PROW + 16 + 4 * g) = hi4;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        vec8<C> ka;  // A operand [key][feature]: Phi_K of key kb*16 + c, paired feature slots
        if constexpr (sizeof(C) == 2) {
          const bf16x4 lo = lds_read_tr4(reinterpret_cast<const bf16*>(ph + (4 * g + (c >> 2)) * PROW + kb * 16 + 4 * (c & 3)));
          const bf16x4 hi = lds_read_tr4(reinterpret_cast<const bf16*>(ph + (16 + 4 * g + (c >> 2)) * PROW + kb * 16 + 4 * (c & 3)));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ka[i] = lo[i];
            ka[i + 4] = hi[i];
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) ka[jj] = ph[(16 * (jj >> 2) + 4 * g + (jj & 3)) * PROW + kb * 16 + c];
        }
        mma16(sc[kb][0], ka, bq[0][fcw]);
        mma16(sc[kb][1], ka, bq[1][fcw]);
      }
    }
    // ---- masked scores as B [key][query] (paired key slots) and the intra term
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<C> sb;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int kb = jj >> 2, i = jj & 3;
        const int key = kb * 16 + 4 * g + i, qry = tb * 16 + c;
        sb[jj] = to_t<C>(key <= qry ? sc[kb][tb][i] : 0.f);
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) mma16(o[cb][tb], vf[cb], sb);
    }

    // ---- chunk t+1 lands and is converted
    if (t + 1 < n) {
      wait_vmcnt<0>();  // its copies, and the stores of chunk t-1
      Rg::template convert<P>(ring[s_nx], qn[s_nx], kn[s_nx], nscale, tend - tok0 - 32);
    }
    lds_barrier();  // Y: slot s_is and the partial outputs of chunk t-1 are no longer read
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int cb = 0; cb < NVB; ++cb)
        *reinterpret_cast<f32x4*>(&xo[w][((tb * NVB + cb) * 64 + lane) * 4]) = o[cb][tb];
      if (g == 0) xo[w][2 * NVB * 256 + tb * 16 + c] = o[NB - 1][tb][0];
    }
    if (t + 2 < n) Rg::issue(Q, K, V, L, rowbase, tok0 + 64, ring0 + s_is * Rg::SLOT, nullptr, ld, vcols);
    s_cur = s_nx;
  }
  lds_barrier();
  store_chunk(n - 1);
}

// ---------------------------------------------------------------- host side
template <typename X> struct TypeTag { using type = X; };

static void segmenting(const Shape& s, int& nseg, int& seg_len) {
  // enough segments for ~512 workgroups, but at least 256 tokens each
  const long long bh = s.bh();
  const int max_seg = std::max(1, (s.L + 255) / 256);
  const int want = (int)std::max(1LL, (512 + bh - 1) / bh);
  nseg = std::min(max_seg, want);
  seg_len = (s.L + nseg - 1) / nseg;
  seg_len = (seg_len + 31) / 32 * 32;
  nseg = (s.L + seg_len - 1) / seg_len;
}

CausalPlan plan_causal(const Shape& s, int dtype) {
  CausalPlan p;
  segmenting(s, p.nseg, p.seg_len);
  p.tpb = (s.L + 31) / 32;
  p.T_all = s.bh() * p.tpb;
  p.G = (int)(s.bh() * p.nseg);
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);  // sizes of the compiled kernels (one column group)
  p.nw_reduce = reduce_waves(ks.mk, s.d);
  const int dc = (s.d + 31) / 32;
  const size_t nfc = (ks.mk + 31) / 32, G = (size_t)p.G;
  size_t off = 0;
  p.off_omf = off;
  off = align256(off + (size_t)s.H * (ks.mk / 16) * dc * 512 * elt(dtype));
  p.off_part = off;
  off = align256(off + G * nfc * (ks.dvk / 16) * 512 * 4);
  p.off_zpart = off;
  off = align256(off + G * nfc * 32 * 4);
  p.off_pmax = off;
  off = align256(off + G * p.nw_reduce * 4);
  p.off_cpart = off;
  off = align256(off + G * nfc * (ks.dvk / 16) * 512 * 4);
  p.off_cz = off;
  off = align256(off + G * nfc * 32 * 4);
  p.off_cmax = off;
  off = align256(off + G * 4);
  p.total = off;
  return p;
}

// One call on the compiled (D, DV, M): the Omega' fragments once, then reduce, scan and sweep per column
// group of DV columns of v and out (one group when dv = DV). GEN: the general kernels.
template <typename T, int D, int DV, int M, bool GEN>
static hipError_t run_causal(const T* q, const T* k, const T* v, const float* omega, const Shape& s, int kind,
                             float eps, int out_f32, void* out, float* S_final, float* z_final, void* ws,
                             hipStream_t st, const void* prep) {
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  constexpr int NWR = RedSplit<M, D>::NW;
  const CausalPlan p = plan_causal(s, sizeof(T) == 4 ? 0 : 1);
  char* base = static_cast<char*>(ws);
  P* omf = prep ? static_cast<P*>(const_cast<void*>(prep)) : reinterpret_cast<P*>(base + p.off_omf);
  float* pmax = reinterpret_cast<float*>(base + p.off_pmax);
  // carries in the contraction type: bf16 for 16-bit inputs (the sweep rounds its state to bf16 for the carried
  // term in any case), fp32 for fp32 inputs
  using CT = typename Ops<T>::C;
  CT* cpart = reinterpret_cast<CT*>(base + p.off_cpart);
  CT* cz = reinterpret_cast<CT*>(base + p.off_cz);
  float* cmax = reinterpret_cast<float*>(base + p.off_cmax);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = omega_scale(kind, sc);
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)s.m);
  const float log2_sqrt_m = 0.5f * std::log2((float)s.m);

  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  if (!prep)
    launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st,
        omega, s.H, s.m, M, D, wscale, omf, 0);
  const int seg_tiles = p.seg_len / 32;
  for (int c0 = 0; c0 < s.dv; c0 += DV) {
    const int vcols = std::min(DV, s.dv - c0);
    const T* vg = v + c0;
    void* og = out_f32 ? static_cast<void*>(static_cast<float*>(out) + c0) : static_cast<void*>(static_cast<T*>(out) + c0);
    // segment sums and their scan, with the partials stored as PT
    auto reduce_scan = [&](auto tag) {
      using PT = typename decltype(tag)::type;
      PT* part = reinterpret_cast<PT*>(base + p.off_part);
      PT* zpart = reinterpret_cast<PT*>(base + p.off_zpart);
      if (kind == kPrf)
        launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, kPrf, false, false, GEN, PT>, p.G, 64 * NWR, 0, st, k, vg,
            omf, nullptr, s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, seg_tiles, p.nseg,
            s.m, s.dv, vcols);
      else if (!GEN && kind == kTrig)  // the trigonometric map on the exact shapes only
        launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, GEN ? kPrf : kTrig, false, false, GEN, PT>, p.G,
            64 * NWR, 0, st, k, vg, omf, nullptr, s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart,
            pmax, seg_tiles, p.nseg, s.m, s.dv, vcols);
      else
        launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, kRelu, false, false, GEN, PT>, p.G, 64 * NWR, 0, st, k,
            vg, omf, nullptr, s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, seg_tiles,
            p.nseg, s.m, s.dv, vcols);
      constexpr int NQ = ((M + 31) / 32) * ((DV / 16) * 512 + 32) / 4;
      launch("scan", scan_kernel<D, DV, M, CT, PT>, (unsigned)(s.bh() * ((NQ + 255) / 256)), 256,
          p.nseg * sizeof(float), st, part, zpart, pmax, p.nseg, kind, log2_sqrt_m, cpart, cz, cmax,
          S_final ? S_final + c0 : nullptr, c0 == 0 ? z_final : nullptr, s.m, s.dv, vcols);
    };
    // partials in bf16 for 16-bit inputs when no final state is asked for (the carries they feed are bf16), else
    // fp32 (the final state is summed from them)
    if constexpr (sizeof(T) == 2) {
      if (!S_final && !z_final)
        reduce_scan(TypeTag<bf16>{});
      else
        reduce_scan(TypeTag<float>{});
    } else {
      reduce_scan(TypeTag<float>{});
    }
    if (kind == kPrf)
      launch("sweep", sweep_kernel<T, D, DV, M, kPrf, GEN, CT>, p.G, 64 * NWR, 0, st, q, k, vg, omf, cpart, cz, cmax, s.H,
          s.L, p.seg_len, p.nseg, eps, inv_sqrt_m, nscale, out_f32, og, s.m, s.dv, vcols);
    else if (!GEN && kind == kTrig)
      launch("sweep", sweep_kernel<T, D, DV, M, GEN ? kPrf : kTrig, GEN, CT>, p.G, 64 * NWR, 0, st, q, k, vg, omf, cpart,
          cz, cmax, s.H, s.L, p.seg_len, p.nseg, eps, inv_sqrt_m, nscale, out_f32, og, s.m, s.dv, vcols);
    else
      launch("sweep", sweep_kernel<T, D, DV, M, kRelu, GEN, CT>, p.G, 64 * NWR, 0, st, q, k, vg, omf, cpart, cz, cmax, s.H,
          s.L, p.seg_len, p.nseg, eps, inv_sqrt_m, nscale, out_f32, og, s.m, s.dv, vcols);
  }
  return hipGetLastError();
}

hipError_t launch_causal(const void* q, const void* k, const void* v, const float* omega, const Shape& s,
                         int dtype, int kind, float eps, int out_f32, void* out, float* S_final, float* z_final,
                         void* ws, hipStream_t st, const void* prep) {
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);
  if (!ks.ok) return hipErrorInvalidValue;
#define X(D_, DV_, M_, GEN_)                                                                                    \
  if (ks.exact == !GEN_ && ks.dk == D_ && ks.dvk == DV_ && ks.mk == M_) {                                       \
    if (dtype == 0) {                                                                                           \
      if constexpr (fp32_built(GEN_, D_, M_))                                                                   \
        return run_causal<float, D_, DV_, M_, GEN_>(static_cast<const float*>(q), static_cast<const float*>(k), \
                                                    static_cast<const float*>(v), omega, s, kind, eps, out_f32,  \
                                                    out, S_final, z_final, ws, st, prep);                       \
      return hipErrorInvalidValue;                                                                              \
    }                                                                                                           \
    return run_causal<bf16, D_, DV_, M_, GEN_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),        \
                                               static_cast<const bf16*>(v), omega, s, kind, eps, out_f32, out,  \
                                               S_final, z_final, ws, st, prep);                                 \
  }
#define XE(D_, DV_, M_) X(D_, DV_, M_, false)
#define XG(D_, DV_, M_) X(D_, DV_, M_, true)
  FAVOR_SHAPES(XE)
  FAVOR_GENERAL_SHAPES(XG)
#undef XG
#undef XE
#undef X
  return hipErrorInvalidValue;
}

}  // namespace favor
