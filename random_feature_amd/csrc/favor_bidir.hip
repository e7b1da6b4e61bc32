// Bidirectional FAVOR+ on gfx950 and the standalone feature map.
//
// Performer paper, equation 4 and Algorithm 1: with C = [V 1],
//   Buf1 = Phi_K^T C  (S and z together),  Buf2 = Phi_Q Buf1,  out = Buf2[:, :dv] / Buf2[:, dv].
// Kernels, in launch order:
//   omega_frag_kernel   Omega (fp32, [H,m,d]) -> scaled MFMA fragments in the workspace
//                       (scale d^-1/4, times log2 e for the exponential map so that the
//                       hardware exp2 needs no extra multiply); fp16 for bf16 inputs
//   kv_reduce_kernel    persistent over pieces of the flattened token-tile space: per tile,
//                       Phi_K on MFMA with the key bias folded into the accumulator start
//                       value, and S_aug += Phi_K^T [V 1] on MFMA; one partial per
//                       (piece, b*h) with the wave's running key maximum
//   combine_kernel      per (b*h, 32-feature chunk): rescale the partials to one maximum,
//                       sum, and lay S_aug out as MFMA fragments
//   q_output_kernel     persistent over pieces: per 32-token tile, Phi_Q on MFMA with the
//                       row maximum taken across the waves, the contraction with S_aug over
//                       each wave's features, the partial outputs summed through LDS, the
//                       division by the z row and the store
// Every stabiliser is a constant per query row or per (b,h) for keys, so it cancels
// in the ratio; none is per feature.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_tiles.hpp"
#include "favor_timing.hpp"

#include "../../include/favor.h"

#include <algorithm>
#include <cmath>
#include <mutex>

namespace favor {

// ---------------------------------------------------------------- combine
// One workgroup per (b*h, 32-feature chunk), one thread per (value block, lane): the
// partials of the pieces of that (b,h), already in fragment layout, scaled by
// 2^(M_piece,wave - M_max) and summed, give the A fragments of S_aug^T:
// sfr[bh][fc][nb][lane][j] = S_aug[fc*32 + 16(j>>2) + 4g + (j&3)][nb*16 + c]; in the last
// block only row c == 0 (the z column) is nonzero.
// PT: the type of the stored partials (fp32; bf16 for 16-bit inputs, whose S_aug fragments are bf16 as well).
template <typename C, int D, int DV, int M, typename PT>
__global__ void __launch_bounds__(1024)
combine_kernel(const PT* __restrict__ part, const PT* __restrict__ zpart, const float* __restrict__ pmax,
               int tpb, long long T_all, int G, int kind, C* __restrict__ sfr, float* __restrict__ gmx) {
  constexpr int NW = RedSplit<M, D>::NW, FB = RedSplit<M, D>::FB;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (M + 31) / 32;
  const int bh = blockIdx.x / NFC, fc = blockIdx.x % NFC;
  const long long i_lo = piece_of((long long)bh * tpb, T_all, G);
  const long long i_hi = piece_of((long long)(bh + 1) * tpb - 1, T_all, G);
  const int np = (int)(i_hi - i_lo + 1);
  const int wv = (fc * 32) / (FB * 16);  // the reducing wave that owned this chunk
  float gmax = -INFINITY;
  const bool scaled = kind != kRelu;  // ReLU features carry no key stabiliser
  if (scaled) {
    // the np*NW maxima of this (b,h) are contiguous: one load per lane, then a wave maximum
    const float* pm = pmax + (size_t)(i_lo + bh) * NW;
    for (int k = threadIdx.x & 63; k < np * NW; k += 64) gmax = fmaxf(gmax, pm[k]);
    gmax = wave_max(gmax);
  }
  if (fc == 0 && threadIdx.x == 0) gmx[bh] = scaled ? gmax : 0.f;  // the keys' common maximum
  for (int e = threadIdx.x; e < NB * 64; e += blockDim.x) {
    const int nb = e >> 6, lane = e & 63;
    const int c = lane & 15, g = lane >> 4;
    f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
    if (nb < NB - 1 || c == 0) {
      // KP partials at a time, all loads issued before the sums (a slot past the last piece
      // is read as the last one and weighted 0)
      constexpr int KP = 8;
      for (int k0 = 0; k0 < np; k0 += KP) {
        f32x4 pl[KP], ph[KP];
        float sc[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) {
          const int k = k0 + j < np ? k0 + j : np - 1;
          const size_t slot = (size_t)(i_lo + k) + bh;
          sc[j] = k0 + j < np ? (scaled ? fast_exp2(pmax[slot * NW + wv] - gmax) : 1.f) : 0.f;
          const PT* src = (nb < NB - 1) ? part + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8
                                        : zpart + ((slot * NFC + fc) * 4 + g) * 8;
          ld8_f32(src, pl[j], ph[j]);
        }
#pragma unroll
        for (int j = 0; j < KP; ++j) {
          lo += pl[j] * sc[j];
          hi += ph[j] * sc[j];
        }
      }
    }
    vec8<C> o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = to_t<C>(lo[i]);
      o[i + 4] = to_t<C>(hi[i]);
    }
    st8<C>(sfr + (((size_t)bh * NFC + fc) * NB + nb) * 512 + lane * 8, o);
  }
}

// ---------------------------------------------------------------- query side

// Workgroup = NW waves over one piece of the flattened tile space. Per 32-token tile:
//   phase 1 (wave w, its FB*16 features, Omega' fragments in registers)
//     projection  A = Omega' (rows = features), B = Q^T (linear d slots) -> [feature][token];
//                 the accumulators start at -b_t, b_t = omax |q_t| >= max_r a'_r (omax the
//                 largest row norm of the rounded Omega' of the head), so the output is
//                 already a non-positive exponent (the |q|^2 term of the map and any
//                 constant per row cancel in the ratio). If some row of the tile has
//                 b_t > kQueryBoundLimit, the tile takes the exact row maximum across the
//                 waves instead (one more barrier).
//     feature map Phi = exp2(.) (ReLU: max(a,0)/sqrt(m) + eps; trigonometric: the sine or
//                 cosine of the projection, whose scale exp(|x|^2/2)/sqrt(m) cancels in the
//                 ratio); the accumulator pairs are
//                 B operands of the contraction as they stand (paired feature slots) and go
//                 to LDS; the wave's share of the denominator z^T Phi^T goes with them
//   every thread then lands, converts and norms its own chunk of tile t+1 and copies its
//   chunk of tile t+2 into the two-slot ring (all its memory traffic, stores included, has
//   settled at that point, so one full wait covers it)
//   barrier
//   phase 2 (wave w: a token half and value-column blocks, or both halves and fewer blocks)
//     contraction out^T block = S^T block (A, registers) x Phi^T (B, all features from LDS)
//     division by the summed denominators and the store
// Shapes as kv_reduce_kernel (GEN): m_valid <= M features (those past it are masked: their rows of
// S_aug are zero, and their exponents are -inf so that the exact-maximum fallback ignores them);
// out rows are ldo elements apart and the call writes its vcols <= DV columns of them.
template <typename T, int D, int DV, int M, int KIND, bool GEN>
__global__ void __launch_bounds__(64 * (FeatSplit<M, D>::NW), (kOutThree<T, M, D> ? 3 : 2))
q_output_kernel(const T* __restrict__ Q, const typename Ops<T>::P* __restrict__ omf,
                const typename Ops<T>::C* __restrict__ sfr, int H, int L, int tpb, long long T_all, int G,
                float eps, float inv_sqrt_m, int out_f32, int renorm, const float* __restrict__ gmx, float nscale,
                float log2_m, void* __restrict__ out, int m_valid_, int ldo_, int vcols_) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M, D>::NW, FB = FeatSplit<M, D>::FB;
  const int m_valid = GEN ? m_valid_ : M, ldo = GEN ? ldo_ : DV, vcols = GEN ? vcols_ : DV;
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;           // blocks of S_aug^T in sfr: values, then z
  constexpr int NVB = DV / 16;              // value-column blocks
  // phase 2 split: with TBS wave w takes token half w & 1 and value blocks (w >> 1) + j*NW/2
  // (half the LDS reads of the features, twice the S fragments); else both halves and
  // blocks w + j*NW (three workgroups per CU: the registers for a third wave on every SIMD)
  constexpr int SF_REGS = sizeof(typename Ops<T>::C) == 2 ? 4 : 8;
  constexpr int NWH = NW / 2 > 0 ? NW / 2 : 1;
  constexpr bool TBS = !kOutThree<T, M, D> && NW >= 2 && ((NVB + NWH - 1) / NWH) * ((M + 31) / 32) * SF_REGS <= 64;
  constexpr int NW2 = TBS ? NWH : NW;
  constexpr int NCB = (NVB + NW2 - 1) / NW2;  // value-column blocks per wave
  constexpr int NTB = TBS ? 1 : 2;             // token halves per wave in phase 2
  constexpr int NFCW = (FB + 1) / 2;        // 32-feature chunks a wave fills (half of one when FB = 1)
  constexpr int NFC = (M + 31) / 32;
  constexpr int KROW = D + 8;
  using Rg = Ring<T, D, DV, NT, false>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P qs[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float qb[2][32];
  __shared__ __attribute__((aligned(16))) C phib[2][NFC][2][64 * 8];
  __shared__ __attribute__((aligned(16))) float dpart[2][2][16][NW];
  __shared__ __attribute__((aligned(16))) float qmx[NW][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  const long long t_beg = piece_start(pc, T_all, G), t_end = piece_start(pc + 1, T_all, G);
  if (t_beg >= t_end) return;
  const int n_tiles = (int)(t_end - t_beg);
  const int fc0 = (w * FB) / 2;
  const int cb0 = TBS ? (w >> 1) : w, tb0 = TBS ? (w & 1) : 0;

  const uint32_t ring0 = lds_addr(&ring[0][0]);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb);
  // prologue: tiles 0 and 1 in flight, tile 0 converted
  Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), true, ring0);
  ahead.next();
  Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), n_tiles > 1, ring0 + Rg::SLOT);
  if (n_tiles > 1) ahead.next();
  wait_vmcnt<Rg::CPT>();
  Rg::template convert<P, KROW, kNormAbs>(ring[0], qs[0], qb[0], kQueryMargin, L);
  lds_barrier();

  vec8<P> om[FB][DC];
  vec8<C> zf[NFCW];
  vec8<C> sf[NCB][NFC];
  float omax = 0.f;
  float gm = 0.f;  // key stabiliser of the current (b,h) (renormalisation off)
  int cur_bh = -1;

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int bh = cur.bh, tok0 = cur.tok0();
    if (bh != cur_bh) {
      const int h = bh % H;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          om[fb][dc] = ld8<P>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw)
        zf[fcw] = ld8<C>(sfr + ((((size_t)bh * NFC + fc0 + fcw) * NB + (NB - 1)) * 64 + lane) * 8);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int nb = cb0 + cb * NW2;
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc)
          sf[cb][fc] = nb < NVB ? ld8<C>(sfr + ((((size_t)bh * NFC + fc) * NB + nb) * 64 + lane) * 8) : zero8<C>();
      }
      cur_bh = bh;
      if constexpr (KIND == kPrf) gm = renorm ? 0.f : gmx[bh];
      if constexpr (KIND == kPrf) omax = omega_norm_max<NW>(om, &qmx[0][0], 32);
      // the fragments have landed: no wait for them is left to the first uses in the tile loop,
      // where it would also drain the copies and stores in flight on every tile
      wait_vmcnt<0>();
    }

    // ---- phase 1: this wave's features of the tile
    // The feature map, and the conversion of the next tile after it, are long runs of dependent
    // vector work; raised issue priority lets this wave's VALU stream go first while the other
    // wave of the SIMD fills the gaps with its MFMAs (dropped again at the barrier before the
    // contraction).
    __builtin_amdgcn_s_setprio(1);
    f32x4 bias[2];
    float shf[2];  // the exponent shift of this lane's query row of each token half
    bool exact = false;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float b = (KIND == kPrf) ? qb[buf][tb * 16 + c] * omax : 0.f;
      bias[tb] = f32x4{-b, -b, -b, -b};
      shf[tb] = b;
      if constexpr (KIND == kPrf) exact |= b > kQueryBoundLimit;
    }
    if constexpr (KIND == kPrf) exact = __builtin_amdgcn_ballot_w64(exact) != 0;  // same in every wave
    f32x4 pacc[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<P> qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        qf[dc] = (col < D) ? ld8<P>(&qs[buf][(tb * 16 + c) * KROW + col]) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pacc[tb][fb] = bias[tb];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(pacc[tb][fb], om[fb][dc], qf[dc]);
      }
    }
    if constexpr (KIND == kPrf) {
      if (m_valid < M) {  // features past m_valid: exponent -inf
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((w * FB + fb) * 16 + 4 * g + i >= m_valid) pacc[tb][fb][i] = -INFINITY;
      }
      if (exact) {
        // rare: shift every row by its exact maximum, taken across the waves
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          float mx = -INFINITY;
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pacc[tb][fb][i]);
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
          for (int fb = 0; fb < FB; ++fb) pacc[tb][fb] -= mx;
          shf[tb] += mx;
        }
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = fast_exp2(pacc[tb][fb][i]);
    } else if constexpr (KIND == kTrig) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = trig_feature(pacc[tb][fb][i], (w * FB + fb) * 16 + 4 * g + i, M);
    } else {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = fmaxf(pacc[tb][fb][i], 0.f) * inv_sqrt_m + eps;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw) {
        vec8<C> bf;
        if constexpr (FB % 2 == 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) bf[j] = to_t<C>(pacc[tb][2 * fcw + (j >> 2)][j & 3]);
          *reinterpret_cast<vec8<C>*>(&phib[buf][fc0 + fcw][tb][lane * 8]) = bf;
        } else {
          // one 16-feature block per wave: it fills half (w & 1) of its 32-feature chunk
          const int half = w & 1;
          vec4<C> hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = to_t<C>(pacc[tb][0][i]);
#pragma unroll
          for (int j = 0; j < 8; ++j) bf[j] = (j >> 2) == half ? hv[j & 3] : to_t<C>(0.f);
          if constexpr (M % 32 != 0)
            *reinterpret_cast<vec8<C>*>(&phib[buf][fc0][tb][lane * 8]) = bf;  // no wave owns the other half
          else
            *reinterpret_cast<vec4<C>*>(&phib[buf][fc0][tb][lane * 8 + half * 4]) = hv;
        }
        mma16(dacc, zf[fcw], bf);
      }
      if (g == 0) dpart[buf][tb][c][w] = dacc[0];
    }

    // land, convert and norm this thread's chunk of tile t+1; copy its chunk of tile t+2
    wait_vmcnt<0>();
    Rg::template convert<P, KROW, kNormAbs>(ring[buf ^ 1], qs[buf ^ 1], qb[buf ^ 1], kQueryMargin, L);
    {
      const bool live = it + 2 < n_tiles;
      Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), live, ring0 + buf * Rg::SLOT);
      if (live) ahead.next();
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();

    // ---- phase 2: this wave's value columns over all features
    float rden[NTB];
#pragma unroll
    for (int tt = 0; tt < NTB; ++tt) {
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) den += dpart[buf][tb0 + tt][c][ww];
      rden[tt] = __builtin_amdgcn_rcpf(den);  // hardware reciprocal (1 ulp)
      if (!renorm) {
        // no D^-1: undo the stabilisers instead, giving phi(q).S in canonical scale
        // (phi = 2^(a' - n') / sqrt(m) on both sides; the keys' constant is gm)
        rden[tt] = 1.f;
        if constexpr (KIND == kPrf) {
          const float qa = qb[buf][(tb0 + tt) * 16 + c] * (1.f / kQueryMargin);
          rden[tt] = fast_exp2(shf[tb0 + tt] - qa * qa * nscale + gm - log2_m);
        }
      }
    }
    f32x4 acc[NCB][NTB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int tt = 0; tt < NTB; ++tt) acc[cb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fc = 0; fc < NFC; ++fc)
#pragma unroll
      for (int tt = 0; tt < NTB; ++tt) {
        const vec8<C> phi = *reinterpret_cast<const vec8<C>*>(&phib[buf][fc][tb0 + tt][lane * 8]);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) mma16(acc[cb][tt], sf[cb][fc], phi);
      }

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int nb = cb0 + cb * NW2;
      if (nb < NVB && nb * 16 < vcols) {
#pragma unroll
        for (int tt = 0; tt < NTB; ++tt) {
          const int tok = tok0 + (tb0 + tt) * 16 + c;
          if (tok < L) {
            const f32x4 o = acc[cb][tt] * rden[tt];
            const size_t off = ((size_t)bh * L + tok) * ldo + nb * 16 + 4 * g;
            if (out_f32) {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = o;
            } else {
              vec4<T> r;
#pragma unroll
              for (int i = 0; i < 4; ++i) r[i] = to_t<T>(o[i]);
              *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(out) + off) = r;
            }
          }
        }
      }
    }
    cur.next();
  }
}

// ---------------------------------------------------------------- standalone features
// Transposed projection as in q_output_kernel; writes phi (stabilised, each row's largest
// entry 1/sqrt(m)) and the per-row log scale. The m features are taken in groups of MG (the
// Omega' fragments of one group are built in LDS from the fp32 matrix by the workgroup); with
// more than one group the positive map first finds every row's maximum over all groups.
// Workgroup = 4 waves over FeatIters * 64 tokens of one (b,h), wave w taking the 16-token blocks
// w, w + 4, ...: every wave loads all its token rows (converted, with their norms) before its
// first store, so no later wait on the memory counter (which counts stores as well) holds the
// stream of phi rows up.
template <typename T, int D>
constexpr int FeatIters = (sizeof(T) == 2 && D <= 64) ? 8 : 4;

template <typename T, int D, int MG, int KIND>
__global__ void __launch_bounds__(256, 2)
features_kernel(const T* __restrict__ X, const float* __restrict__ omega, int H, int L, int m, float eps,
                float inv_sqrt_m, float wscale, float nscale_ln, float* __restrict__ phi,
                float* __restrict__ logscale, int tok_per_wg, int n_tiles) {
  constexpr int IT = FeatIters<T, D>;
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  constexpr int NFB = MG / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  P* oms = reinterpret_cast<P*>(smem);
  float* rmax = reinterpret_cast<float*>(smem + (size_t)NFB * DC * 512 * sizeof(P));  // [tok_per_wg]
  const int bh = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int ng = (m + MG - 1) / MG;
  const float half_log2_m = -__log2f(inv_sqrt_m);
  const T* Xb = X + (size_t)bh * L * D;
  const int tstart = tile * tok_per_wg, tstop = min(L, tstart + tok_per_wg);

  auto build = [&](int gi) {  // Omega' fragments of features [gi*MG, gi*MG + MG), zero past m
    __syncthreads();
    for (int id = threadIdx.x; id < NFB * DC * 64; id += 256) {
      const int l = id & 63, dc = (id >> 6) % DC, fb = (id >> 6) / DC;
      const int lc = l & 15, lg = l >> 4;
      const int r = gi * MG + fb * 16 + lc;
      const float* row = omega + ((size_t)h * m + (r < m ? r : 0)) * D;
      vec8<P> x;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = dc * 32 + 8 * lg + j;
        x[j] = to_t<P>((col < D && r < m) ? row[col] * wscale : 0.f);
      }
      st8<P>(oms + (size_t)id * 8, x);
    }
    __syncthreads();
  };
  // the wave's token rows, converted to the projection type (block it: tokens tstart + (w + 4 it) * 16 + c),
  // and their squared norms |x|^2; rows past L are zero
  vec8<P> xq[IT][DC];
  float xs2[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int tok = tstart + (w + 4 * it) * 16 + c;
    float s2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int col = dc * 32 + 8 * g;
      const vec8<T> raw = (tok < tstop && col < D) ? ld8<T>(Xb + (size_t)tok * D + col) : zero8<T>();
      float c2 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = to_f(raw[j]);
        c2 += v * v;
        xq[it][dc][j] = to_t<P>(v);
      }
      if constexpr (sizeof(P) == 2 && sizeof(T) == 2)
        if (c2 >= kF16MaxSq) clamp_to_f16<P>(raw, xq[it][dc]);
      s2 += c2;
    }
    xs2[it] = group_sum(s2);
  }
  // projection of the wave's token block it against the group in LDS: pacc[fb][i] is feature fb*16 + 4g + i
  // of token tstart + (w + 4 it) * 16 + c
  auto project = [&](int it, f32x4 (&pacc)[NFB]) {
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
      pacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) mma16(pacc[fb], ld8<P>(oms + ((fb * DC + dc) * 64 + lane) * 8), xq[it][dc]);
    }
  };
  // largest valid exponent of the row among this group's features (a whole group needs no mask: a per-element
  // mask turns the chain of three-input maxima into selects)
  auto row_max = [&](int gi, const f32x4 (&pacc)[NFB]) {
    float mx = -INFINITY;
    if (gi * MG + MG <= m) {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pacc[fb][i]);
    } else {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, gi * MG + fb * 16 + 4 * g + i < m ? pacc[fb][i] : -INFINITY);
    }
    return group_max(mx);
  };

  if (KIND == kPrf && ng > 1) {
    for (int gi = 0; gi < ng; ++gi) {
      build(gi);
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int t0 = tstart + (w + 4 * it) * 16;
        if (t0 >= tstop) break;
        f32x4 pacc[NFB];
        project(it, pacc);
        const float mx = row_max(gi, pacc);
        if (g == 0 && t0 + c < tstop) rmax[t0 + c - tstart] = gi == 0 ? mx : fmaxf(rmax[t0 + c - tstart], mx);
      }
    }
  }
  for (int gi = 0; gi < ng; ++gi) {
    build(gi);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t0 = tstart + (w + 4 * it) * 16;
      if (t0 >= tstop) break;
      const int tok = t0 + c;
      const float s2 = xs2[it];
      f32x4 pacc[NFB];
      project(it, pacc);
      float ls = 0.f;
      if constexpr (KIND == kPrf) {
        const float mx = ng > 1 ? rmax[min(tok, tstop - 1) - tstart] : row_max(gi, pacc);
        const float sh = mx + half_log2_m;  // the row's largest entry becomes 2^-log2(sqrt m) = 1/sqrt(m)
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[fb][i] = fast_exp2(pacc[fb][i] - sh);
        ls = mx * kLn2 - s2 * nscale_ln;
      } else if constexpr (KIND == kTrig) {
        // m/2 vectors: the scale 1/sqrt(m/2); exp(|x|^2/2) goes to the log scale
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pacc[fb][i] = trig_feature(pacc[fb][i], gi * MG + fb * 16 + 4 * g + i, m) * (inv_sqrt_m * 1.41421356f);
        ls = s2 * nscale_ln;
      } else {
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[fb][i] = fmaxf(pacc[fb][i], 0.f) * inv_sqrt_m + eps;
      }
      if (tok < L) {
        float* prow = phi + ((size_t)bh * L + tok) * m + gi * MG;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb)
          if (gi * MG + fb * 16 < m) *reinterpret_cast<f32x4*>(prow + fb * 16 + 4 * g) = pacc[fb];
        if (g == 0 && gi == 0) logscale[(size_t)bh * L + tok] = ls;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

KShape kernel_shape(int dtype, int d, int dv, int m) {
  KShape k;
#define X(D_, DV_, M_)                          \
  if (d == D_ && dv == DV_ && m == M_) {        \
    k.dk = D_, k.dvk = DV_, k.mk = M_;          \
    k.exact = k.ok = true;                      \
    return k;                                   \
  }
  FAVOR_SHAPES(X)
#undef X
  if (!(d == 16 || d == 32 || d == 64 || d == 128)) return k;
  if (dv < 16 || dv > 256 || dv % 16 != 0 || m < 16 || m > 512 || m % 16 != 0) return k;
  k.dk = d;
  k.dvk = 64;
  k.mk = d > 64 ? 64 : 32;
  while (k.mk < m) k.mk *= 2;
  k.ok = dtype != 0 || fp32_built(true, d, k.mk);
  return k;
}

bool shape_built(int dtype, int d, int dv, int m) { return kernel_shape(dtype, d, dv, m).ok; }

#ifndef FAVOR_BIDIR_PIECES
#define FAVOR_BIDIR_PIECES 512
#endif
constexpr int kMaxPieces = FAVOR_BIDIR_PIECES;  // two resident 4-wave workgroups on each of 256 CUs
constexpr int kMaxPiecesThree = 3 * FAVOR_BIDIR_PIECES / 2;  // three (the output kernel where kOutThree holds)

// Pieces of the flattened tile space: at most max_pieces, and a whole number per (b,h) when
// that still gives at least 7/8 of them, so that no piece straddles two (b,h) (one set of
// operands per workgroup, one partial per piece).
static int pieces(long long bh, long long tpb, int max_pieces = kMaxPieces) {
  const long long total = bh * tpb;
  long long g = std::min<long long>(total, max_pieces);
  if (bh <= max_pieces) {
    const long long per = std::min<long long>(tpb, max_pieces / bh);
    if (per * bh * 8 >= g * 7) g = per * bh;
  }
  return (int)g;
}

BidirPlan plan_bidir(const Shape& s, int dtype, int Lq) {
  BidirPlan p;
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);  // sizes of the compiled kernels (one column group)
  p.tpb = (s.L + 31) / 32;  // keys
  p.T_all = s.bh() * p.tpb;
  p.G = pieces(s.bh(), p.tpb);
  p.tpb_q = ((Lq > 0 ? Lq : s.L) + 31) / 32;  // queries
  p.T_all_q = s.bh() * p.tpb_q;
  // the output kernel runs three workgroups per CU for 16-bit inputs on at most four waves (kOutThree)
  p.G_q = pieces(s.bh(), p.tpb_q, dtype != 0 && output_waves(ks.mk, ks.dk) <= 4 ? kMaxPiecesThree : kMaxPieces);
  p.nw_reduce = reduce_waves(ks.mk, s.d);
  const int dc = (s.d + 31) / 32, nb = ks.dvk / 16 + 1;
  const size_t slots = (size_t)p.G + (size_t)s.bh();
  size_t off = 0;
  p.off_omf = off;
  off = align256(off + (size_t)s.H * (ks.mk / 16) * dc * 512 * elt(dtype));
  const size_t nfc = (ks.mk + 31) / 32;
  p.off_part = off;
  off = align256(off + slots * nfc * (ks.dvk / 16) * 512 * 4);
  p.off_zpart = off;
  off = align256(off + slots * nfc * 32 * 4);
  p.off_pmax = off;
  off = align256(off + slots * p.nw_reduce * 4);
  p.off_sfr = off;
  off = align256(off + (size_t)s.bh() * nfc * nb * 512 * elt(dtype));
  p.off_gmax = off;
  off = align256(off + (size_t)s.bh() * 4);
  p.total = off;
  return p;
}


// One call on the compiled (D, DV, M): the Omega' fragments once, then reduce, combine and output per
// column group of DV columns of v and out (one group when dv = DV). GEN: the general kernels (runtime
// feature count and column groups); otherwise the exact ones, which also have the trigonometric map.
template <typename T, int D, int DV, int M, bool GEN>
static hipError_t run_bidir(const T* q, const T* k, const T* v, const float* omega, const Shape& s, int Lq,
                            int renorm, int kind, float eps, int out_f32, void* out, void* ws, hipStream_t st,
                            const void* prep) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M, D>::NW;
  constexpr int NWR = RedSplit<M, D>::NW;
  constexpr int DC = (D + 31) / 32;
  const BidirPlan p = plan_bidir(s, sizeof(T) == 4 ? 0 : 1, Lq);
  char* base = static_cast<char*>(ws);
  P* omf = prep ? static_cast<P*>(const_cast<void*>(prep)) : reinterpret_cast<P*>(base + p.off_omf);
  // partials in the contraction type: bf16 for 16-bit inputs (S_aug is rounded to bf16 for the output
  // contraction in any case), fp32 for fp32 inputs
  using PT = C;
  PT* part = reinterpret_cast<PT*>(base + p.off_part);
  PT* zpart = reinterpret_cast<PT*>(base + p.off_zpart);
  float* pmax = reinterpret_cast<float*>(base + p.off_pmax);
  C* sfr = reinterpret_cast<C*>(base + p.off_sfr);
  float* gmx = reinterpret_cast<float*>(base + p.off_gmax);
  const float log2_m = std::log2((float)s.m);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = omega_scale(kind, sc);
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)s.m);

  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  if (!prep)
    launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st,
        omega, s.H, s.m, M, D, wscale, omf, 0);
  for (int c0 = 0; c0 < s.dv; c0 += DV) {
    const int vcols = std::min(DV, s.dv - c0);
    const T* vg = v + c0;
    void* og = out_f32 ? static_cast<void*>(static_cast<float*>(out) + c0) : static_cast<void*>(static_cast<T*>(out) + c0);
    if (kind == kPrf)
      launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, kPrf, false, false, GEN, PT>, p.G, 64 * NWR, 0, st, k, vg, omf, nullptr,
          s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, 0, 0, s.m, s.dv, vcols);
    else if (!GEN && kind == kTrig)
      launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, GEN ? kPrf : kTrig, false, false, GEN, PT>, p.G, 64 * NWR, 0, st, k, vg,
          omf, nullptr, s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, 0, 0, s.m, s.dv,
          vcols);
    else
      launch("reduce", kv_reduce_kernel<T, D, DV, M, kReduceRing, kRelu, false, false, GEN, PT>, p.G, 64 * NWR, 0, st, k, vg, omf, nullptr,
          s.H, s.L, p.tpb, p.T_all, p.G, eps, inv_sqrt_m, nscale, part, zpart, pmax, 0, 0, s.m, s.dv, vcols);
    // one thread per (value block, lane): every partial is requested in a single round
    constexpr int NBC = DV / 16 + 1;
    launch("combine", combine_kernel<C, D, DV, M, PT>, (unsigned)(s.bh() * ((M + 31) / 32)), 64 * (NBC < 16 ? NBC : 16), 0,
        st, part, zpart, pmax, p.tpb, p.T_all, p.G, kind, sfr, gmx);
    if (kind == kPrf)
      launch("output", q_output_kernel<T, D, DV, M, kPrf, GEN>, p.G_q, 64 * NW, 0, st, q, omf, sfr, s.H, Lq, p.tpb_q,
          p.T_all_q, p.G_q, eps, inv_sqrt_m, out_f32, renorm, gmx, nscale, log2_m, og, s.m, s.dv, vcols);
    else if (!GEN && kind == kTrig)
      launch("output", q_output_kernel<T, D, DV, M, GEN ? kPrf : kTrig, GEN>, p.G_q, 64 * NW, 0, st, q, omf, sfr, s.H, Lq,
          p.tpb_q, p.T_all_q, p.G_q, eps, inv_sqrt_m, out_f32, renorm, gmx, nscale, log2_m, og, s.m, s.dv, vcols);
    else
      launch("output", q_output_kernel<T, D, DV, M, kRelu, GEN>, p.G_q, 64 * NW, 0, st, q, omf, sfr, s.H, Lq, p.tpb_q,
          p.T_all_q, p.G_q, eps, inv_sqrt_m, out_f32, renorm, gmx, nscale, log2_m, og, s.m, s.dv, vcols);
  }
  return hipGetLastError();
}

hipError_t launch_bidir(const void* q, const void* k, const void* v, const float* omega, const Shape& s, int Lq,
                        int renorm, int dtype, int kind, float eps, int out_f32, void* out, void* ws,
                        hipStream_t st, const void* prep) {
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);
  if (!ks.ok || (!ks.exact && kind == kTrig)) return hipErrorInvalidValue;
#define X(D_, DV_, M_, GEN_)                                                                                   \
  if (ks.exact == !GEN_ && ks.dk == D_ && ks.dvk == DV_ && ks.mk == M_) {                                      \
    if (dtype == 0) {                                                                                          \
      if constexpr (fp32_built(GEN_, D_, M_))                                                                  \
        return run_bidir<float, D_, DV_, M_, GEN_>(static_cast<const float*>(q), static_cast<const float*>(k), \
                                                   static_cast<const float*>(v), omega, s, Lq, renorm, kind,   \
                                                   eps, out_f32, out, ws, st, prep);                            \
      return hipErrorInvalidValue;                                                                             \
    }                                                                                                          \
    return run_bidir<bf16, D_, DV_, M_, GEN_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),        \
                                              static_cast<const bf16*>(v), omega, s, Lq, renorm, kind, eps,     \
                                              out_f32, out, ws, st, prep);                                      \
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

size_t omega_prepared_bytes(const Shape& s, int dtype) {
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);
  if (!ks.ok) return 0;
  return align256((size_t)s.H * (ks.mk / 16) * ((s.d + 31) / 32) * 512 * elt(dtype));
}

hipError_t launch_prepare_omega(const float* omega, const Shape& s, int dtype, int kind, void* prep, hipStream_t st) {
  const KShape ks = kernel_shape(dtype, s.d, s.dv, s.m);
  if (!ks.ok) return hipErrorInvalidValue;
  const float wscale = omega_scale(kind, std::pow((float)ks.dk, -0.25f));
  const long long nfrag = (long long)s.H * (ks.mk / 16) * ((ks.dk + 31) / 32) * 64;
  const unsigned grid = (unsigned)std::min<long long>((nfrag + 255) / 256, 4096);
  if (dtype == 0)
    launch("omega_frag", omega_frag_kernel<float>, grid, 256, 0, st, omega, s.H, s.m, ks.mk, ks.dk, wscale,
        static_cast<float*>(prep), 0);
  else
    launch("omega_frag", omega_frag_kernel<f16>, grid, 256, 0, st, omega, s.H, s.m, ks.mk, ks.dk, wscale,
        static_cast<f16*>(prep), 0);
  return hipGetLastError();
}

}  // namespace favor

// ---------------------------------------------------------------- workspace without allocation
// The workspace of favor_bidir_noalloc: one array per device, held from the library's first use on that device
// until the process ends. In host code `scratch` names a host-side stand-in, not the device memory: the device
// address is resolved once per device with hipGetSymbolAddress and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[FAVOR_BIDIR_NOALLOC_MAX_BYTES];

namespace favor {
namespace {
constexpr int kNoallocDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kNoallocDevices];  // device address of `scratch` on each device, null until resolved
}  // namespace

hipError_t noalloc_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kNoallocDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // `dev` is the current device
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_addr[dev] = p;
  }
  *ptr = scratch_addr[dev];
  return hipSuccess;
}

// The feature map on groups of MG features (every m up to MG; 512 as two groups of 256).
template <typename T, int D, int MG, int KIND>
static hipError_t run_features(const T* x, const float* omega, const Shape& s, float eps, float* phi,
                               float* logscale, hipStream_t st) {
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = omega_scale(KIND, sc);
  const float nscale_ln = sc * sc * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)s.m);
  const int tpw = 64 * FeatIters<T, D>;  // tokens per workgroup: 4 waves x FeatIters blocks of 16
  const int n_tiles = (s.L + tpw - 1) / tpw;
  const size_t lds = (size_t)(MG / 16) * DC * 512 * sizeof(P) + tpw * sizeof(float);
  // once per instantiation (a function-local static is initialised exactly once, also under concurrent
  // first calls)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&features_kernel<T, D, MG, KIND>), hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  launch("features", features_kernel<T, D, MG, KIND>, (unsigned)(s.bh() * n_tiles), 256, lds, st, x, omega, s.H,
      s.L, s.m, eps, inv_sqrt_m, wscale, nscale_ln, phi, logscale, tpw, n_tiles);
  return hipGetLastError();
}

hipError_t launch_features(const void* x, const float* omega, const Shape& s, int dtype, int kind, float eps,
                           float* phi, float* logscale, hipStream_t st) {
  // feature groups: up to 256 features, 128 where the fragments and accumulators of a group would not fit the
  // registers (fp32 at d >= 64, 16-bit inputs at d = 128)
  const int mg_max = (dtype == 0 ? s.d >= 64 : s.d > 64) ? 128 : 256;
  int mg = 16;
  while (mg < s.m && mg < mg_max) mg *= 2;
#define XK(D_, MG_, K_)                                                                                          \
  if (kind == K_) {                                                                                              \
    if (dtype == 0)                                                                                              \
      return run_features<float, D_, MG_, K_>(static_cast<const float*>(x), omega, s, eps, phi, logscale, st);   \
    return run_features<bf16, D_, MG_, K_>(static_cast<const bf16*>(x), omega, s, eps, phi, logscale, st);       \
  }
#define X(D_, MG_)                  \
  if (s.d == D_ && mg == MG_) {     \
    XK(D_, MG_, kPrf)               \
    XK(D_, MG_, kRelu)              \
    XK(D_, MG_, kTrig)              \
    return hipErrorInvalidValue;    \
  }
#define XD(D_) X(D_, 16) X(D_, 32) X(D_, 64) X(D_, 128)
  XD(16) XD(32) XD(64) XD(128)
  X(16, 256) X(32, 256) X(64, 256)
#undef XD
#undef X
#undef XK
  return hipErrorInvalidValue;
}

}  // namespace favor
