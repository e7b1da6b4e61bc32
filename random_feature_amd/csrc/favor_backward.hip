// Gradients of bidirectional FAVOR+ on gfx950.
//
// Performer paper, equation 4 and Algorithm 1: out_i = N_i / D_i with N = Phi_Q S, D = Phi_Q z,
// S = Phi_K^T V, z = Phi_K^T 1. For an upstream gradient g = dL/dout the chain rule gives
//   W_i = [g_i, -(g_i . out_i)] / D_i                       (dv + 1 columns)
//   dPhi_Q = W S_aug^T,  dS_aug = Phi_Q^T W,   S_aug = [S z], dS_aug = [dS dz]
//   dPhi_K = [V 1] dS_aug^T,  dV = Phi_K dS
// and through the positive feature map phi(x) = exp(w.xs - |xs|^2/2)/sqrt(m), xs = d^-1/4 x:
//   dx = d^-1/4 (Omega^T (phi * dphi) - xs sum_r phi_r dphi_r).
// For the queries sum_r phi_r dphi_r = g_i . out_i - g_i . out_i = 0, so only the first term
// remains. Through the ReLU map phi_r(x) = max(w_r.xs, 0)/sqrt(m) + eps (appendix A.4 of the
// Performer paper) the derivative is a mask: dx = d^-1/4 Omega^T (1[w.xs > 0] * dphi)/sqrt(m); the
// kernels below take KIND = kRelu with phi' = phi itself (no stabiliser, key scale F_j = 1). Every per-row constant of the query features and the keys' common constant
// cancel in phi * dphi (query side) or come out as one per-key factor (key side), so the
// kernels work with stabilised features throughout:
//   query side: phi' = 2^(a' - max_r a'), features of the row scaled to a largest entry of 1;
//   key side:   phi' likewise, and the key's true scale F_j = 2^(max_r a'_j - n'_j - M) / sqrt(m)
//               relative to the stabilised sums (M the keys' common maximum of the forward).
// Kernels, in launch order:
//   omega_frag_kernel / omegaT_frag_kernel  Omega' fragments for the projections and for
//                       Omega'^T (the gradient's back-projection)
//   kv_reduce_kernel    the forward key/value reduction (recomputed), then
//   combine_rows_kernel S_aug of every (b,h) as fp32 rows, and the keys' maximum M
//   bwd_q_kernel        per 32-query tile: Phi_Q, D, W, dPhi_Q = W S_aug^T on MFMA, dq, and
//                       the piece's partial dS_aug += Phi_Q^T W
//   combine_rows_kernel dS_aug of every (b,h) as fp32 rows
//   bwd_k_kernel        per 32-key tile: Phi_K, dPhi_K = [V 1] dS_aug^T, dk and dV
// The two products that subtract nearly equal terms (dPhi_Q's S g - z (g . out) and dPhi_K's
// dS v + dz) take fp16 operands (11-bit mantissas) scaled by powers of two: S_aug and dS_aug
// per (b,h) to a largest magnitude in [8, 16), W and [V 1] per row to one in [1/2, 1); the
// scales are undone exactly on the results. The sums whose terms cancel across tokens take
// bf16 operands as hi + lo pairs: the recomputed S_aug (key features split, two MFMAs) and
// dS_aug (phi' and W split, three MFMAs), which keeps them near fp32 accuracy. Products
// without cancellation use bf16.
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_tiles.hpp"
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

// operand types of the backward: XS for the scaled products, XB for the range-safe ones
template <typename T> struct BwdOps;
template <> struct BwdOps<bf16> { using XS = f16; using XB = bf16; };
template <> struct BwdOps<float> { using XS = float; using XB = float; };

// Omega'^T fragments, the A operand (rows = d, k = features): frag[h][db][fc][lane][j] =
// scale * omega[h][f][db*16 + c] with f = fc*32 + 8g + j (0 past m or d), the order in which
// lane (c, g) reads 8 consecutive features of a row operand.
template <typename T>
__global__ void omegaT_frag_kernel(const float* __restrict__ omega, int H, int m, int d, float scale,
                                   T* __restrict__ frag) {
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
    vec8<T> x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = fc * 32 + 8 * g + j;
      x[j] = to_t<T>((f < m && dd < d) ? omega[((size_t)h * m + f) * d + dd] * scale : 0.f);
    }
    st8<T>(frag + (size_t)id * 8, x);
  }
}

// Row length (floats) of S_aug / dS_aug rows: dv + 1 columns padded to whole 32-column chunks.
template <int DV> struct Rows {
  static constexpr int RC = ((DV + 1 + 31) / 32) * 32;
  static constexpr int KC = RC / 32;
};

// Per (b*h, 32-feature chunk): the partials of the pieces of that (b,h) (fragment layout of
// kv_reduce_kernel), scaled by 2^(M_piece,wave - M_max) when `scaled`, summed and written as
// fp32 rows rows[bh][f][RC] (value columns, the z column at DV, zeros after); the common
// maximum goes to gmx[bh] (0 when not scaled) unless gmx is null. tpb, T_all and G describe
// the pieces that wrote the partials (slot = piece + bh); NWP waves per piece wrote maxima.
template <int DV, int M, int NWP>
__global__ void __launch_bounds__(256)
combine_rows_kernel(const float* __restrict__ part, const float* __restrict__ zpart, const float* __restrict__ pmax,
                    int tpb, long long T_all, int G, int scaled, float* __restrict__ rows,
                    float* __restrict__ gmx) {
  constexpr int FBP = M / (16 * NWP);
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (M + 31) / 32;
  constexpr int RC = Rows<DV>::RC;
  const int bh = blockIdx.x / NFC, fc = blockIdx.x % NFC;
  const long long i_lo = piece_of((long long)bh * tpb, T_all, G);
  const long long i_hi = piece_of((long long)(bh + 1) * tpb - 1, T_all, G);
  const int np = (int)(i_hi - i_lo + 1);
  const int wv = (fc * 32) / (FBP * 16);
  float gmax = -INFINITY;
  if (scaled) {
    // the np*NWP maxima of this (b,h) are contiguous: one load per lane, then a wave maximum
    const float* pm = pmax + (size_t)(i_lo + bh) * NWP;
    for (int k = threadIdx.x & 63; k < np * NWP; k += 64) gmax = fmaxf(gmax, pm[k]);
    gmax = wave_max(gmax);
  }
  if (gmx && fc == 0 && threadIdx.x == 0) gmx[bh] = scaled ? gmax : 0.f;
  float* out = rows + (size_t)bh * M * RC;
  for (int e = threadIdx.x; e < NB * 64; e += blockDim.x) {
    const int nb = e >> 6, lane = e & 63;
    const int c = lane & 15, g = lane >> 4;
    f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f}, hi = lo;
    if (nb < NB - 1 || c == 0) {
      for (int k = 0; k < np; ++k) {
        const size_t slot = (size_t)(i_lo + k) + bh;
        const float sc = scaled ? fast_exp2(pmax[slot * NWP + wv] - gmax) : 1.f;
        const float* src = (nb < NB - 1) ? part + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8
                                         : zpart + ((slot * NFC + fc) * 4 + g) * 8;
        lo += reinterpret_cast<const f32x4*>(src)[0] * sc;
        hi += reinterpret_cast<const f32x4*>(src)[1] * sc;
      }
    }
    const int col = nb * 16 + c;  // the z column is DV = (NB - 1) * 16; past it zeros
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f0 = fc * 32 + 4 * g + i, f1 = f0 + 16;
      if (f0 < M) out[(size_t)f0 * RC + col] = lo[i];
      if (f1 < M) out[(size_t)f1 * RC + col] = hi[i];
    }
  }
  // columns past the last block
  constexpr int PAD = RC - NB * 16;
  if constexpr (PAD > 0)
    for (int e = threadIdx.x; e < 32 * PAD; e += blockDim.x) {
      const int f = fc * 32 + e / PAD, col = NB * 16 + e % PAD;
      if (f < M) out[(size_t)f * RC + col] = 0.f;
    }
}

// Largest magnitude across the NW waves of a workgroup (xch: NW floats; two barriers).
template <int NW>
__device__ __forceinline__ float wg_absmax(float x, float* xch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max(x);
  if (lane == 0) xch[w] = x;
  lds_barrier();
  float r = xch[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, xch[i]);
  lds_barrier();
  return r;
}

// exponent e with x * 2^-e in [1/2, 1) (0 for x = 0 or not finite)
__device__ __forceinline__ int scale_exp(float x) {
  int e = 0;
  if (x > 0.f && x < INFINITY) (void)frexpf(x, &e);
  return e;
}

// ---------------------------------------------------------------- query side
// Workgroup = NW waves over one piece of the flattened query-tile space; wave w owns FB*16
// features. Per tile of 32 queries (Q and dOut rows arrive through a two-slot DMA ring):
//   g rows       scaled per query to [1/2, 1) (fp16, exponent e_i)
//   projection   A = Omega' (rows = features), B = Q rows -> a'[feature][query]; the exact
//                row maximum across the waves; phi' = 2^(a' - max) in (0, 1]
//   u            A = S rows (fp16, scaled by 2^-eS per (b,h)), B = g rows -> u = S g (scaled)
//   D', A        D'_i = phi'_i . z and A_i = phi'_i . u_i, fp32 sums over the features, across
//                the waves through LDS; gamma_i = g_i . out_i = A_i 2^(eS + e_i) / D'_i
//   dPhi_Q       phi' * (u - z A/D'), the scaled dPhi_Q (phi'.dPhi_Q = 0 by construction),
//                written as fp16 rows [query][feature] to LDS
//   dq           per wave BPW blocks of dq^T (16 dims x 16 queries): A = Omega'^T fragments
//                over all features, B = the rows above; times 2^(eS + e_i)/D'_i, stored
//   dS_aug       W_i = [g_i, -gamma_i]/D'_i (rows), A = phi'^T (transposing reads of the phi' rows
//                in LDS), B = W (transposing reads), both as sums of two bf16 parts;
//                accumulated over the piece's tiles of one (b,h) and written as a partial in
//                the reduction's fragment layout
// The dq and dS_aug contractions of a tile run during the next tile, between its row-maximum and
// sums exchanges, so a tile has three barriers: the rows they read are published by the next
// tile's first barrier.
// KIND = kRelu: phi' = max(a, 0)/sqrt(m) + eps (the features themselves, no row maximum), and the
// rows of dPhi_Q carry the mask 1[a > 0] instead of the factor phi' (1/sqrt(m) goes into the scale).
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
bwd_q_kernel(const T* __restrict__ Q, const T* __restrict__ dOut, const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo,
             const typename Ops<T>::P* __restrict__ omT, const float* __restrict__ srow, int H, int L, int tpb,
             long long T_all, int G, int grad_f32, float* __restrict__ dpart, float* __restrict__ dzpart,
             void* __restrict__ dq, float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using XS = typename BwdOps<T>::XS;
  using XB = typename BwdOps<T>::XB;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB % 2 == 0 || NW == 1, "an odd block count per wave only with a single wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NDB = D / 16;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (M + 31) / 32;
  constexpr int NFCW = (FB + 1) / 2;
  constexpr int BPW = 2 * NDB / NW;  // dq^T blocks (dims db, queries tb) per wave
  static_assert(BPW >= 1 && (2 * NDB) % NW == 0, "dq blocks split evenly over the waves");
  constexpr int NDBW = (BPW + 1) / 2;  // dimension blocks per wave
  constexpr int RC = Rows<DV>::RC, KC = Rows<DV>::KC;
  constexpr int KROW = D + 8;
  // row strides (elements) of the LDS rows: the transposing reads of W take 8 rows of 32 bytes per half wave,
  // which land in 8 different bank groups when the stride is an odd multiple of 8 dwords; the g rows keep a
  // stride whose 16 rows per quarter wave fall into distinct 4-bank groups for their row reads
  constexpr int EROW = FB * 16 + 8;
  constexpr int WROW = RC + 8;
  constexpr int WBROW = RC + 16;
  constexpr int PROW = NFC * 32 + 8;
  constexpr int CPR = DV / 8;                     // 8-column chunks of a g row
  constexpr int IPT = (32 * CPR + NT - 1) / NT;  // (query, chunk) items per thread
  using Rg = Ring<T, D, DV, NT, true>;  // Q rows and dOut rows of a tile
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P qs[32 * KROW];
  constexpr int NSPL = sizeof(XB) == 2 ? 2 : 1;  // bf16 operands of dS_aug as a sum of two (hi + lo)
  __shared__ __attribute__((aligned(16))) XB erow[NSPL][NW][32 * EROW];
  __shared__ __attribute__((aligned(16))) XS gsr[32 * WROW];
  __shared__ __attribute__((aligned(16))) XB wbr[NSPL][32 * WBROW];
  __shared__ __attribute__((aligned(16))) XS prow[32 * PROW];
  // per-wave partials across the waves, [query][wave], a lane reading its query's NW (one padding column: the
  // rows of a quarter wave then fall into distinct banks)
  __shared__ __attribute__((aligned(16))) float qmx[32][NW + 1];
  __shared__ __attribute__((aligned(16))) float dsum[32][NW + 1];
  __shared__ __attribute__((aligned(16))) float asum[32][NW + 1];
  __shared__ __attribute__((aligned(16))) float gex[32], rsc[32];
  __shared__ float xch[NW];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  const long long t_beg = piece_start(pc, T_all, G), t_end = piece_start(pc + 1, T_all, G);
  if (t_beg >= t_end) return;
  const int n_tiles = (int)(t_end - t_beg);
  const uint32_t ring0 = lds_addr(&ring[0][0]);
  TileCursor cur(t_beg, tpb), ahead(t_beg, tpb);

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
  vec8<P> omt[NDBW][NFC];
  vec8<XS> sa[FB][KC];
  float zv[FB][4];  // z of this lane's features (4g + i of each block)
  f32x4 sacc[FB][NB];
  int eS = 0;  // S rows were scaled by 2^-eS
  int cur_bh = -1;
  // the contractions of a tile (dq and dS_aug) run one tile late, after the next tile's row maxima
  // are exchanged, beside that tile's feature map; the tile's dq blocks are stored from there
  f32x4 pend[BPW];
  int pend_bh = -1, pend_tok0 = 0;
  bool pending = false;
  auto store_pending = [&]() {
    if (pend_bh < 0) return;
    // the (b,h)'s rows from a base common to the wave and 32-bit offsets within them (one register per lane
    // instead of a 64-bit address, which the tile loop otherwise keeps in scratch)
    const size_t bh_off = (size_t)pend_bh * L * D;
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = w * BPW + bi, db = blk >> 1, tb = blk & 1;
      const int tok = pend_tok0 + tb * 16 + c;
      if (tok < L) {
        const uint32_t off = (uint32_t)tok * D + db * 16 + 4 * g;
        if (grad_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dq) + bh_off + off) = pend[bi];
        } else {
          vec4<T> o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = to_t<T>(pend[bi][i]);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(dq) + bh_off + off) = o4;
        }
      }
    }
  };

  auto zero_sums = [&]() {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // partial dS_aug of (piece, bh) in the reduction's fragment layout (slot = piece + bh)
  auto flush = [&](int fbh) {
    const size_t slot = (size_t)pc + fbh;
#pragma unroll
    for (int p = 0; p < NFCW; ++p) {
      const int fc = (w * FB) / 2 + p;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 lo = sacc[2 * p][nb];
        const f32x4 hi = (2 * p + 1 < FB) ? sacc[2 * p + 1][nb] : f32x4{0.f, 0.f, 0.f, 0.f};
        float* dst = (nb < NB - 1) ? dpart + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8
                                   : dzpart + ((slot * NFC + fc) * 4 + g) * 8;
        if (nb < NB - 1 || c == 0) {
          reinterpret_cast<f32x4*>(dst)[0] = lo;
          reinterpret_cast<f32x4*>(dst)[1] = hi;
        }
      }
    }
  };

  // dq and dS_aug of the pending tile, from its rows in LDS (prow, wbr, the wave's own erow, rsc): between
  // the next tile's row-maximum exchange and the exchange of its sums (which precedes every write of
  // those rows), or before the sums of the pending tile's (b,h) are flushed
  auto contract_pending = [&]() {
    if (!pending) return;
    pending = false;
    // ---- dq: this wave's blocks of dq^T over all features, scaled and stored
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
      const int blk = w * BPW + bi, tb = blk & 1;
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fc = 0; fc < NFC; ++fc) mma16(a, omt[bi >> 1][fc], ld8<XS>(&prow[(tb * 16 + c) * PROW + fc * 32 + 8 * g]));
      pend[bi] = a * rsc[tb * 16 + c];
    }
    store_pending();

    // ---- dS_aug += phi'^T W over the tile's queries: with bf16 operands as hi + lo pairs,
    // hi*hi + hi*lo + lo*hi (the sums over the queries cancel, so 8-bit operands would not do)
    {
      auto tr8 = [&](const XB* base, int stride, int col0) {
        vec8<XB> r;
        if constexpr (sizeof(XB) == 2) {
          const bf16x4 lo = lds_read_tr4(reinterpret_cast<const bf16*>(base + (4 * g + (c >> 2)) * stride + col0 + 4 * (c & 3)));
          const bf16x4 hi = lds_read_tr4(reinterpret_cast<const bf16*>(base + (16 + 4 * g + (c >> 2)) * stride + col0 + 4 * (c & 3)));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r[i] = lo[i];
            r[i + 4] = hi[i];
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) r[jj] = base[(16 * (jj >> 2) + 4 * g + (jj & 3)) * stride + col0 + c];
        }
        return r;
      };
      // the phi' fragments of the wave's features once, then W one column block at a time (fewer live
      // registers beside the next tile's projections)
      vec8<XB> ea[FB], el[NSPL == 2 ? FB : 1];
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        ea[fb] = tr8(&erow[0][w][0], EROW, fb * 16);
        if constexpr (NSPL == 2) el[fb] = tr8(&erow[NSPL - 1][w][0], EROW, fb * 16);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const vec8<XB> w0 = tr8(wbr[0], WBROW, nb * 16);
        vec8<XB> w1 = w0;
        if constexpr (NSPL == 2) w1 = tr8(wbr[NSPL - 1], WBROW, nb * 16);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          mma16(sacc[fb][nb], ea[fb], w0);
          if constexpr (NSPL == 2) {
            mma16(sacc[fb][nb], ea[fb], w1);
            mma16(sacc[fb][nb], el[fb], w0);
          }
        }
      }
    }
  };

  Rg::issue(Q, dOut, L, ahead.bh, ahead.tok0(), true, ring0);
  ahead.next();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int bh = cur.bh, tok0 = cur.tok0();
    // ---- this tile's Q and dOut rows land (the dOut rows are read across threads), Q is
    // converted; the next tile's copies start
    wait_vmcnt<0>();  // the copies, and every store of the previous tile
    lds_barrier();
    Rg::template convert<P, KROW, kNormNone>(ring[buf], qs, nullptr, 0.f, L);
    if (it + 1 < n_tiles) {
      Rg::issue(Q, dOut, L, ahead.bh, ahead.tok0(), true, ring0 + (buf ^ 1) * Rg::SLOT);
      ahead.next();
    }
    // ---- a new (b,h): close the old one's sums, load this one's operands
    if (bh != cur_bh) {
      contract_pending();  // the previous tile's rows are complete (top barrier); before Omega'^T is replaced
      if (cur_bh >= 0) flush(cur_bh);
      zero_sums();
      const int h = bh % H;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
#pragma unroll
      for (int i = 0; i < NDBW; ++i)
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc)
          omt[i][fc] = ld8<P>(omT + ((((size_t)h * NDB + (w * BPW) / 2 + i) * NFC + fc) * 64 + lane) * 8);
      const float* rows = srow + (size_t)bh * M * RC;
      f32x8 sf[FB][KC];
      float amax = 0.f;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const int f = (w * FB + fb) * 16 + c;
          const f32x4* src = reinterpret_cast<const f32x4*>(rows + (size_t)f * RC + kc * 32 + 8 * g);
          const f32x4 a = src[0], b = src[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sf[fb][kc][j] = a[j];
            sf[fb][kc][j + 4] = b[j];
            amax = fmaxf(amax, fmaxf(fabsf(a[j]), fabsf(b[j])));
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) zv[fb][i] = rows[(size_t)((w * FB + fb) * 16 + 4 * g + i) * RC + DV];
      }
      eS = scale_exp(wg_absmax<NW>(amax, xch)) - 4;  // largest |S_aug| * 2^-eS in [8, 16)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int j = 0; j < 8; ++j) sa[fb][kc][j] = to_t<XS>(ldexpf(sf[fb][kc][j], -eS));
      // every operand has landed here, so no wait for them falls to their first uses in the tile,
      // where it would also hold up the next tile's copies on every tile
      wait_vmcnt<0>();
      cur_bh = bh;
    }
    // ---- g rows scaled per query (rows past L: zero)
    float gv[IPT][8];
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int item = threadIdx.x + u * NT;
      const int row = item / CPR, c8 = item % CPR;
      const bool ok = item < 32 * CPR && tok0 + row < L;
      const vec8<T> g8 = ld8<T>(reinterpret_cast<const T*>(ring[buf] + Rg::v_off(min(row, 31), c8 * 8)));
      float mabs = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        gv[u][j] = ok ? to_f(g8[j]) : 0.f;
        mabs = fmaxf(mabs, fabsf(gv[u][j]));
      }
      mabs = lanes_max<CPR>(mabs);
      if (item < 32 * CPR) {
        const int eg = scale_exp(mabs);
        vec8<XS> x8;
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] = to_t<XS>(ldexpf(gv[u][j], -eg));
        *reinterpret_cast<vec8<XS>*>(&gsr[row * WROW + c8 * 8]) = x8;
        if (c8 == 0) {
          for (int col = DV; col < RC; ++col) gsr[row * WROW + col] = to_t<XS>(0.f);
          gex[row] = (float)eg;
        }
      }
    }
    lds_barrier();  // qs of this tile, scaled g rows

    // ---- projection and row maxima
    f32x4 pq[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<P> qf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        qf[dc] = (col < D) ? ld8<P>(&qs[(tb * 16 + c) * KROW + col]) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pq[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16_split_a<PSO>(pq[tb][fb], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0], qf[dc]);
      }
      if constexpr (KIND == kPrf) {
        float mx = -INFINITY;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pq[tb][fb][i]);
        mx = group_max(mx);
        if (g == 0) qmx[tb * 16 + c][w] = mx;
      }
    }
    // ---- u = S g (scaled), [feature][query]
    f32x4 uq[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<XS> gf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) gf[kc] = ld8<XS>(&gsr[(tb * 16 + c) * WROW + kc * 32 + 8 * g]);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        uq[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma16(uq[tb][fb], sa[fb][kc], gf[kc]);
      }
    }
    lds_barrier();  // B1: row maxima
    // the two waves of a SIMD (w and w + NW/2) take the pending contractions and the feature map below in opposite
    // orders, so that one's matrix work overlaps the other's vector work; the phi' rows that the contractions read
    // are rewritten only after both
    // (the ReLU map keeps one order: its mask bits leave no registers for the other)
    const bool first_half = KIND != kPrf || __builtin_amdgcn_readfirstlane(w) < NW / 2;
    if (first_half) contract_pending();

    // ---- phi' = 2^(a' - max) (ReLU: the features); D' and A partials; phi' rows for the dS transposes
    unsigned pos = 0;  // ReLU: bit (tb*FB + fb)*4 + i set where a > 0
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float mx = 0.f;
      if constexpr (KIND == kPrf) {
        mx = qmx[tb * 16 + c][0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, qmx[tb * 16 + c][ww]);
      }
      float dz = 0.f, da = 0.f;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ph;
          if constexpr (KIND == kPrf) {
            ph = fast_exp2(pq[tb][fb][i] - mx);
          } else {
            const float a = pq[tb][fb][i];
            if (a > 0.f) pos |= 1u << ((tb * FB + fb) * 4 + i);
            ph = fmaxf(a, 0.f) * inv_sqrt_m + eps;
          }
          pq[tb][fb][i] = ph;
          dz += ph * zv[fb][i];
          da += ph * uq[tb][fb][i];
        }
      }
      dz = group_sum(dz);
      da = group_sum(da);
      if (g == 0) {
        dsum[tb * 16 + c][w] = dz;
        asum[tb * 16 + c][w] = da;
      }
    }
    if (!first_half) contract_pending();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        vec4<XB> e4, e4lo;
        split_all<4>(e4, e4lo, [&](int i) { return pq[tb][fb][i]; });
        *reinterpret_cast<vec4<XB>*>(&erow[0][w][(tb * 16 + c) * EROW + fb * 16 + 4 * g]) = e4;
        if constexpr (NSPL == 2) *reinterpret_cast<vec4<XB>*>(&erow[NSPL - 1][w][(tb * 16 + c) * EROW + fb * 16 + 4 * g]) = e4lo;
      }
    lds_barrier();  // B2: D' and A partials, phi' rows

    // ---- phi' * dPhi_Q (scaled) as rows [query][feature]
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float den = 0.f, aa = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        den += dsum[tb * 16 + c][ww];
        aa += asum[tb * 16 + c][ww];
      }
      const float ad = aa * __builtin_amdgcn_rcpf(den);  // hardware reciprocal (1 ulp)
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        vec4<XS> p4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float fac = (KIND == kPrf) ? pq[tb][fb][i] : ((pos >> ((tb * FB + fb) * 4 + i)) & 1u ? 1.f : 0.f);
          p4[i] = to_t<XS>(fac * (uq[tb][fb][i] - zv[fb][i] * ad));
        }
        *reinterpret_cast<vec4<XS>*>(&prow[(tb * 16 + c) * PROW + (w * FB + fb) * 16 + 4 * g]) = p4;
      }
    }
    // ---- W rows (bf16): [g, -gamma] / D'
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int item = threadIdx.x + u * NT;
      if (item < 32 * CPR) {
        const int row = item / CPR, c8 = item % CPR;
        float den = 0.f, aa = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          den += dsum[row][ww];
          aa += asum[row][ww];
        }
        // rows past L: W = 0 (their denominators are not used; a ReLU row of zero features has D' = 0)
        const float rd = tok0 + row < L ? __builtin_amdgcn_rcpf(den) : 0.f;  // hardware reciprocal (1 ulp)
        vec8<XB> wb, wl;
        split_all<8>(wb, wl, [&](int j) { return gv[u][j] * rd; });
        *reinterpret_cast<vec8<XB>*>(&wbr[0][row * WBROW + c8 * 8]) = wb;
        if constexpr (NSPL == 2) *reinterpret_cast<vec8<XB>*>(&wbr[NSPL - 1][row * WBROW + c8 * 8]) = wl;
        if (c8 == 0) {
          const int e = (int)gex[row] + eS;
          const float gam = ldexpf(aa, e) * rd;  // g . out
          for (int col = DV; col < RC; ++col) {
            const float x = col == DV ? -gam * rd : 0.f;
            const XB xh = to_t<XB>(x);
            wbr[0][row * WBROW + col] = xh;
            if constexpr (NSPL == 2) wbr[NSPL - 1][row * WBROW + col] = to_t<XB>(x - to_f(xh));
          }
          rsc[row] = ldexpf(rd * (KIND == kPrf ? 1.f / kLog2e : inv_sqrt_m), e);
        }
      }
    }
    // the rows of this tile (dPhi_Q, W, phi', the dq scales) are read by its contractions, after the
    // next tile's top barrier
    pending = true;
    pend_bh = bh;
    pend_tok0 = tok0;
    cur.next();
  }
  lds_barrier();  // the last tile's rows
  contract_pending();
  flush(cur_bh);
}

// ---------------------------------------------------------------- key side
// Workgroup = NW waves over one piece of the flattened key-tile space; wave w owns FB*16
// features. Per tile of 32 keys:
//   projection   A = Omega', B = K rows (fp16, converted with |k|^2 n'-norms) -> a'[feature][key];
//                exact row maximum across the waves; phi' = 2^(a' - max) in (0, 1]; the key's
//                scale F_j = 2^(max_j - n'_j - M) (0 for keys past L)
//   [V 1] rows   scaled per key to [1/2, 1), fp16, in LDS
//   dPhi_K       A = dS_aug rows (fp16, scaled per (b,h)), B = [V 1] rows -> [feature][key];
//                P = phi' * dPhi_K and phi' written as rows [key][feature] to LDS
//   dk           per wave, blocks of dk^T: A = Omega'^T over all features, B = P rows; minus
//                d^-1/2 k_j sum_r P_jr (that sum across the waves through LDS)
//   dV           per wave, blocks of dV^T: A = dS^T (bf16 fragments over all features),
//                B = phi' rows (bf16)
//   both scaled by F_j (and the operand scales) and stored.
// KIND = kRelu: phi' = max(a, 0)/sqrt(m) + eps (no row maximum, F_j = 1), P = 1[a > 0] * dPhi_K with
// 1/sqrt(m) in the scale of dk, and no norm term.
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * BwdSplit<M>::NW, 1)
bwd_k_kernel(const T* __restrict__ K, const T* __restrict__ V, const typename Ops<T>::P* __restrict__ omf,
    const typename Ops<T>::P* __restrict__ omf_lo,
             const typename Ops<T>::P* __restrict__ omT, const float* __restrict__ dsrow,
             const float* __restrict__ gmx, int H, int L, int tpb, long long T_all, int G, float nscale,
             float s2, int grad_f32, void* __restrict__ dk, void* __restrict__ dv, float inv_sqrt_m, float eps) {
  using P = typename Ops<T>::P;
  using XS = typename BwdOps<T>::XS;
  using XB = typename BwdOps<T>::XB;
  constexpr int NW = BwdSplit<M>::NW, FB = BwdSplit<M>::FB;
  static_assert(FB % 2 == 0 || NW == 1, "an odd block count per wave only with a single wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NDB = D / 16;
  constexpr int NVB = DV / 16;
  constexpr int NFC = (M + 31) / 32;
  constexpr int BPWK = 2 * NDB / NW, BPWV = 2 * NVB / NW;  // dk^T and dV^T blocks per wave
  static_assert(BPWK >= 1 && (2 * NDB) % NW == 0 && BPWV >= 1 && (2 * NVB) % NW == 0,
                "gradient blocks split evenly over the waves");
  constexpr int NDBW = (BPWK + 1) / 2, NVBW = (BPWV + 1) / 2;
  constexpr int RC = Rows<DV>::RC, KC = Rows<DV>::KC;
  constexpr int KROW = D + 8;
  constexpr int WROW = RC + 8;
  constexpr int PROW = NFC * 32 + 8;
  constexpr int CPR = DV / 8;
  constexpr int IPT = (32 * CPR + NT - 1) / NT;
  using Rg = Ring<T, D, DV, NT, true>;
  __shared__ __attribute__((aligned(16))) unsigned char ring[2][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P ks[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  __shared__ __attribute__((aligned(16))) XS vsr[32 * WROW];
  __shared__ __attribute__((aligned(16))) XS prow[32 * PROW];
  __shared__ __attribute__((aligned(16))) XB frow[32 * PROW];
  __shared__ __attribute__((aligned(16))) float qmx[32][NW + 1];  // [key][wave], one padding column
  __shared__ __attribute__((aligned(16))) float rho[32][NW + 1];
  __shared__ __attribute__((aligned(16))) float vex[32];
  __shared__ float xch[NW];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  const long long t_beg = piece_start(pc, T_all, G), t_end = piece_start(pc + 1, T_all, G);
  if (t_beg >= t_end) return;
  const int n_tiles = (int)(t_end - t_beg);
  const uint32_t ring0 = lds_addr(&ring[0][0]);
  TileCursor cur(t_beg, tpb), ahead(t_beg, tpb);

  vec8<P> om[FB][DC];
  constexpr bool PSO = sizeof(P) == 2;  // the projections through Omega' hi + lo (fp16 fragments)
  vec8<P> oml[PSO ? FB : 1][PSO ? DC : 1];
  vec8<P> omt[NDBW][NFC];
  vec8<XS> da[FB][KC];
  vec8<XB> dt[NVBW][NFC];
  float eD = 0.f, gm = 0.f;
  int cur_bh = -1;
  // dk and dV blocks of the previous tile, scaled: stored one tile late (after the next
  // tile's first barriers), so the top of a tile does not wait for them
  constexpr int NBLK = BPWK + BPWV;
  f32x4 pend[NBLK];
  int pend_bh = -1, pend_tok0 = 0;
  auto store_pending = [&]() {
    if (pend_bh < 0) return;
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
      const bool isk = bi < BPWK;
      const int blk = isk ? w * BPWK + bi : w * BPWV + (bi - BPWK);
      const int cb = blk >> 1, tb = blk & 1;
      const int tok = pend_tok0 + tb * 16 + c;
      if (tok < L) {
        const int ncol = isk ? D : DV;
        void* dst = isk ? dk : dv;
        const size_t off = ((size_t)pend_bh * L + tok) * ncol + cb * 16 + 4 * g;
        if (grad_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + off) = pend[bi];
        } else {
          vec4<T> o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = to_t<T>(pend[bi][i]);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(dst) + off) = o4;
        }
      }
    }
  };

  Rg::issue(K, V, L, ahead.bh, ahead.tok0(), true, ring0);
  ahead.next();
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int bh = cur.bh, tok0 = cur.tok0();
    wait_vmcnt<0>();  // this tile's copies, and every store of the previous tile
    Rg::template convert<P, KROW, kNormSq>(ring[buf], ks[buf], kn[buf], nscale, L - tok0);
    if (it + 1 < n_tiles) {
      Rg::issue(K, V, L, ahead.bh, ahead.tok0(), true, ring0 + (buf ^ 1) * Rg::SLOT);
      ahead.next();
    }
    if (bh != cur_bh) {
      const int h = bh % H;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          {
            const size_t o_ = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
            om[fb][dc] = ld8<P>(omf + o_);
            if constexpr (PSO) oml[fb][dc] = ld8<P>(omf_lo + o_);
          }
#pragma unroll
      for (int i = 0; i < NDBW; ++i)
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc)
          omt[i][fc] = ld8<P>(omT + ((((size_t)h * NDB + (w * BPWK) / 2 + i) * NFC + fc) * 64 + lane) * 8);
      const float* rows = dsrow + (size_t)bh * M * RC;
      f32x8 sf[FB][KC];
      float amax = 0.f;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const int f = (w * FB + fb) * 16 + c;
          const f32x4* src = reinterpret_cast<const f32x4*>(rows + (size_t)f * RC + kc * 32 + 8 * g);
          const f32x4 a = src[0], b = src[1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            sf[fb][kc][j] = a[j];
            sf[fb][kc][j + 4] = b[j];
            amax = fmaxf(amax, fmaxf(fabsf(a[j]), fabsf(b[j])));
          }
        }
      // dS^T fragments for dV: A[m = value column][k = feature fc*32 + 8g + j], unscaled bf16
#pragma unroll
      for (int i = 0; i < NVBW; ++i)
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int f = fc * 32 + 8 * g + j;
            dt[i][fc][j] = to_t<XB>(f < M ? rows[(size_t)f * RC + ((w * BPWV) / 2 + i) * 16 + c] : 0.f);
          }
      gm = gmx[bh];
      eD = (float)(scale_exp(wg_absmax<NW>(amax, xch)) - 4);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
#pragma unroll
          for (int j = 0; j < 8; ++j) da[fb][kc][j] = to_t<XS>(ldexpf(sf[fb][kc][j], -(int)eD));
      wait_vmcnt<0>();  // every operand has landed (as in bwd_q_kernel)
      cur_bh = bh;
    }
    lds_barrier();  // ks, kn of this tile; every thread's copies landed

    // ---- projection and row maxima
    f32x4 pk[2][FB];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      vec8<P> kf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? ld8<P>(&ks[buf][(tb * 16 + c) * KROW + col]) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pk[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16_split_a<PSO>(pk[tb][fb], om[fb][dc], oml[PSO ? fb : 0][PSO ? dc : 0], kf[dc]);
      }
      if constexpr (KIND == kPrf) {
        float mx = -INFINITY;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pk[tb][fb][i]);
        mx = group_max(mx);
        if (g == 0) qmx[tb * 16 + c][w] = mx;
      }
    }
    // ---- [V 1] rows scaled per key to [1/2, 1) (fp16)
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int item = threadIdx.x + u * NT;
      const int row = item / CPR, c8 = item % CPR;
      float vals[8];
      float mabs = 0.f;
      const vec8<T> v8 = ld8<T>(reinterpret_cast<const T*>(ring[buf] + Rg::v_off(min(row, 31), c8 * 8)));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vals[j] = item < 32 * CPR ? to_f(v8[j]) : 0.f;
        mabs = fmaxf(mabs, fabsf(vals[j]));
      }
      mabs = lanes_max<CPR>(mabs);
      if (item < 32 * CPR) {
        const int ev = scale_exp(fmaxf(mabs, 1.f));
        vec8<XS> x8;
#pragma unroll
        for (int j = 0; j < 8; ++j) x8[j] = to_t<XS>(ldexpf(vals[j], -ev));
        *reinterpret_cast<vec8<XS>*>(&vsr[row * WROW + c8 * 8]) = x8;
        if (c8 == 0) {
          for (int col = DV; col < RC; ++col) vsr[row * WROW + col] = to_t<XS>(col == DV ? ldexpf(1.f, -ev) : 0.f);
          vex[row] = (float)ev;
        }
      }
    }
    lds_barrier();  // B1: row maxima, [V 1] rows
    store_pending();

    // ---- phi', dPhi_K, P, rho; P and phi' rows
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float mx = 0.f;
      if constexpr (KIND == kPrf) {
        mx = qmx[tb * 16 + c][0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, qmx[tb * 16 + c][ww]);
      }
      vec8<XS> vf[KC];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) vf[kc] = ld8<XS>(&vsr[(tb * 16 + c) * WROW + kc * 32 + 8 * g]);
      float r = 0.f;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma16(dp, da[fb][kc], vf[kc]);
        vec4<XS> p4;
        vec4<XB> f4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ph, pp;
          if constexpr (KIND == kPrf) {
            ph = fast_exp2(pk[tb][fb][i] - mx);
            pp = ph * dp[i];  // P = phi' * dPhi_K (scaled)
          } else {
            const float a = pk[tb][fb][i];
            ph = fmaxf(a, 0.f) * inv_sqrt_m + eps;
            pp = a > 0.f ? dp[i] : 0.f;  // P = 1[a > 0] * dPhi_K (scaled)
          }
          r += pp;
          p4[i] = to_t<XS>(pp);
          f4[i] = to_t<XB>(ph);
        }
        const int off = (tb * 16 + c) * PROW + (w * FB + fb) * 16 + 4 * g;
        *reinterpret_cast<vec4<XS>*>(&prow[off]) = p4;
        *reinterpret_cast<vec4<XB>*>(&frow[off]) = f4;
      }
      r = group_sum(r);
      if (g == 0) rho[tb * 16 + c][w] = r;
    }
    lds_barrier();  // B2: P and phi' rows, rho partials

    // ---- dk and dV blocks over all features, times the key's scale (stored later)
#pragma unroll
    for (int bi = 0; bi < NBLK; ++bi) {
      const bool isk = bi < BPWK;
      const int blk = isk ? w * BPWK + bi : w * BPWV + (bi - BPWK);
      const int cb = blk >> 1, tb = blk & 1;
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
      if (isk) {
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc) mma16(a, omt[bi >> 1][fc], ld8<XS>(&prow[(tb * 16 + c) * PROW + fc * 32 + 8 * g]));
      } else {
#pragma unroll
        for (int fc = 0; fc < NFC; ++fc)
          mma16(a, dt[(bi - BPWK) >> 1][fc], ld8<XB>(&frow[(tb * 16 + c) * PROW + fc * 32 + 8 * g]));
      }
      const int krow = tb * 16 + c;
      if constexpr (KIND != kPrf) {
        // ReLU: no key scale, no norm term
        a = a * (isk ? ldexpf(inv_sqrt_m, (int)(eD + vex[krow])) : 1.f);
        pend[bi] = a;
        continue;
      }
      float mx = qmx[krow][0];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, qmx[krow][ww]);
      const float lf = mx - kn[buf][krow] - gm;  // log2 of the key's scale F_j (keys past L: -inf)
      if (isk) {
        float rs = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) rs += rho[krow][ww];
        const float f = fast_exp2(lf + eD + vex[krow]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = f * (a[i] * (1.f / kLog2e) - s2 * to_f(ks[buf][krow * KROW + cb * 16 + 4 * g + i]) * rs);
      } else {
        a = a * fast_exp2(lf);
      }
      pend[bi] = a;
    }
    pend_bh = bh;
    pend_tok0 = tok0;
    cur.next();
  }
  store_pending();
}

// ---------------------------------------------------------------- host side
bool bwd_shape_built(int d, int dv, int m) {
#define X(D_, DV_, M_) \
  if (d == D_ && dv == DV_ && m == M_) return true;
  FAVOR_BWD_SHAPES(X)
#undef X
  return false;
}

constexpr int kBwdPieces = 256;  // one workgroup per CU (eight waves: two per SIMD)

BackwardPlan plan_backward(const Shape& s, int dtype) {
  BackwardPlan p;
  const BidirPlan f = plan_bidir(s, dtype);
  p.tpb = f.tpb;
  p.T_all = f.T_all;
  p.G_red = f.G;
  p.G = (int)std::min<long long>(p.T_all, kBwdPieces);
  p.nw_reduce = f.nw_reduce;
  const int dc = (s.d + 31) / 32;
  const size_t nfc = (s.m + 31) / 32;
  const size_t rc = ((s.dv + 1 + 31) / 32) * 32;
  const size_t slots_red = (size_t)p.G_red + (size_t)s.bh(), slots = (size_t)p.G + (size_t)s.bh();
  size_t off = 0;
  p.off_omf = off;
  off = align256(off + (size_t)s.H * (s.m / 16) * dc * 512 * elt(dtype));
  p.off_omlo = off;
  off = align256(off + (size_t)s.H * (s.m / 16) * dc * 512 * elt(dtype));
  p.off_omt = off;
  off = align256(off + (size_t)s.H * (s.d / 16) * nfc * 512 * elt(dtype));
  p.off_part = off;
  off = align256(off + slots_red * nfc * (s.dv / 16) * 512 * 4);
  p.off_zpart = off;
  off = align256(off + slots_red * nfc * 32 * 4);
  p.off_pmax = off;
  off = align256(off + slots_red * p.nw_reduce * 4);
  p.off_srow = off;
  off = align256(off + (size_t)s.bh() * s.m * rc * 4);
  p.off_gmax = off;
  off = align256(off + (size_t)s.bh() * 4);
  p.off_dpart = off;
  off = align256(off + slots * nfc * (s.dv / 16) * 512 * 4);
  p.off_dzpart = off;
  off = align256(off + slots * nfc * 32 * 4);
  p.off_dsrow = off;
  off = align256(off + (size_t)s.bh() * s.m * rc * 4);
  p.total = off;
  return p;
}

template <typename T, int D, int DV, int M, int KIND>
static hipError_t run_backward(const T* q, const T* k, const T* v, const float* omega, const T* dout,
                               const Shape& s, float eps, int grad_f32, void* dq, void* dk, void* dv, void* ws,
                               hipStream_t st) {
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  constexpr int NWR = RedSplit<M, D>::NW;
  constexpr int NWB = BwdSplit<M>::NW;
  const BackwardPlan p = plan_backward(s, sizeof(T) == 4 ? 0 : 1);
  char* base = static_cast<char*>(ws);
  P* omf = reinterpret_cast<P*>(base + p.off_omf);
  P* omlo = reinterpret_cast<P*>(base + p.off_omlo);
  P* omt = reinterpret_cast<P*>(base + p.off_omt);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* zpart = reinterpret_cast<float*>(base + p.off_zpart);
  float* pmax = reinterpret_cast<float*>(base + p.off_pmax);
  float* srow = reinterpret_cast<float*>(base + p.off_srow);
  float* gmx = reinterpret_cast<float*>(base + p.off_gmax);
  float* dpart = reinterpret_cast<float*>(base + p.off_dpart);
  float* dzpart = reinterpret_cast<float*>(base + p.off_dzpart);
  float* dsrow = reinterpret_cast<float*>(base + p.off_dsrow);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = KIND == kPrf ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)M);
  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  const long long nfragT = (long long)s.H * (D / 16) * ((M + 31) / 32) * 64;
  {
    launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st,
        omega, s.H, M, M, D, wscale, omf, 0);
    if constexpr (sizeof(P) == 2)
      launch("omega_frag", omega_frag_kernel<P>, (unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0,
          st, omega, s.H, M, M, D, wscale, omlo, 1);
    launch("omega_frag", omegaT_frag_kernel<P>, (unsigned)std::min<long long>((nfragT + 255) / 256, 4096), 256, 0, st,
        omega, s.H, M, D, wscale, omt);
  }
  {
    launch("reduce", kv_reduce_kernel<T, D, DV, M, 4, KIND, true, true>, p.G_red, 64 * NWR, 0, st, k, v, omf,
        omlo, s.H,
        s.L, p.tpb, p.T_all, p.G_red, eps, inv_sqrt_m, nscale, part, zpart, pmax, 0, 0, s.m, DV, DV);
  }
  {
    launch("combine", combine_rows_kernel<DV, M, NWR>, (unsigned)(s.bh() * ((M + 31) / 32)), 256, 0, st, part, zpart,
        pmax, p.tpb, p.T_all, p.G_red, KIND == kPrf ? 1 : 0, srow, gmx);
  }
  {
    launch("bwd_q", bwd_q_kernel<T, D, DV, M, KIND>, p.G, 64 * NWB, 0, st, q, dout, omf, omlo, omt, srow, s.H, s.L,
        p.tpb, p.T_all, p.G, grad_f32, dpart, dzpart, dq, inv_sqrt_m, eps);
  }
  {
    launch("combine_d", combine_rows_kernel<DV, M, NWB>, (unsigned)(s.bh() * ((M + 31) / 32)), 256, 0, st, dpart,
        dzpart, nullptr, p.tpb, p.T_all, p.G, 0, dsrow, nullptr);
  }
  {
    launch("bwd_k", bwd_k_kernel<T, D, DV, M, KIND>, p.G, 64 * NWB, 0, st, k, v, omf, omlo, omt, dsrow, gmx, s.H, s.L,
        p.tpb, p.T_all, p.G, nscale, sc * sc, grad_f32, dk, dv, inv_sqrt_m, eps);
  }
  return hipGetLastError();
}

template <typename T, int D, int DV, int M>
static hipError_t run_backward_kind(const void* q, const void* k, const void* v, const float* omega, const void* dout,
                                    const Shape& s, int kind, float eps, int grad_f32, void* dq, void* dk, void* dv,
                                    void* ws, hipStream_t st) {
  const T* q_ = static_cast<const T*>(q);
  const T* k_ = static_cast<const T*>(k);
  const T* v_ = static_cast<const T*>(v);
  const T* o_ = static_cast<const T*>(dout);
  if (kind == kPrf) return run_backward<T, D, DV, M, kPrf>(q_, k_, v_, omega, o_, s, eps, grad_f32, dq, dk, dv, ws, st);
  if (kind == kRelu) return run_backward<T, D, DV, M, kRelu>(q_, k_, v_, omega, o_, s, eps, grad_f32, dq, dk, dv, ws, st);
  return hipErrorInvalidValue;
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* omega, const void* dout,
                           const Shape& s, int dtype, int kind, float eps, int grad_f32, void* dq, void* dk, void* dv,
                           void* ws, hipStream_t st) {
#define X(D_, DV_, M_)                                                                                           \
  if (s.d == D_ && s.dv == DV_ && s.m == M_) {                                                                   \
    if (dtype == 0) return run_backward_kind<float, D_, DV_, M_>(q, k, v, omega, dout, s, kind, eps, grad_f32, dq, \
                                                                 dk, dv, ws, st);                                 \
    return run_backward_kind<bf16, D_, DV_, M_>(q, k, v, omega, dout, s, kind, eps, grad_f32, dq, dk, dv, ws, st); \
  }
  FAVOR_BWD_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace favor
