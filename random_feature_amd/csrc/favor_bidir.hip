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
#include "favor_timing.hpp"

#include <algorithm>
#include <cmath>

namespace favor {

// Waves per workgroup and 16-feature blocks per wave for m features.
template <int M> struct FeatSplit {
  static constexpr int NW = (M / 16) < 4 ? (M / 16) : 4;
  static constexpr int FB = M / (16 * NW);
};
// Waves of the key/value reduction (RW_MAX at most, 32 features per wave or more). Two
// workgroups per CU: NW/2 waves per SIMD (the second launch bound is waves per EU).
#ifndef FAVOR_REDUCE_WAVES
#define FAVOR_REDUCE_WAVES 4
#endif
template <int M> struct RedSplit {
  static constexpr int RW_MAX = FAVOR_REDUCE_WAVES;
  static constexpr int NW = M < 32 ? 1 : ((M / 32) < RW_MAX ? (M / 32) : RW_MAX);
  static constexpr int FB = M / (16 * NW);
};

constexpr int kNormNone = 0, kNormSq = 1, kNormAbs = 2;

// ---------------------------------------------------------------- tile ring
// 32-token tiles of X (keys or queries) and V arrive in an R-slot LDS ring through
// asynchronous 16-byte copies issued R-1 tiles ahead. Chunk q of a slot (16 bytes) is
// copied by thread q mod NT, so every thread can convert the chunks it copied itself as
// soon as its own copies have landed. X chunks come first (row-major); V chunks follow,
// row-major with the chunk column XOR-swizzled by the row for 16-bit types (spreads the
// transposing reads over the LDS banks). Rows past L are copied from row L-1 and masked
// by the consumer; slots past the end of a piece are filled with harmless copies so that
// every tile costs the same number of copies and the waits stay uniform.
template <typename T, int D, int DV, int NT, bool WITH_V>
struct Ring {
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int CPR_X = D / EPC;
  static constexpr int CPR_V = WITH_V ? DV / EPC : 1;
  static constexpr int XC = 32 * CPR_X;
  static constexpr int VC = WITH_V ? 32 * CPR_V : 0;
  static constexpr int CPT = (XC + VC + NT - 1) / NT;
  static constexpr int SLOT = CPT * NT * 16;
  static constexpr bool SWZ = sizeof(T) == 2 && WITH_V;

  // copies of the tile at (bh, tok0) into the slot at LDS byte address `slot`; !live: filler
  static __device__ __forceinline__ void issue(const T* X, const T* V, int L, int bh, int tok0, bool live,
                                               uint32_t slot) {
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t rowbase = (size_t)bh * L;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + tid;
      const void* src = X;
      if (live) {
        if ((XC % NT == 0) ? (u * NT < XC) : (q < XC)) {
          const int row = q / CPR_X, cc = q % CPR_X;
          src = X + (rowbase + min(tok0 + row, L - 1)) * D + cc * EPC;
        } else if (WITH_V && q < XC + VC) {
          const int p = q - XC, row = p / CPR_V, pc = p % CPR_V;
          const int cc = SWZ ? (pc ^ (row & (CPR_V - 1))) : pc;
          src = V + (rowbase + min(tok0 + row, L - 1)) * DV + cc * EPC;
        }
      }
      lds_dma16(src, slot + (uint32_t)(u * NT + w * 64) * 16u);
    }
  }

  // byte offset of V element (row, col) inside a slot
  static __device__ __forceinline__ int v_off(int row, int col) {
    const int cc = col / EPC, within = col % EPC;
    const int pc = SWZ ? (cc ^ (row & (CPR_V - 1))) : cc;
    return (XC + row * CPR_V + pc) * 16 + within * (int)sizeof(T);
  }

  // this thread's X chunks of a landed slot -> projection type in `conv` (row stride KROW),
  // and per row into `nrm`: NORM == kNormSq: |x|^2 * nscale (+inf for rows at or past
  // nvalid); NORM == kNormAbs: |x| * nscale
  template <typename P, int KROW, int NORM>
  static __device__ __forceinline__ void convert(const unsigned char* slot, P* conv, float* nrm, float nscale,
                                                 int nvalid) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + threadIdx.x;
      if (u * NT >= XC) break;  // no X chunks left (known at compile time)
      const int row = q / CPR_X, cc = q % CPR_X;
      float s2 = 0.f;
      const bool has = (XC % NT == 0) || q < XC;  // every thread has a chunk when XC % NT == 0
      if (has) {
        if constexpr (sizeof(T) == 2) {
          const vec8<T> x = *reinterpret_cast<const vec8<T>*>(slot + q * 16);
          vec8<P> y;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float f = to_f(x[j]);
            s2 += f * f;
            y[j] = to_t<P>(f);
          }
          *reinterpret_cast<vec8<P>*>(conv + row * KROW + cc * 8) = y;
        } else {
          const f32x4 x = *reinterpret_cast<const f32x4*>(slot + q * 16);
          vec4<P> y;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s2 += x[j] * x[j];
            y[j] = to_t<P>(x[j]);
          }
          *reinterpret_cast<vec4<P>*>(conv + row * KROW + cc * 4) = y;
        }
      }
      if constexpr (NORM != kNormNone) {
        s2 = lanes_sum<CPR_X>(s2);  // the CPR_X chunks of a row sit on consecutive lanes
        if (has) {  // every lane of the row holds the sum and stores the same value
          if constexpr (NORM == kNormSq)
            nrm[row] = row < nvalid ? s2 * nscale : INFINITY;
          else
            nrm[row] = __builtin_sqrtf(s2) * nscale;
        }
      }
    }
  }
};

// Walks the flattened tile index space as (b*h, token offset) without divisions.
struct TileCursor {
  int bh, tt, tpb;
  __device__ __forceinline__ TileCursor(long long t, int tpb_) : bh((int)(t / tpb_)), tt((int)(t % tpb_)), tpb(tpb_) {}
  __device__ __forceinline__ void next() {
    if (++tt == tpb) {
      tt = 0;
      ++bh;
    }
  }
  __device__ __forceinline__ int tok0() const { return tt * 32; }
};

// B fragments of [V 1] for the contraction over tokens (paired token slots) straight from
// the raw V rows of a slot; the last block is the ones column (z).
template <typename T, int D, int DV, int NT>
__device__ __forceinline__ void value_frags(const unsigned char* slot, vec8<typename Ops<T>::C> (&vf)[DV / 16 + 1],
                                            int c, int g) {
  using C = typename Ops<T>::C;
  using Rg = Ring<T, D, DV, NT, true>;
  constexpr int NB = DV / 16 + 1;
#pragma unroll
  for (int nb = 0; nb < NB - 1; ++nb) {
    if constexpr (sizeof(T) == 2) {
      // lane c of group g addresses 4 elements of row 4g + c/4 at column nb*16 + 4(c%4); the
      // transposing read hands lane c the column nb*16 + c of rows 4g..4g+3 (then +16)
      const int row = 4 * g + (c >> 2), col = nb * 16 + 4 * (c & 3);
      const bf16x4 lo = lds_read_tr4(reinterpret_cast<const bf16*>(slot + Rg::v_off(row, col)));
      const bf16x4 hi = lds_read_tr4(reinterpret_cast<const bf16*>(slot + Rg::v_off(row + 16, col)));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[nb][j] = lo[j];
        vf[nb][j + 4] = hi[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 16 * (j >> 2) + 4 * g + (j & 3);
        vf[nb][j] = *reinterpret_cast<const float*>(slot + Rg::v_off(row, nb * 16 + c));
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) vf[NB - 1][j] = to_t<C>(c == 0 ? 1.f : 0.f);
}

// ---------------------------------------------------------------- K/V reduction
// Workgroup = NW waves over one piece of the flattened tile space; wave w owns FB*16
// features. Per tile every wave
//   projects    A = K tile (rows = tokens, linear d slots), B = Omega' fragments; the
//               accumulators start at -(n'_t + M) (n'_t = log2e |x_t|^2/2, M the wave's
//               running key maximum) so the MFMA output is already the stabilised exponent
//   stabilises  if the tile maximum exceeds 0 (or on the first tile of a (b,h)), shift M
//               to kKeyMargin above it and rescale the accumulated S_aug by the same
//               power of two
//   maps        Phi = exp2(.) (ReLU: max(a,0)/sqrt(m) + eps), rounded to the contraction type
//   contracts   S_aug += Phi^T [V 1]: A = Phi^T (paired token slots, the accumulators as
//               they are), B = the value fragments
// The projection runs one tile ahead, and each iteration is two stretches in which matrix
// and vector work of different tiles are independent: the projection MFMAs of tile t+1 run
// beside the exponentials of tile t, the contraction MFMAs of tile t beside the conversion
// of the K rows of tile t+2 and the next copies. The stabiliser of tile t (whose projection
// is complete) comes first, so tile t+1 is projected against the current maximum. Tiles
// stream through an R-slot asynchronous ring R-1 ahead; two K buffers; one barrier per tile.
// Headroom (log2 units) the key stabiliser leaves below its running maximum: the largest
// feature after a shift is 2^-8, far above the bottom of the fp32/bf16 range.
constexpr float kKeyMargin = 8.f;

template <typename T, int D, int DV, int M, int R, int KIND>
__global__ void __launch_bounds__(64 * RedSplit<M>::NW, RedSplit<M>::NW < 2 ? 1 : RedSplit<M>::NW / 2)
kv_reduce_kernel(const T* __restrict__ K, const T* __restrict__ V, const typename Ops<T>::P* __restrict__ omf,
                 int H, int L, int tpb, long long T_all, int G, float eps, float inv_sqrt_m, float nscale,
                 float* __restrict__ part, float* __restrict__ zpart, float* __restrict__ pmax) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = RedSplit<M>::NW, FB = RedSplit<M>::FB;
  constexpr int NFC = (M + 31) / 32;
  static_assert(FB % 2 == 0 || NW == 1, "an odd block count per wave only with a single wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;  // value-column blocks + the ones column (z = Phi^T 1)
  constexpr int KROW = D + 8;
  static_assert(R >= 4, "ring: the tile contracted, one converted ahead, one being converted, one in flight");
  using Rg = Ring<T, D, DV, NT, true>;
  // at the wait of iteration t the copies issued so far reach tile t+R-2 (each iteration
  // issues at its end): R-4 tiles are newer than tile t+2
  constexpr int WAIT_NEXT = Rg::CPT * (R - 4);
  __shared__ __attribute__((aligned(16))) unsigned char ring[R][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P ks[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float kn[2][32];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  const long long t_beg = piece_start(pc, T_all, G), t_end = piece_start(pc + 1, T_all, G);
  if (t_beg >= t_end) return;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  f32x4 sacc[FB][NB];
  float runmax = 0.f;
  bool first = true;
  vec8<P> om[FB][DC];

  // one (b,h)'s sums of this piece, as fp32 A fragments of S^T (the layout of sfr):
  // part[slot][fc][nb][lane][j], the z column compacted to zpart[slot][fc][g][j] (lanes c = 0)
  auto flush = [&](int fbh, float fmax) {
    const size_t slot = (size_t)pc + fbh;
#pragma unroll
    for (int p = 0; p < (FB + 1) / 2; ++p) {
      const int fc = (w * FB) / 2 + p;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 lo = sacc[2 * p][nb], hi = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FB % 2 == 0) hi = sacc[2 * p + 1][nb];
        float* dst;
        if (nb < NB - 1)
          dst = part + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8;
        else
          dst = zpart + ((slot * NFC + fc) * 4 + g) * 8;
        if (nb < NB - 1 || c == 0) {
          reinterpret_cast<f32x4*>(dst)[0] = lo;
          reinterpret_cast<f32x4*>(dst)[1] = hi;
        }
      }
    }
    if (lane == 0) pmax[slot * NW + w] = fmax;
  };
  auto zero_sums = [&]() {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto load_om = [&](int bh) {
    const int h = bh % H;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        om[fb][dc] = ld8<P>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);
    wait_vmcnt<0>();  // settle the fragment (and any partial) traffic here, off the per-tile path
  };
  // projection of the converted tile in ks[kb], exponents relative to the running maximum rm
  auto project = [&](f32x4 (&pa)[2][FB], int kb, float rm) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 bias = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KIND == kPrf) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[kb][tb * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[i] = -(n4[i] + rm);
      }
      vec8<P> kf[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const int col = dc * 32 + 8 * g;
        kf[dc] = (col < D) ? ld8<P>(&ks[kb][(tb * 16 + c) * KROW + col]) : zero8<P>();
      }
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        pa[tb][fb] = bias;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(pa[tb][fb], kf[dc], om[fb][dc]);
      }
    }
  };

  const int n_tiles = (int)(t_end - t_beg);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb), cv(t_beg, tpb);
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    Rg::issue(K, V, L, ahead.bh, ahead.tok0(), s < n_tiles, ring0 + s * Rg::SLOT);
    if (s < n_tiles) ahead.next();
  }
  // tiles 0 and 1 converted up front; iteration t converts tile t+2
  wait_vmcnt<Rg::CPT * (R - 2)>();
  Rg::template convert<P, KROW, kNormSq>(ring[0], ks[0], kn[0], nscale, L - cv.tok0());
  cv.next();
  wait_vmcnt<Rg::CPT * (R - 3)>();
  Rg::template convert<P, KROW, kNormSq>(ring[1], ks[1], kn[1], nscale, L - cv.tok0());
  cv.next();
  int cur_bh = cur.bh;
  load_om(cur_bh);
  lds_barrier();
  zero_sums();
  f32x4 pa0[2][FB], pa1[2][FB];  // projections of tile t and t+1, alternating roles
  project(pa0, 0, 0.f);
  lds_barrier();  // every wave has read ks[0] before iteration 0 converts tile 2 into it

  int s_iss = R - 1;  // ring slot of the next copy:  (t + R - 1) mod R
  int s_cur = 0;      // ring slot of tile t
  int s_cv = 2 % R;   // ring slot of tile t + 2
  int flush_bh = -1;  // (b,h) whose partial is written at the top of the next iteration
  float flush_max = 0.f;
  int it = 0;

  auto step = [&](f32x4 (&pcur)[2][FB], f32x4 (&pnext)[2][FB]) {
    const int buf = it & 1;
    const int tok0 = cur.tok0();
    if (flush_bh >= 0) {
      // tile t opened a new (b,h); the old one's sums closed with the previous contraction
      flush(flush_bh, flush_max);
      zero_sums();
      flush_bh = -1;
      wait_vmcnt<0>();  // no stores may stay in flight under the partial waits of the ring
    }
    // stabiliser of tile t (its projection is complete)
    if constexpr (KIND == kPrf) {
      float lmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, pcur[tb][fb][i]);
      // the running maximum moves only if some exponent is positive (or on a new (b,h))
      // it moves kKeyMargin past the tile maximum, so later tiles seldom move it again
      if (first || __builtin_amdgcn_ballot_w64(lmax > 0.f) != 0) {
        const float shift = wave_max(lmax) + kKeyMargin;
        if (!first) {
          const float sc = fast_exp2(-shift);
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] *= sc;
        }
        runmax = first ? shift : runmax + shift;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int fb = 0; fb < FB; ++fb) pcur[tb][fb] -= shift;
        first = false;
      }
    }
    TileCursor nx = cur;
    nx.next();
    const bool more = it + 1 < n_tiles;
    const bool next_new = more && nx.bh != cur_bh;
    if (next_new) load_om(nx.bh);  // Omega' of tile t+1's head (tile t's projection is done)
    wait_vmcnt<WAIT_NEXT>();

    // stretch 1: projection of tile t+1 beside the feature map of tile t
    project(pnext, buf ^ 1, next_new ? 0.f : runmax);
    vec8<C> af[FB];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = pcur[j >> 2][fb][j & 3];
        float f;
        if constexpr (KIND == kPrf) {
          f = fast_exp2(a);  // rows past L carry an infinite norm: exp2(-inf) = 0
        } else {
          const bool ok = tok0 + 16 * (j >> 2) + 4 * g + (j & 3) < L;
          f = ok ? fmaxf(a, 0.f) * inv_sqrt_m + eps : 0.f;
        }
        af[fb][j] = to_t<C>(f);
      }
    // stretch 2: contraction of tile t beside the conversion of tile t+2 (past the end of
    // the piece: a filler slot into an unused buffer) and the next copies
    vec8<C> vf[NB];
    value_frags<T, D, DV, NT>(ring[s_cur], vf, c, g);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma16(sacc[fb][nb], af[fb], vf[nb]);
    Rg::template convert<P, KROW, kNormSq>(ring[s_cv], ks[buf], kn[buf], nscale, L - cv.tok0());
    cv.next();
    {
      const bool live = it + R - 1 < n_tiles;
      Rg::issue(K, V, L, ahead.bh, ahead.tok0(), live, ring0 + s_iss * Rg::SLOT);
      if (live) ahead.next();
    }
    lds_barrier();

    if (next_new) {
      flush_bh = cur_bh;
      flush_max = runmax;
      cur_bh = nx.bh;
      first = true;
    }
    cur = nx;
    s_iss = s_iss + 1 == R ? 0 : s_iss + 1;
    s_cur = s_cur + 1 == R ? 0 : s_cur + 1;
    s_cv = s_cv + 1 == R ? 0 : s_cv + 1;
    ++it;
  };
  while (it + 1 < n_tiles) {
    step(pa0, pa1);
    step(pa1, pa0);
  }
  if (it < n_tiles) step(pa0, pa1);
  flush(cur_bh, runmax);
}

// ---------------------------------------------------------------- combine
// One workgroup per (b*h, 32-feature chunk), one thread per (value block, lane): the
// partials of the pieces of that (b,h), already in fragment layout, scaled by
// 2^(M_piece,wave - M_max) and summed, give the A fragments of S_aug^T:
// sfr[bh][fc][nb][lane][j] = S_aug[fc*32 + 16(j>>2) + 4g + (j&3)][nb*16 + c]; in the last
// block only row c == 0 (the z column) is nonzero.
template <typename C, int DV, int M>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ part, const float* __restrict__ zpart, const float* __restrict__ pmax,
               int tpb, long long T_all, int G, int kind, C* __restrict__ sfr) {
  constexpr int NW = RedSplit<M>::NW, FB = RedSplit<M>::FB;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (M + 31) / 32;
  const int bh = blockIdx.x / NFC, fc = blockIdx.x % NFC;
  const long long i_lo = piece_of((long long)bh * tpb, T_all, G);
  const long long i_hi = piece_of((long long)(bh + 1) * tpb - 1, T_all, G);
  const int np = (int)(i_hi - i_lo + 1);
  const int wv = (fc * 32) / (FB * 16);  // the reducing wave that owned this chunk
  float gmax = -INFINITY;
  if (kind == kPrf)
    for (int k = 0; k < np * NW; ++k) gmax = fmaxf(gmax, pmax[(size_t)(i_lo + k / NW + bh) * NW + k % NW]);
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
          sc[j] = k0 + j < np ? ((kind == kPrf) ? fast_exp2(pmax[slot * NW + wv] - gmax) : 1.f) : 0.f;
          const float* src = (nb < NB - 1) ? part + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8
                                           : zpart + ((slot * NFC + fc) * 4 + g) * 8;
          pl[j] = reinterpret_cast<const f32x4*>(src)[0];
          ph[j] = reinterpret_cast<const f32x4*>(src)[1];
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
// Exponent bound (log2 units) under which the bound stabiliser keeps every query feature
// a normal float: the features lie in [2^(-2 bound), 1].
constexpr float kQueryBoundLimit = 60.f;

// Workgroup = NW waves over one piece of the flattened tile space. Per 32-token tile:
//   phase 1 (wave w, its FB*16 features, Omega' fragments in registers)
//     projection  A = Omega' (rows = features), B = Q^T (linear d slots) -> [feature][token];
//                 the accumulators start at -b_t, b_t = omax |q_t| >= max_r a'_r (omax the
//                 largest row norm of the rounded Omega' of the head), so the output is
//                 already a non-positive exponent (the |q|^2 term of the map and any
//                 constant per row cancel in the ratio). If some row of the tile has
//                 b_t > kQueryBoundLimit, the tile takes the exact row maximum across the
//                 waves instead (one more barrier).
//     feature map Phi = exp2(.) (ReLU: max(a,0)/sqrt(m) + eps); the accumulator pairs are
//                 B operands of the contraction as they stand (paired feature slots) and go
//                 to LDS; the wave's share of the denominator z^T Phi^T goes with them
//   every thread then lands, converts and norms its own chunk of tile t+1 and copies its
//   chunk of tile t+2 into the two-slot ring (all its memory traffic, stores included, has
//   settled at that point, so one full wait covers it)
//   barrier
//   phase 2 (wave w: a token half and value-column blocks, or both halves and fewer blocks)
//     contraction out^T block = S^T block (A, registers) x Phi^T (B, all features from LDS)
//     division by the summed denominators and the store
template <typename T, int D, int DV, int M, int KIND>
__global__ void __launch_bounds__(64 * FeatSplit<M>::NW, 2)
q_output_kernel(const T* __restrict__ Q, const typename Ops<T>::P* __restrict__ omf,
                const typename Ops<T>::C* __restrict__ sfr, int H, int L, int tpb, long long T_all, int G,
                float eps, float inv_sqrt_m, int out_f32, void* __restrict__ out) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M>::NW, FB = FeatSplit<M>::FB;
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;           // blocks of S_aug^T in sfr: values, then z
  constexpr int NVB = DV / 16;              // value-column blocks
  // phase 2 split: with TBS wave w takes token half w & 1 and value blocks (w >> 1) + j*NW/2
  // (half the LDS reads of the features, twice the S fragments); else both halves and
  // blocks w + j*NW
  constexpr int SF_REGS = sizeof(typename Ops<T>::C) == 2 ? 4 : 8;
  constexpr int NWH = NW / 2 > 0 ? NW / 2 : 1;
  constexpr bool TBS = NW >= 2 && ((NVB + NWH - 1) / NWH) * ((M + 31) / 32) * SF_REGS <= 64;
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
  constexpr float kMargin = 1.f + 1.f / 512.f;  // rounding of q to the projection type and of the MFMA sums

  const uint32_t ring0 = lds_addr(&ring[0][0]);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb);
  // prologue: tiles 0 and 1 in flight, tile 0 converted
  Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), true, ring0);
  ahead.next();
  Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), n_tiles > 1, ring0 + Rg::SLOT);
  if (n_tiles > 1) ahead.next();
  wait_vmcnt<Rg::CPT>();
  Rg::template convert<P, KROW, kNormAbs>(ring[0], qs[0], qb[0], kMargin, L);
  lds_barrier();

  vec8<P> om[FB][DC];
  vec8<C> zf[NFCW];
  vec8<C> sf[NCB][NFC];
  float omax = 0.f;
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
      if constexpr (KIND == kPrf) {
        // largest row norm of this head's rounded Omega': the wave's rows, then across waves
        float n2 = 0.f;
#pragma unroll
        for (int fb = 0; fb < FB; ++fb) {
          float s2 = 0.f;
#pragma unroll
          for (int dc = 0; dc < DC; ++dc)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float x = to_f(om[fb][dc][j]);
              s2 += x * x;
            }
          n2 = fmaxf(n2, group_sum(s2));
        }
        n2 = wave_max(n2);
        if (lane == 0) qmx[w][0] = n2;
        lds_barrier();
        float m2 = qmx[0][0];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) m2 = fmaxf(m2, qmx[ww][0]);
        omax = __builtin_sqrtf(m2);
        lds_barrier();  // qmx is reused by the exact-maximum path
      } else {
        wait_vmcnt<0>();
      }
    }

    // ---- phase 1: this wave's features of the tile
    f32x4 bias[2];
    bool exact = false;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float b = (KIND == kPrf) ? qb[buf][tb * 16 + c] * omax : 0.f;
      bias[tb] = f32x4{-b, -b, -b, -b};
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
        }
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = fast_exp2(pacc[tb][fb][i]);
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
    Rg::template convert<P, KROW, kNormAbs>(ring[buf ^ 1], qs[buf ^ 1], qb[buf ^ 1], kMargin, L);
    {
      const bool live = it + 2 < n_tiles;
      Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), live, ring0 + buf * Rg::SLOT);
      if (live) ahead.next();
    }
    lds_barrier();

    // ---- phase 2: this wave's value columns over all features
    float rden[NTB];
#pragma unroll
    for (int tt = 0; tt < NTB; ++tt) {
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) den += dpart[buf][tb0 + tt][c][ww];
      rden[tt] = 1.0f / den;
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
      if (nb < NVB) {
#pragma unroll
        for (int tt = 0; tt < NTB; ++tt) {
          const int tok = tok0 + (tb0 + tt) * 16 + c;
          if (tok < L) {
            const f32x4 o = acc[cb][tt] * rden[tt];
            const size_t off = ((size_t)bh * L + tok) * DV + nb * 16 + 4 * g;
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
// entry 1/sqrt(m)) and the per-row log scale. Omega' fragments are built in LDS from the
// fp32 matrix by the workgroup itself.
template <typename T, int D, int M>
__global__ void __launch_bounds__(256)
features_kernel(const T* __restrict__ X, const float* __restrict__ omega, int H, int L, int kind, float eps,
                float inv_sqrt_m, float wscale, float nscale_ln, float* __restrict__ phi,
                float* __restrict__ logscale, int tok_per_wg, int n_tiles) {
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  constexpr int NFB = M / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  P* oms = reinterpret_cast<P*>(smem);
  const int bh = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  for (int id = threadIdx.x; id < NFB * DC * 64; id += 256) {
    const int l = id & 63, dc = (id >> 6) % DC, fb = (id >> 6) / DC;
    const int lc = l & 15, lg = l >> 4;
    const float* row = omega + ((size_t)h * M + fb * 16 + lc) * D;
    vec8<P> x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = dc * 32 + 8 * lg + j;
      x[j] = to_t<P>(col < D ? row[col] * wscale : 0.f);
    }
    st8<P>(oms + (size_t)id * 8, x);
  }
  __syncthreads();
  const T* Xb = X + (size_t)bh * L * D;
  const int tstart = tile * tok_per_wg, tstop = min(L, tstart + tok_per_wg);
  for (int t0 = tstart + w * 16; t0 < tstop; t0 += 64) {
    const int tok = t0 + c;
    vec8<P> xf[DC];
    float s2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const int col = dc * 32 + 8 * g;
      const vec8<T> raw = (tok < L && col < D) ? ld8<T>(Xb + (size_t)tok * D + col) : zero8<T>();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = to_f(raw[j]);
        s2 += v * v;
        xf[dc][j] = to_t<P>(v);
      }
    }
    s2 = group_sum(s2);
    f32x4 pacc[NFB];
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {
      pacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) mma16(pacc[fb], ld8<P>(oms + ((fb * DC + dc) * 64 + lane) * 8), xf[dc]);
    }
    float ls = 0.f;
    if (kind == kPrf) {
      float mx = -INFINITY;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, pacc[fb][i]);
      mx = group_max(mx);
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pacc[fb][i] = fast_exp2(pacc[fb][i] - mx) * inv_sqrt_m;
      ls = mx * kLn2 - s2 * nscale_ln;
    } else {
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pacc[fb][i] = fmaxf(pacc[fb][i], 0.f) * inv_sqrt_m + eps;
    }
    if (tok < L) {
      float* prow = phi + ((size_t)bh * L + tok) * M;
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) *reinterpret_cast<f32x4*>(prow + fb * 16 + 4 * g) = pacc[fb];
      if (g == 0) logscale[(size_t)bh * L + tok] = ls;
    }
  }
}

// ---------------------------------------------------------------- host side

bool shape_built(int dtype, int d, int dv, int m) {
  (void)dtype;
#define X(D_, DV_, M_) \
  if (d == D_ && dv == DV_ && m == M_) return true;
  FAVOR_SHAPES(X)
#undef X
  return false;
}

static inline int fb_for(int m) { return std::min(4, m / 16); }
static inline int nw_for(int m) { return m / (16 * fb_for(m)); }
static inline int nw_split(int m) { return m < 32 ? 1 : std::min(FAVOR_REDUCE_WAVES, m / 32); }  // RedSplit<M>::NW
static inline size_t elt(int dtype) { return dtype == 0 ? 4 : 2; }
constexpr int kMaxPieces = 512;  // two resident 4-wave workgroups on each of 256 CUs
constexpr int kRing = 5;         // LDS ring slots of the key/value reduction

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

BidirPlan plan_bidir(const Shape& s, int dtype) {
  BidirPlan p;
  p.tpb = (s.L + 31) / 32;
  p.T_all = s.bh() * p.tpb;
  p.G = (int)std::min<long long>(p.T_all, kMaxPieces);
  p.nw_reduce = nw_split(s.m);
  const int dc = (s.d + 31) / 32, nb = s.dv / 16 + 1;
  const size_t slots = (size_t)p.G + (size_t)s.bh();
  size_t off = 0;
  p.off_omf = off;
  off = align256(off + (size_t)s.H * (s.m / 16) * dc * 512 * elt(dtype));
  const size_t nfc = (s.m + 31) / 32;
  p.off_part = off;
  off = align256(off + slots * nfc * (s.dv / 16) * 512 * 4);
  p.off_zpart = off;
  off = align256(off + slots * nfc * 32 * 4);
  p.off_pmax = off;
  off = align256(off + slots * p.nw_reduce * 4);
  p.off_sfr = off;
  off = align256(off + (size_t)s.bh() * ((s.m + 31) / 32) * nb * 512 * elt(dtype));
  p.total = off;
  return p;
}

CausalPlan plan_causal(const Shape& s, int dtype) {
  CausalPlan p;
  segmenting(s, p.nseg, p.seg_len);
  p.nw_reduce = nw_for(s.m);
  const int dc = (s.d + 31) / 32;
  size_t off = 0;
  p.off_omf = off;
  off = align256(off + (size_t)s.H * (s.m / 16) * dc * 512 * elt(dtype));
  p.off_part = off;
  off = align256(off + (size_t)s.bh() * p.nseg * s.m * (s.dv + 1) * 4);
  p.off_pmax = off;
  off = align256(off + (size_t)s.bh() * p.nseg * p.nw_reduce * 4);
  p.off_carry = off;
  off = align256(off + (size_t)s.bh() * p.nseg * s.m * (s.dv + 1) * 4);
  p.off_cmax = off;
  off = align256(off + (size_t)s.bh() * p.nseg * 4);
  p.total = off;
  return p;
}

template <typename T, int D, int DV, int M>
static hipError_t run_bidir(const T* q, const T* k, const T* v, const float* omega, const Shape& s, int kind,
                            float eps, int out_f32, void* out, void* ws, hipStream_t st) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M>::NW;
  constexpr int DC = (D + 31) / 32;
  const BidirPlan p = plan_bidir(s, sizeof(T) == 4 ? 0 : 1);
  char* base = static_cast<char*>(ws);
  P* omf = reinterpret_cast<P*>(base + p.off_omf);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  float* zpart = reinterpret_cast<float*>(base + p.off_zpart);
  float* pmax = reinterpret_cast<float*>(base + p.off_pmax);
  C* sfr = reinterpret_cast<C*>(base + p.off_sfr);
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = (kind == kPrf) ? sc * kLog2e : sc;
  const float nscale = sc * sc * kLog2e * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)M);

  const long long nfrag = (long long)s.H * (M / 16) * DC * 64;
  {
    FAVOR_TIMED("omega_frag", st);
    omega_frag_kernel<P><<<(unsigned)std::min<long long>((nfrag + 255) / 256, 4096), 256, 0, st>>>(
        omega, s.H, M, D, wscale, omf);
  }
  {
    FAVOR_TIMED("reduce", st);
    constexpr int NWR = RedSplit<M>::NW;
    if (kind == kPrf)
      kv_reduce_kernel<T, D, DV, M, kRing, kPrf><<<p.G, 64 * NWR, 0, st>>>(k, v, omf, s.H, s.L, p.tpb, p.T_all, p.G, eps,
                                                                        inv_sqrt_m, nscale, part, zpart, pmax);
    else
      kv_reduce_kernel<T, D, DV, M, kRing, kRelu><<<p.G, 64 * NWR, 0, st>>>(k, v, omf, s.H, s.L, p.tpb, p.T_all, p.G,
                                                                         eps, inv_sqrt_m, nscale, part, zpart, pmax);
  }
  {
    FAVOR_TIMED("combine", st);
    combine_kernel<C, DV, M><<<(unsigned)(s.bh() * ((M + 31) / 32)), 256, 0, st>>>(
        part, zpart, pmax, p.tpb, p.T_all, p.G, kind, sfr);
  }
  {
    FAVOR_TIMED("output", st);
    if (kind == kPrf)
      q_output_kernel<T, D, DV, M, kPrf><<<p.G, 64 * NW, 0, st>>>(q, omf, sfr, s.H, s.L, p.tpb, p.T_all, p.G, eps,
                                                                inv_sqrt_m, out_f32, out);
    else
      q_output_kernel<T, D, DV, M, kRelu><<<p.G, 64 * NW, 0, st>>>(q, omf, sfr, s.H, s.L, p.tpb, p.T_all, p.G, eps,
                                                                 inv_sqrt_m, out_f32, out);
  }
  return hipGetLastError();
}

hipError_t launch_bidir(const void* q, const void* k, const void* v, const float* omega, const Shape& s,
                        int dtype, int kind, float eps, int out_f32, void* out, void* ws, hipStream_t st) {
#define X(D_, DV_, M_)                                                                                         \
  if (s.d == D_ && s.dv == DV_ && s.m == M_) {                                                                 \
    if (dtype == 0)                                                                                            \
      return run_bidir<float, D_, DV_, M_>(static_cast<const float*>(q), static_cast<const float*>(k),        \
                                           static_cast<const float*>(v), omega, s, kind, eps, out_f32, out, ws, \
                                           st);                                                                \
    return run_bidir<bf16, D_, DV_, M_>(static_cast<const bf16*>(q), static_cast<const bf16*>(k),             \
                                        static_cast<const bf16*>(v), omega, s, kind, eps, out_f32, out, ws, st); \
  }
  FAVOR_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

template <typename T, int D, int M>
static hipError_t run_features(const T* x, const float* omega, const Shape& s, int kind, float eps, float* phi,
                               float* logscale, hipStream_t st) {
  using P = typename Ops<T>::P;
  constexpr int DC = (D + 31) / 32;
  const float sc = std::pow((float)D, -0.25f);
  const float wscale = (kind == kPrf) ? sc * kLog2e : sc;
  const float nscale_ln = sc * sc * 0.5f;
  const float inv_sqrt_m = 1.0f / std::sqrt((float)M);
  const int tpw = 256;
  const int n_tiles = (s.L + tpw - 1) / tpw;
  const size_t lds = (size_t)(M / 16) * DC * 512 * sizeof(P);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&features_kernel<T, D, M>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  {
    FAVOR_TIMED("features", st);
    features_kernel<T, D, M><<<(unsigned)(s.bh() * n_tiles), 256, lds, st>>>(
        x, omega, s.H, s.L, kind, eps, inv_sqrt_m, wscale, nscale_ln, phi, logscale, tpw, n_tiles);
  }
  return hipGetLastError();
}

hipError_t launch_features(const void* x, const float* omega, const Shape& s, int dtype, int kind, float eps,
                           float* phi, float* logscale, hipStream_t st) {
#define X(D_, DV_, M_)                                                                                   \
  if (s.d == D_ && s.m == M_) {                                                                          \
    if (dtype == 0)                                                                                      \
      return run_features<float, D_, M_>(static_cast<const float*>(x), omega, s, kind, eps, phi, logscale, st); \
    return run_features<bf16, D_, M_>(static_cast<const bf16*>(x), omega, s, kind, eps, phi, logscale, st);     \
  }
  FAVOR_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace favor
