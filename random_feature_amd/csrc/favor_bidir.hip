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
  // and (NORMS) the scaled squared row norms into kn
  template <typename P, int KROW, bool NORMS>
  static __device__ __forceinline__ void convert(const unsigned char* slot, P* conv, float* kn, float nscale) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + threadIdx.x;
      if (u * NT >= XC) break;  // no X chunks left (known at compile time)
      const int row = q / CPR_X, cc = q % CPR_X;
      float s2 = 0.f;
      if (q < XC) {
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
      if constexpr (NORMS) {
#pragma unroll
        for (int o = 1; o < CPR_X; o <<= 1) s2 += __shfl_xor(s2, o, 64);
        if (q < XC && cc == 0) kn[row] = s2 * nscale;
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
//               and rescale the accumulated S_aug by the same power of two
//   maps        Phi = exp2(.) (ReLU: max(a,0)/sqrt(m) + eps), rounded to the contraction type
//   contracts   S_aug += Phi^T [V 1]: A = Phi^T (paired token slots, the accumulators as
//               they are), B = the value fragments
// Tiles stream through the asynchronous ring R-1 ahead; one barrier per tile.
template <typename T, int D, int DV, int M, int R>
__global__ void __launch_bounds__(64 * FeatSplit<M>::NW, 2)
kv_reduce_kernel(const T* __restrict__ K, const T* __restrict__ V, const typename Ops<T>::P* __restrict__ omf,
                 int H, int L, int tpb, long long T_all, int G, int kind, float eps, float inv_sqrt_m, float nscale,
                 float* __restrict__ part, float* __restrict__ pmax) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M>::NW, FB = FeatSplit<M>::FB;
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;
  constexpr int KROW = D + 8;
  using Rg = Ring<T, D, DV, NT, true>;
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
  int cur_bh = -1;

  auto flush = [&]() {
    float* Pp = part + ((size_t)pc + cur_bh) * M * (DV + 1);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (w * FB + fb) * 16 + 4 * g + i;
#pragma unroll
        for (int nb = 0; nb < NB - 1; ++nb) Pp[(size_t)r * (DV + 1) + nb * 16 + c] = sacc[fb][nb][i];
        if (c == 0) Pp[(size_t)r * (DV + 1) + DV] = sacc[fb][NB - 1][i];
      }
    if (lane == 0) pmax[((size_t)pc + cur_bh) * NW + w] = runmax;
  };

  const int n_tiles = (int)(t_end - t_beg);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb);
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    Rg::issue(K, V, L, ahead.bh, ahead.tok0(), s < n_tiles, ring0 + s * Rg::SLOT);
    if (s < n_tiles) ahead.next();
  }
  wait_vmcnt<Rg::CPT * (R - 2)>();
  Rg::template convert<P, KROW, true>(ring[0], ks[0], kn[0], nscale);
  lds_barrier();

  for (int it = 0; it < n_tiles; ++it, cur.next()) {
    const int buf = it & 1;
    const int bh = cur.bh, tok0 = cur.tok0();
    {
      const bool live = it + R - 1 < n_tiles;
      Rg::issue(K, V, L, ahead.bh, ahead.tok0(), live, ring0 + ((it + R - 1) % R) * Rg::SLOT);
      if (live) ahead.next();
    }
    if (bh != cur_bh) {
      if (cur_bh >= 0) {
        flush();
        wait_vmcnt<0>();
      }
      const int h = bh % H;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          om[fb][dc] = ld8<P>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      runmax = 0.f;
      first = true;
      cur_bh = bh;
    }

    // accumulator start values: the negated key bias of rows 4g+i (-inf for rows past L)
    f32x4 bias[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = tok0 + tb * 16 + 4 * g + i < L;
        bias[tb][i] = (kind == kPrf) ? (ok ? -(n4[i] + runmax) : -INFINITY) : 0.f;
      }
    }
    f32x4 pacc[2][FB];
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
        pacc[tb][fb] = bias[tb];
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(pacc[tb][fb], kf[dc], om[fb][dc]);
      }
    }
    if (kind == kPrf) {
      float tmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, pacc[tb][fb][i]);
      tmax = wave_max(tmax);
      if (first || tmax > 0.f) {
        if (!first) {
          const float sc = fast_exp2(-tmax);
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sacc[fb][nb] *= sc;
        }
        runmax += tmax;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int fb = 0; fb < FB; ++fb) pacc[tb][fb] -= tmax;
        first = false;
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
        for (int i = 0; i < 4; ++i) {
          const bool ok = tok0 + tb * 16 + 4 * g + i < L;
#pragma unroll
          for (int fb = 0; fb < FB; ++fb)
            pacc[tb][fb][i] = ok ? fmaxf(pacc[tb][fb][i], 0.f) * inv_sqrt_m + eps : 0.f;
        }
    }
    vec8<C> vf[NB];
    value_frags<T, D, DV, NT>(ring[it % R], vf, c, g);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      vec8<C> af;
#pragma unroll
      for (int j = 0; j < 8; ++j) af[j] = to_t<C>(pacc[j >> 2][fb][j & 3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mma16(sacc[fb][nb], af, vf[nb]);
    }
    wait_vmcnt<Rg::CPT * (R - 2)>();
    if (it + 1 < n_tiles) Rg::template convert<P, KROW, true>(ring[(it + 1) % R], ks[buf ^ 1], kn[buf ^ 1], nscale);
    lds_barrier();
  }
  flush();
}

// ---------------------------------------------------------------- combine
// One workgroup per (b*h, 32-feature chunk): S_aug rows of the chunk summed over the
// pieces of that (b,h), each partial scaled by 2^(M_piece,wave - M_max), written as A
// fragments of S_aug^T (row = value column, paired feature slots):
// sfr[bh][fc][nb][lane][j] = S_aug[fc*32 + 16(j>>2) + 4g + (j&3)][nb*16 + c]; in the last
// block only row c == 0 (the z column) is nonzero.
template <typename C, int DV, int M>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ part, const float* __restrict__ pmax, int tpb, long long T_all, int G,
               int kind, C* __restrict__ sfr) {
  constexpr int NW = FeatSplit<M>::NW;
  constexpr int FPW = M / NW;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFC = (M + 31) / 32;
  extern __shared__ float scl[];  // [pieces of this bh][NW]
  const int bh = blockIdx.x / NFC, fc = blockIdx.x % NFC;
  const long long i_lo = piece_of((long long)bh * tpb, T_all, G);
  const long long i_hi = piece_of((long long)(bh + 1) * tpb - 1, T_all, G);
  const int np = (int)(i_hi - i_lo + 1);
  float gmax = -INFINITY;
  for (int k = 0; k < np * NW; ++k) gmax = fmaxf(gmax, pmax[(size_t)(i_lo + k / NW + bh) * NW + k % NW]);
  for (int k = threadIdx.x; k < np * NW; k += blockDim.x)
    scl[k] = (kind == kPrf) ? fast_exp2(pmax[(size_t)(i_lo + k / NW + bh) * NW + k % NW] - gmax) : 1.f;
  __syncthreads();
  C* out = sfr + ((size_t)bh * NFC + fc) * NB * 512;
  for (int e = threadIdx.x; e < NB * 512; e += blockDim.x) {
    const int j = e & 7, l = (e >> 3) & 63, nb = e >> 9;
    const int c = l & 15, g = l >> 4;
    const int r = fc * 32 + 16 * (j >> 2) + 4 * g + (j & 3);
    const int n = (nb < NB - 1) ? nb * 16 + c : (c == 0 ? DV : -1);
    float acc = 0.f;
    if (n >= 0 && r < M) {
      const int wv = r / FPW;
      for (int k = 0; k < np; ++k)
        acc += part[((size_t)(i_lo + k) + bh) * M * (DV + 1) + (size_t)r * (DV + 1) + n] * scl[k * NW + wv];
    }
    out[e] = to_t<C>(acc);
  }
}

// ---------------------------------------------------------------- query side
// Workgroup = NW waves over one piece of the flattened tile space; wave w owns FB*16
// features and keeps their Omega' and S_aug^T fragments in registers (reloaded when the
// piece moves to the next (b,h)). Per 32-token tile:
//   projection   A = Omega' (rows = features), B = Q^T (linear d slots) -> [feature][token]
//   row maximum  over the wave's features, then across waves through LDS (PRF)
//   feature map  Phi = exp2(a' - max) (the |q|^2 term is constant per row and cancels)
//   contraction  out^T partial = S_aug^T Phi^T over the wave's features (paired slots)
//   combination  partial tiles summed across waves through LDS; the z row gives the
//                denominator; each wave divides and stores its share of the tile.
template <typename T, int D, int DV, int M, int R>
__global__ void __launch_bounds__(64 * FeatSplit<M>::NW, 2)
q_output_kernel(const T* __restrict__ Q, const typename Ops<T>::P* __restrict__ omf,
                const typename Ops<T>::C* __restrict__ sfr, int H, int L, int tpb, long long T_all, int G, int kind,
                float eps, float inv_sqrt_m, int out_f32, void* __restrict__ out) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = FeatSplit<M>::NW, FB = FeatSplit<M>::FB;
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;
  constexpr int NFCW = (FB + 1) / 2;       // 32-feature chunks a wave touches (one half of one when FB = 1)
  constexpr int NFC = (M + 31) / 32;
  constexpr int KROW = D + 8;
  // Only wave 0 copies and converts Q tiles, and it issues no stores, so its vmcnt counts
  // nothing but the ring copies; the other waves store the outputs. (With a single wave
  // the wave does both, and its waits drain the stores as well.)
  using Rg = Ring<T, D, DV, 64, false>;
  constexpr int WAIT_N = NW > 1 ? Rg::CPT * (R - 2) : 0;
  __shared__ __attribute__((aligned(16))) unsigned char ring[R][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P qs[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float qmx[NW][32];
  __shared__ __attribute__((aligned(16))) float xch[NW][2][NB][64 * 4];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  const long long t_beg = piece_start(pc, T_all, G), t_end = piece_start(pc + 1, T_all, G);
  if (t_beg >= t_end) return;

  vec8<P> om[FB][DC];
  vec8<C> sf[NFCW][NB];
  int cur_bh = -1;
  const int fc0 = (w * FB) / 2;

  const uint32_t ring0 = lds_addr(&ring[0][0]);
  const int n_tiles = (int)(t_end - t_beg);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb);
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    if (w == 0) Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), s < n_tiles, ring0 + s * Rg::SLOT);
    if (s < n_tiles) ahead.next();
  }
  if (w == 0) {
    wait_vmcnt<Rg::CPT * (R - 2)>();
    Rg::template convert<P, KROW, false>(ring[0], qs[0], nullptr, 0.f);
  }
  lds_barrier();

  for (int it = 0; it < n_tiles; ++it, cur.next()) {
    const int buf = it & 1;
    const int bh = cur.bh, tok0 = cur.tok0();
    {
      const bool live = it + R - 1 < n_tiles;
      if (w == 0) Rg::issue(Q, nullptr, L, ahead.bh, ahead.tok0(), live, ring0 + ((it + R - 1) % R) * Rg::SLOT);
      if (live) ahead.next();
    }
    if (bh != cur_bh) {
      const int h = bh % H;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb)
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          om[fb][dc] = ld8<P>(omf + ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8);
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw) {
        const int fc = fc0 + fcw;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sf[fcw][nb] = ld8<C>(sfr + ((((size_t)bh * NFC + fc) * NB + nb) * 64 + lane) * 8);
      }
      cur_bh = bh;
    }

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
        pacc[tb][fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) mma16(pacc[tb][fb], om[fb][dc], qf[dc]);
      }
    }
    if (kind == kPrf) {
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
    }
    lds_barrier();
    if (kind == kPrf) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        float mx = qmx[0][tb * 16 + c];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) mx = fmaxf(mx, qmx[ww][tb * 16 + c]);
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pacc[tb][fb][i] = fast_exp2(pacc[tb][fb][i] - mx);
      }
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
      f32x4 oacc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int fcw = 0; fcw < NFCW; ++fcw) {
        vec8<C> bf;
        if constexpr (FB % 2 == 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) bf[j] = to_t<C>(pacc[tb][2 * fcw + (j >> 2)][j & 3]);
        } else {
          // one 16-feature block per wave: it fills half (w & 1) of its 32-feature chunk
          const int half = w & 1;
#pragma unroll
          for (int j = 0; j < 8; ++j) bf[j] = to_t<C>((j >> 2) == half ? pacc[tb][0][j & 3] : 0.f);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) mma16(oacc[nb], sf[fcw][nb], bf);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4*>(&xch[w][tb][nb][lane * 4]) = oacc[nb];
    }
    lds_barrier();
    // tiles (tb, nb) of value columns, shared out over the waves other than the copying one
    constexpr int NSW = NW > 1 ? NW - 1 : 1;
    for (int u = (NW > 1 ? w - 1 : 0); u < 2 * (NB - 1); u += NSW) {
      if (NW > 1 && w == 0) break;
      const int tb = u / (NB - 1), nb = u % (NB - 1);
      f32x4 num = *reinterpret_cast<const f32x4*>(&xch[0][tb][nb][lane * 4]);
      float den = xch[0][tb][NB - 1][c * 4];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        num += *reinterpret_cast<const f32x4*>(&xch[ww][tb][nb][lane * 4]);
        den += xch[ww][tb][NB - 1][c * 4];
      }
      const int tok = tok0 + tb * 16 + c;
      if (tok < L) {
        const float rden = 1.0f / den;
        const size_t o = ((size_t)bh * L + tok) * DV + nb * 16 + 4 * g;
        if (out_f32) {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o) = num * rden;
        } else {
          vec4<T> r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = to_t<T>(num[i] * rden);
          *reinterpret_cast<vec4<T>*>(reinterpret_cast<T*>(out) + o) = r;
        }
      }
    }
    if (w == 0) {
      wait_vmcnt<WAIT_N>();
      if (it + 1 < n_tiles) Rg::template convert<P, KROW, false>(ring[(it + 1) % R], qs[buf ^ 1], nullptr, 0.f);
    }
    lds_barrier();
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
static inline int nw_split(int m) { return std::min(4, m / 16); }
static inline size_t elt(int dtype) { return dtype == 0 ? 4 : 2; }
constexpr int kMaxPieces = 512;  // two resident 4-wave workgroups on each of 256 CUs
constexpr int kRing = 4;         // LDS ring slots: tiles in flight = kRing - 1

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
  p.off_part = off;
  off = align256(off + slots * s.m * (s.dv + 1) * 4);
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
    kv_reduce_kernel<T, D, DV, M, kRing><<<p.G, 64 * NW, 0, st>>>(k, v, omf, s.H, s.L, p.tpb, p.T_all, p.G, kind, eps,
                                                           inv_sqrt_m, nscale, part, pmax);
  }
  {
    const int max_pieces = (int)(p.G / s.bh()) + 3;
    FAVOR_TIMED("combine", st);
    combine_kernel<C, DV, M><<<(unsigned)(s.bh() * ((M + 31) / 32)), 256, (size_t)max_pieces * NW * sizeof(float),
                               st>>>(part, pmax, p.tpb, p.T_all, p.G, kind, sfr);
  }
  {
    FAVOR_TIMED("output", st);
    q_output_kernel<T, D, DV, M, kRing><<<p.G, 64 * NW, 0, st>>>(q, omf, sfr, s.H, s.L, p.tpb, p.T_all, p.G, kind, eps,
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
