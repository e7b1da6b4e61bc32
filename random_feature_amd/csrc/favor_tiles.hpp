// Tiles of tokens on gfx950: the asynchronous LDS ring, the value fragments and the
// key/value reduction kernel, shared by the bidirectional and the causal paths.
#pragma once
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"

#include <algorithm>

namespace favor {

// Most features one wave owns at projection width D: a wave holds its rows of Omega' (D/32
// fragments per 16 features) and its accumulators in registers, so at D = 128 a wave takes half
// as many features as at D <= 64.
template <int D> constexpr int kFeatPerWave = D > 64 ? 32 : 64;

// Waves per workgroup and 16-feature blocks per wave of the query-side kernels for m features:
// up to four waves of up to kFeatPerWave features, then up to eight.
template <int M, int D> struct FeatSplit {
  static constexpr int BASE = (M / 16) < 4 ? (M / 16) : 4;
  static constexpr int NW = M / BASE > kFeatPerWave<D> ? (M / kFeatPerWave<D> < 8 ? M / kFeatPerWave<D> : 8) : BASE;
  static constexpr int FB = M / (16 * NW);
};
// Three output workgroups per CU (three waves per SIMD) where the registers allow it: 16-bit inputs with at most
// four waves of up to 64 features. Their phase 2 then takes both token halves per wave, which holds the S fragments
// of fewer value blocks (half the registers) for twice the LDS reads of the features.
template <typename T, int M, int D> constexpr bool kOutThree = sizeof(T) == 2 && FeatSplit<M, D>::NW <= 4;
// Waves of the key/value reduction (and of the causal sweep, which shares its split): up to
// RW_MAX waves of 32 features or more, then up to eight when a wave would own more than
// kFeatPerWave features. Up to four waves: two workgroups per CU (NW/2 waves per SIMD; the
// second launch bound is waves per EU); eight waves: one workgroup per CU.
template <int M, int D> struct RedSplit {
  static constexpr int RW_MAX = FAVOR_REDUCE_WAVES;
  static constexpr int BASE = M < 32 ? 1 : ((M / 32) < RW_MAX ? (M / 32) : RW_MAX);
  static constexpr int NW = M / BASE > kFeatPerWave<D> ? (M / kFeatPerWave<D> < 8 ? M / kFeatPerWave<D> : 8) : BASE;
  static constexpr int FB = M / (16 * NW);
  static constexpr int WPE = NW < 2 ? 1 : (NW / 2 < 2 ? NW / 2 : 2);
};

// Waves of the gradient kernels: one per 32 features, at most FAVOR_BWD_WAVES. Eight waves in
// one workgroup per CU put two waves on every SIMD, so one wave's vector work overlaps
// another's matrix work.
#ifndef FAVOR_BWD_WAVES
#define FAVOR_BWD_WAVES 8
#endif
template <int M> struct BwdSplit {
  static constexpr int NW = M < 32 ? 1 : ((M / 32) < FAVOR_BWD_WAVES ? (M / 32) : FAVOR_BWD_WAVES);
  static constexpr int FB = M / (16 * NW);
};

constexpr int kNormNone = 0, kNormSq = 1, kNormAbs = 2, kNormNegSq = 3;

// ---------------------------------------------------------------- tile ring
// 32-token tiles of X (keys or queries) and V arrive in an R-slot LDS ring through
// asynchronous 16-byte copies issued R-1 tiles ahead. Chunk q of a slot (16 bytes) is
// copied by thread q mod NT, so every thread can convert the chunks it copied itself as
// soon as its own copies have landed. X chunks come first (row-major); V chunks follow,
// row-major with the chunk column XOR-swizzled by the row for 16-bit types (spreads the
// transposing reads over the LDS banks). Rows past L are copied from row L-1 and masked
// by the consumer; slots past the end of a piece are filled with harmless copies so that
// every tile costs the same number of copies and the waits stay uniform. V rows are ldv elements
// apart and hold vcols valid columns (a column group of a wider V: DV columns are compiled,
// chunks at or past vcols are copied from the row's start and masked by the consumer).
template <typename T, int D, int DV, int NT, bool WITH_V>
struct Ring {
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int CPR_X = D / EPC;
  static constexpr int CPR_V = WITH_V ? DV / EPC : 1;
  static constexpr int XC = 32 * CPR_X;
  static constexpr int VC = WITH_V ? 32 * CPR_V : 0;
  static constexpr int CPT = (XC + VC + NT - 1) / NT;
  static_assert(XC % 64 == 0 && VC % 64 == 0 && NT % 64 == 0, "each wave's copies come from one tensor");
  static constexpr int SLOT = CPT * NT * 16;
  static constexpr bool SWZ = sizeof(T) == 2 && WITH_V;

  // copies of the tile at (bh, tok0) into the slot at LDS byte address `slot`; !live: filler. The tile's rows
  // come through buffer resources that end at the tile's last row inside L, so rows past L (and every row of a
  // filler) land as zeros, and each thread's byte offset stays the same from tile to tile.
  static __device__ __forceinline__ void issue(const T* X, const T* V, int L, int bh, int tok0, bool live,
                                               uint32_t slot, int ldv = DV, int vcols = DV) {
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t row0 = (size_t)bh * L + (live ? tok0 : 0);
    const uint32_t nrows = live ? (uint32_t)min(32, L - tok0) : 0u;
    const u32x4 rx = raw_buffer(X + row0 * D, nrows * (uint32_t)(D * sizeof(T)));
    u32x4 rv = rx;
    if constexpr (WITH_V) rv = raw_buffer(V + row0 * ldv, nrows * (uint32_t)ldv * (uint32_t)sizeof(T));
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + tid;
      const uint32_t lds = slot + (uint32_t)(u * NT + w * 64) * 16u;
      if ((XC % NT == 0) ? (u * NT < XC) : (q < XC)) {
        const int row = q / CPR_X, cc = q % CPR_X;
        lds_dma16_buf(rx, (uint32_t)((row * D + cc * EPC) * sizeof(T)), lds);
      } else if (WITH_V && q < XC + VC) {
        const int p = q - XC, row = p / CPR_V, pc = p % CPR_V;
        const int cc = SWZ ? (pc ^ (row & (CPR_V - 1))) : pc;
        lds_dma16_buf(rv, (uint32_t)((row * ldv + (cc * EPC < vcols ? cc * EPC : 0)) * sizeof(T)), lds);
      } else {
        lds_dma16_buf(rx, 0xfffffff0u, lds);  // past every resource: zeros
      }
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
  // nvalid); kNormNegSq: its negation; NORM == kNormAbs: |x| * nscale
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
          if constexpr (sizeof(P) == 2)
            if (s2 >= kF16MaxSq) clamp_to_f16<P>(x, y);
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
          else if constexpr (NORM == kNormNegSq)
            nrm[row] = row < nvalid ? s2 * -nscale : -INFINITY;
          else
            nrm[row] = __builtin_amdgcn_sqrtf(s2) * nscale;  // hardware square root (1 ulp; the bound's margin covers it)
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
// the raw V rows of a slot; the last block is the ones column (z). Blocks at or past vcols
// (a narrower column group) are zero.
template <typename T, int D, int DV, int NT>
__device__ __forceinline__ void value_frags(const unsigned char* slot, vec8<typename Ops<T>::C> (&vf)[DV / 16 + 1],
                                            int c, int g, int vcols = DV) {
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
  if (vcols < DV) {
#pragma unroll
    for (int nb = 0; nb < NB - 1; ++nb)
      if (nb * 16 >= vcols) vf[nb] = zero8<C>();
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
// Pieces: with seg_tiles == 0 the flattened (b*h, tile) space is cut into G even pieces and
// the partial of (piece i, b*h) goes to slot i + b*h; with seg_tiles > 0 piece i is segment
// i % nseg (seg_tiles tiles) of (b,h) i / nseg and its partial goes to slot i.
// LDS ring slots of the key/value reduction.
constexpr int kReduceRing = 5;

// Headroom (log2 units) the key stabiliser leaves below its running maximum: the largest
// feature after a shift is 2^-8, far above the bottom of the fp32/bf16 range.
constexpr float kKeyMargin = 8.f;

// PSPLIT (16-bit projection type): the projection runs through the Omega' fragments and their
// residuals (omf_lo, see omega_frag_kernel), two MFMAs per block, so the exponents carry the fp32
// Omega' instead of its 11-bit rounding (the gradient kernels need that at large input norms).
// Each wave keeps its residual fragments in its own part of LDS (registers are full); launch this
// variant with a 4-slot ring so that two workgroups still fit on a CU.
// Shapes: D, DV and M are compiled. With GEN a call may use fewer features (m_valid <= M, a
// multiple of 16: the features past it are masked to zero and their wave maxima written as -inf)
// and a column group of a wider V (rows ldv apart, vcols <= DV valid columns); without GEN those
// arguments are ignored (m_valid = M, ldv = vcols = DV).
// PT: the type the partial sums are stored in (fp32, or bf16 where the reader rounds them to bf16 anyway).
template <typename T, int D, int DV, int M, int R, int KIND, bool SPLIT = false, bool PSPLIT = false, bool GEN = false,
          typename PT = float>
__global__ void __launch_bounds__(64 * (RedSplit<M, D>::NW), (RedSplit<M, D>::WPE))
kv_reduce_kernel(const T* __restrict__ K, const T* __restrict__ V, const typename Ops<T>::P* __restrict__ omf,
                 const typename Ops<T>::P* __restrict__ omf_lo,
                 int H, int L, int tpb, long long T_all, int G, float eps, float inv_sqrt_m, float nscale,
                 PT* __restrict__ part, PT* __restrict__ zpart, float* __restrict__ pmax, int seg_tiles,
                 int nseg, int m_valid_, int ldv_, int vcols_) {
  using P = typename Ops<T>::P;
  using C = typename Ops<T>::C;
  constexpr int NW = RedSplit<M, D>::NW, FB = RedSplit<M, D>::FB;
  const int m_valid = GEN ? m_valid_ : M, ldv = GEN ? ldv_ : DV, vcols = GEN ? vcols_ : DV;
  constexpr int NFC = (M + 31) / 32;
  static_assert(FB % 2 == 0 || NW == 1, "an odd block count per wave only with a single wave");
  constexpr int NT = 64 * NW;
  constexpr int DC = (D + 31) / 32;
  constexpr int NB = DV / 16 + 1;  // value-column blocks + the ones column (z = Phi^T 1)
  constexpr int KROW = D + 8;
  static_assert(R >= 4, "ring: the tile contracted, one converted ahead, one being converted, one in flight");
  using Rg = Ring<T, D, DV, NT, true>;
  // key norms as stored: negated for the positive map, whose exponents start from -(n'_t + M)
  constexpr int KN = KIND == kPrf ? kNormNegSq : kNormSq;
  // at the wait of iteration t the copies issued so far reach tile t+R-1 (each iteration issues
  // at its start, into the slot its predecessor has just released): R-3 tiles are newer than tile t+2
  constexpr int WAIT_NEXT = Rg::CPT * (R - 3);
  __shared__ __attribute__((aligned(16))) unsigned char ring[R][Rg::SLOT];
  __shared__ __attribute__((aligned(16))) P ks[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) float kn[2][32];
  constexpr bool PS = PSPLIT && sizeof(P) == 2;
  __shared__ __attribute__((aligned(16))) P oml_s[PS ? NW * FB * DC * 64 * 8 : 8];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const long long pc = xcd_remap(blockIdx.x, gridDim.x);
  long long t_beg, t_end;
  if (seg_tiles > 0) {
    // segments: piece pc is segment pc % nseg of (b,h) pc / nseg, and its partial goes to slot pc
    const long long sb = pc / nseg, sp = pc % nseg;
    t_beg = sb * tpb + sp * seg_tiles;
    t_end = sb * tpb + std::min<long long>((sp + 1) * seg_tiles, tpb);
  } else {
    t_beg = piece_start(pc, T_all, G);
    t_end = piece_start(pc + 1, T_all, G);
  }
  if (t_beg >= t_end) return;
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  f32x4 sacc[FB][NB];
  float runmax = 0.f;
  bool first = true;
  vec8<P> om[FB][DC];

  // one (b,h)'s sums of this piece, as A fragments of S^T (the layout of sfr) in PT:
  // part[slot][fc][nb][lane][j], the z column compacted to zpart[slot][fc][g][j] (lanes c = 0)
  auto flush = [&](int fbh, float fmax) {
    const size_t slot = (size_t)pc + (seg_tiles > 0 ? 0 : fbh);
#pragma unroll
    for (int p = 0; p < (FB + 1) / 2; ++p) {
      const int fc = (w * FB) / 2 + p;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 lo = sacc[2 * p][nb], hi = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FB % 2 == 0) hi = sacc[2 * p + 1][nb];
        PT* dst;
        if (nb < NB - 1)
          dst = part + (((slot * NFC + fc) * (NB - 1) + nb) * 64 + lane) * 8;
        else
          dst = zpart + ((slot * NFC + fc) * 4 + g) * 8;
        if (nb < NB - 1 || c == 0) st8_f32(dst, lo, hi);
      }
    }
    if (lane == 0) pmax[slot * NW + w] = w * FB * 16 < m_valid ? fmax : -INFINITY;  // -inf: no valid feature
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
      for (int dc = 0; dc < DC; ++dc) {
        const size_t o = ((((size_t)h * (M / 16) + w * FB + fb) * DC + dc) * 64 + lane) * 8;
        om[fb][dc] = ld8<P>(omf + o);
        // written and read back by this wave only (LDS operations of a wave complete in order)
        if constexpr (PS) st8<P>(&oml_s[(((w * FB + fb) * DC + dc) * 64 + lane) * 8], ld8<P>(omf_lo + o));
      }
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
        for (int i = 0; i < 4; ++i) bias[i] = n4[i] - rm;  // n4 = -n'_t
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
        for (int dc = 0; dc < DC; ++dc) {
          mma16(pa[tb][fb], kf[dc], om[fb][dc]);
          if constexpr (PS)
            mma16(pa[tb][fb], kf[dc], ld8<P>(&oml_s[(((w * FB + fb) * DC + dc) * 64 + lane) * 8]));
        }
      }
    }
  };

  const int n_tiles = (int)(t_end - t_beg);
  TileCursor ahead(t_beg, tpb), cur(t_beg, tpb), cv(t_beg, tpb);
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    Rg::issue(K, V, L, ahead.bh, ahead.tok0(), s < n_tiles, ring0 + s * Rg::SLOT, ldv, vcols);
    if (s < n_tiles) ahead.next();
  }
  // tiles 0 and 1 converted up front; iteration t converts tile t+2
  wait_vmcnt<Rg::CPT * (R - 2)>();
  Rg::template convert<P, KROW, KN>(ring[0], ks[0], kn[0], nscale, L - cv.tok0());
  cv.next();
  wait_vmcnt<Rg::CPT * (R - 3)>();
  Rg::template convert<P, KROW, KN>(ring[1], ks[1], kn[1], nscale, L - cv.tok0());
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
    {
      // the copies of tile t+R-1, into the slot of tile t-1 (its value rows were read before the last barrier)
      const bool live = it + R - 1 < n_tiles;
      Rg::issue(K, V, L, ahead.bh, ahead.tok0(), live, ring0 + s_iss * Rg::SLOT, ldv, vcols);
      if (live) ahead.next();
    }
    // stabiliser of tile t (its projection is complete)
    // trigonometric features: the keys' own scale exp(|y|^2/2) = 2^(n'_t) rides on a running
    // maximum of n'_t in the same way (rows past L carry an infinite norm: weight 0)
    float tw[2][4];
    if constexpr (KIND == kTrig) {
      float lmax = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(&kn[buf][tb * 16 + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tw[tb][i] = n4[i] < INFINITY ? n4[i] - (first ? 0.f : runmax) : -INFINITY;
          lmax = fmaxf(lmax, tw[tb][i]);
        }
      }
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
          for (int i = 0; i < 4; ++i) tw[tb][i] -= shift;
        first = false;
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tw[tb][i] = fast_exp2(tw[tb][i]);
    }
    if constexpr (KIND == kPrf) {
      if (m_valid < M) {  // features past m_valid: exponent -inf, feature 0
#pragma unroll
        for (int fb = 0; fb < FB; ++fb)
          if ((w * FB + fb) * 16 + c >= m_valid) {
            pcur[0][fb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            pcur[1][fb] = pcur[0][fb];
          }
      }
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
        const float tmx = wave_max(lmax);  // -inf only in a wave without a valid feature
        const float shift = (tmx > -INFINITY ? tmx : 0.f) + kKeyMargin;
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

    // stretch 1: projection of tile t+1 beside the feature map of tile t, at raised issue
    // priority so that the feature map's vector work of this wave goes ahead of the other
    // wave's contraction, which fills the gaps
    __builtin_amdgcn_s_setprio(1);
    project(pnext, buf ^ 1, next_new ? 0.f : runmax);
    // SPLIT (16-bit contraction type): each feature as the sum of two values of that type,
    // both contracted, so S_aug carries the features' fp32 precision
    constexpr bool LO = SPLIT && sizeof(C) == 2;
    vec8<C> af[FB], al[LO ? FB : 1];
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      float fv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = pcur[j >> 2][fb][j & 3];
        float f;
        if constexpr (KIND == kPrf) {
          f = fast_exp2(a);  // rows past L carry an infinite norm: exp2(-inf) = 0
        } else if constexpr (KIND == kTrig) {
          f = trig_feature(a, (w * FB + fb) * 16 + c, M) * tw[j >> 2][j & 3];
        } else {
          const bool ok = tok0 + 16 * (j >> 2) + 4 * g + (j & 3) < L && (!GEN || (w * FB + fb) * 16 + c < m_valid);
          f = ok ? fmaxf(a, 0.f) * inv_sqrt_m + eps : 0.f;
        }
        fv[j] = f;
      }
      if constexpr (LO) {
        split_all<8>(af[fb], al[fb], [&](int j) { return fv[j]; });
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) af[fb][j] = to_t<C>(fv[j]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // stretch 2: contraction of tile t beside the conversion of tile t+2 (past the end of
    // the piece: a filler slot into an unused buffer)
    vec8<C> vf[NB];
    value_frags<T, D, DV, NT>(ring[s_cur], vf, c, g, vcols);
#pragma unroll
    for (int fb = 0; fb < FB; ++fb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        mma16(sacc[fb][nb], af[fb], vf[nb]);
        if constexpr (LO) mma16(sacc[fb][nb], al[fb], vf[nb]);
      }
    Rg::template convert<P, KROW, KN>(ring[s_cv], ks[buf], kn[buf], nscale, L - cv.tok0());
    cv.next();
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

// ---------------------------------------------------------------- query bound
// Exponent bound (log2 units) under which the bound stabiliser of the queries keeps every
// query feature a normal float: the features lie in [2^(-2 bound), 1]. Above it a tile
// takes the exact row maxima instead.
constexpr float kQueryBoundLimit = 60.f;
// |q| is scaled by this before the bound is formed: it covers the rounding of q to the
// projection type and of the MFMA sums.
constexpr float kQueryMargin = 1.f + 1.f / 512.f;

// Largest row norm of a head's rounded Omega' (the fragments of the workgroup's NW waves
// together cover every row): per wave, then across the waves through xch[w * stride]
// (two barriers, so xch is free again on return).
template <int NW, typename V8, int FB, int DC>
__device__ __forceinline__ float omega_norm_max(const V8 (&om)[FB][DC], float* xch, int stride) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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
  if (lane == 0) xch[w * stride] = n2;
  lds_barrier();
  float m2 = xch[0];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) m2 = fmaxf(m2, xch[ww * stride]);
  lds_barrier();
  return __builtin_sqrtf(m2);
}

}  // namespace favor
