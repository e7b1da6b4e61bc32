// Segments of the causal path on gfx950: the scan that joins the per-segment sums of the
// key/value reduction into carries, and the LDS ring of 32-token chunks read by the
// segment sweeps (the forward sweep and the two gradient sweeps).
#pragma once
#include "favor_device.hpp"
#include "favor_plan.hpp"
#include "favor_reduce.hpp"
#include "favor_tiles.hpp"

namespace favor {

// ---------------------------------------------------------------- scan over segments
// Grid b*h x (chunks of 256 float4 elements), flattened: every thread scans four consecutive
// elements of a segment partial (fragment layout, see kv_reduce_kernel) over the segments of
// its (b,h), loading a batch of segments before it sums them. Element e of a partial:
// e < NP: part[fc][nb][lane][j] = S_aug[fc*32 + 16(j>>2) + 4g + (j&3)][nb*16 + c];
// e >= NP: zpart[fc][g][j] = z[fc*32 + 16(j>>2) + 4g + (j&3)] (c = lane & 15, g = lane >> 4);
// the four elements of a thread share fc and g and differ in j & 3.
// The final state (S_final, z_final: nullable) goes out in canonical scale for the m_valid real features,
// S_final rows ldS apart (a column group writes its vcols columns; z_final only when non-null).
// CT: the type the carries are stored in (fp32; bf16 where the sweep rounds the carried state to bf16 for its
// contractions anyway); PT: the type of the segment partials (fp32; bf16 when no final state is asked for). The
// sums themselves and the final state are fp32.
template <int D, int DV, int M, typename CT = float, typename PT = float>
__global__ void __launch_bounds__(256)
scan_kernel(const PT* __restrict__ part, const PT* __restrict__ zpart, const float* __restrict__ pmax,
            int nseg, int kind, float log2_sqrt_m, CT* __restrict__ cpart, CT* __restrict__ cz,
            float* __restrict__ cmax, float* __restrict__ S_final, float* __restrict__ z_final, int m_valid,
            int ldS, int vcols) {
  constexpr int NWR = RedSplit<M, D>::NW, FBR = RedSplit<M, D>::FB;
  constexpr int NFC = (M + 31) / 32, NVB = DV / 16;
  constexpr int NP = NFC * NVB * 512, NZ = NFC * 32;
  constexpr int NQ = (NP + NZ) / 4;  // float4 elements per partial
  constexpr int NBLK = (NQ + 255) / 256;
  constexpr int KB = 8;  // segments loaded per batch
  extern __shared__ float pre[];  // [nseg] prefix maxima over segments and waves
  // the keys carry a stabiliser (a running maximum of their exponents, or of their norms for the
  // trigonometric map) except under ReLU
  const bool scaled = kind != kRelu;
  const int bh = blockIdx.x / NBLK, blk = blockIdx.x % NBLK;
  for (int p = threadIdx.x; p < nseg; p += blockDim.x) {  // the segments' own maxima
    const size_t slot = (size_t)bh * nseg + p;
    float mx = -INFINITY;
    for (int w = 0; w < NWR; ++w) mx = fmaxf(mx, pmax[slot * NWR + w]);
    pre[p] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // prefix maxima
    float run = -INFINITY;
    for (int p = 0; p < nseg; ++p) {
      run = fmaxf(run, pre[p]);
      pre[p] = scaled ? run : 0.f;
      if (blk == 0) cmax[(size_t)bh * nseg + p] = pre[p];
    }
  }
  __syncthreads();
  const int e4 = blk * 256 + threadIdx.x;
  if (e4 >= NQ) return;
  const int e = e4 * 4;
  const bool isz = e >= NP;
  int fc, col, g, j0;
  if (!isz) {
    fc = e / (NVB * 512);
    const int rest = e % (NVB * 512), nb = rest / 512, lane = (rest / 8) % 64;
    j0 = rest % 8;
    g = lane >> 4;
    col = nb * 16 + (lane & 15);
  } else {
    const int ez = e - NP;
    fc = ez / 32;
    g = (ez / 8) % 4;
    j0 = ez % 8;
    col = DV;
  }
  const int r0 = fc * 32 + 16 * (j0 >> 2) + 4 * g;  // features r0..r0+3 (rows of S_aug)
  const int wv = (fc * 32) / (FBR * 16);           // the reducing wave that owned them
  const PT* src = isz ? zpart + (e - NP) : part + e;  // four partials at src[slot * NE]
  CT* dst = isz ? cz + (e - NP) : cpart + e;  // four carries at dst[slot * NE]
  const size_t stride = (isz ? NZ : NP) / 4;
  const size_t NE = stride * 4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float prev = 0.f;
  for (int p0 = 0; p0 < nseg; p0 += KB) {
    f32x4 x[KB];
    float sc[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {  // a segment past the last is read as the last, weight 0
      const int p = p0 + u < nseg ? p0 + u : nseg - 1;
      const size_t slot = (size_t)bh * nseg + p;
      x[u] = ld4_f32(src + slot * NE);
      sc[u] = scaled ? pmax[slot * NWR + wv] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int p = p0 + u;
      if (p < nseg) {
        const size_t slot = (size_t)bh * nseg + p;
        const float mp = pre[p];
        if (p > 0) acc *= fast_exp2(prev - mp);
        st4_f32(dst + slot * NE, acc);
        acc += x[u] * (scaled ? fast_exp2(sc[u] - mp) : 1.f);
        prev = mp;
      }
    }
  }
  if (S_final && r0 < m_valid) {
    const float f = (kind == kPrf) ? fast_exp2(prev - log2_sqrt_m) : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!isz) {
        if (col < vcols) S_final[((size_t)bh * m_valid + r0 + i) * ldS + col] = acc[i] * f;
      } else if (z_final) {
        z_final[(size_t)bh * m_valid + r0 + i] = acc[i] * f;
      }
    }
  }
}

// ---------------------------------------------------------------- sweep ring
// One slot per 32-token chunk: Q rows, K rows, V rows, in 16-byte chunks copied
// asynchronously (global_load_lds), chunk q of the slot by thread q mod NT. Q and K chunks
// are XOR-swizzled by row (chunk cc of row r at position cc ^ (r mod CPR_X)) so that the
// projection reads of 16 rows spread over the banks, and are converted in place to the
// projection type by the thread that copied them; V rows are laid out as in Ring (so
// value_frags reads them from slot + XC*16). Rows past L are copies of row L-1.
template <typename T, int D, int DV, int NT, bool WITH_G = false>
struct SweepRing {
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int CPR_X = D / EPC;
  static constexpr int CPR_V = DV / EPC;
  static constexpr int XC = 32 * CPR_X;
  static constexpr int VC = 32 * CPR_V;
  static constexpr int NCH = 2 * XC + (WITH_G ? 2 : 1) * VC;  // Q, K, V (and G) chunks
  static constexpr int CPT = (NCH + NT - 1) / NT;
  static_assert(XC % 64 == 0 && VC % 64 == 0 && NT % 64 == 0, "each wave's copies come from one tensor");
  static constexpr int SLOT = CPT * NT * 16;
  static constexpr bool SWZ_V = sizeof(T) == 2;
  static_assert((CPR_X & (CPR_X - 1)) == 0 && CPR_X <= 64, "rows of whole, power-of-two chunk counts");

  static __device__ __forceinline__ int x_off(int x, int row, int cc) {
    return (x * XC + row * CPR_X + (cc ^ (row & (CPR_X - 1)))) * 16;
  }

  // G (WITH_G): rows of a fourth [.., DV] array (the upstream gradient), laid out like V after it. V rows
  // are ldv elements apart with vcols valid columns (chunks past them are copied from the row's start
  // and masked by the consumer).
  // Rows arrive through buffer resources that end at the chunk's last row inside L: rows past L land as zeros,
  // and each thread's byte offsets stay the same from chunk to chunk.
  static __device__ __forceinline__ void issue(const T* Q, const T* K, const T* V, int L, size_t rowbase, int tok0,
                                               uint32_t slot, const T* G = nullptr, int ldv = DV, int vcols = DV) {
    const int tid = threadIdx.x, w = tid >> 6;
    const size_t row0 = rowbase + tok0;
    const uint32_t nrows = (uint32_t)max(0, min(32, L - tok0));
    const u32x4 rq = raw_buffer(Q + row0 * D, nrows * (uint32_t)(D * sizeof(T)));
    const u32x4 rk = raw_buffer(K + row0 * D, nrows * (uint32_t)(D * sizeof(T)));
    const u32x4 rv = raw_buffer(V + row0 * ldv, nrows * (uint32_t)ldv * (uint32_t)sizeof(T));
    u32x4 rg = rv;
    if constexpr (WITH_G) rg = raw_buffer(G + row0 * DV, nrows * (uint32_t)(DV * sizeof(T)));
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + tid;
      const uint32_t lds = slot + (uint32_t)(u * NT + w * 64) * 16u;
      if (q < 2 * XC) {
        const int x = q / XC, p = q % XC, row = p / CPR_X;
        const int cc = (p % CPR_X) ^ (row & (CPR_X - 1));
        lds_dma16_buf(x == 0 ? rq : rk, (uint32_t)((row * D + cc * EPC) * sizeof(T)), lds);
      } else if (q < NCH) {
        const bool isg = WITH_G && q >= 2 * XC + VC;
        const int p = q - 2 * XC - (isg ? VC : 0), row = p / CPR_V, pc = p % CPR_V;
        const int cc = SWZ_V ? (pc ^ (row & (CPR_V - 1))) : pc;
        if (isg)
          lds_dma16_buf(rg, (uint32_t)((row * DV + cc * EPC) * sizeof(T)), lds);
        else
          lds_dma16_buf(rv, (uint32_t)((row * ldv + (cc * EPC < vcols ? cc * EPC : 0)) * sizeof(T)), lds);
      } else {
        lds_dma16_buf(rq, 0xfffffff0u, lds);  // past every resource: zeros
      }
    }
  }

  // this thread's Q and K chunks of a landed slot, converted in place to P; per row
  // qn = |q| * kQueryMargin and kn = |k|^2 * nscale (+inf for rows at or past nvalid)
  template <typename P>
  static __device__ __forceinline__ void convert(unsigned char* slot, float* qn, float* kn, float nscale,
                                                 int nvalid) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int q = u * NT + threadIdx.x;
      if (u * NT >= 2 * XC) break;  // no X chunks left (known at compile time)
      const bool has = ((2 * XC) % NT == 0) || q < 2 * XC;
      const int x = q / XC, row = (q % XC) / CPR_X;
      float s2 = 0.f;
      if (has) {
        if constexpr (sizeof(T) == 2) {
          const vec8<T> v8 = *reinterpret_cast<const vec8<T>*>(slot + q * 16);
          vec8<P> y;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float f = to_f(v8[j]);
            s2 += f * f;
            y[j] = to_t<P>(f);
          }
          if constexpr (sizeof(P) == 2)
            if (s2 >= kF16MaxSq) clamp_to_f16<P>(v8, y);
          *reinterpret_cast<vec8<P>*>(slot + q * 16) = y;
        } else {
          const f32x4 v4 = *reinterpret_cast<const f32x4*>(slot + q * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) s2 += v4[j] * v4[j];
        }
      }
      s2 = lanes_sum<CPR_X>(s2);  // the CPR_X chunks of a row sit on consecutive lanes
      if (has) {
        if (x == 0)
          qn[row] = __builtin_amdgcn_sqrtf(s2) * kQueryMargin;  // hardware square root (1 ulp, inside the margin)
        else
          kn[row] = row < nvalid ? s2 * nscale : INFINITY;
      }
    }
  }

  // 8 elements of row r of X (0: Q, 1: K) from column col (a multiple of 8), converted slot
  template <typename P>
  static __device__ __forceinline__ vec8<P> ld_x8(const unsigned char* slot, int x, int r, int col) {
    if constexpr (sizeof(P) == 2) {
      return *reinterpret_cast<const vec8<P>*>(slot + x_off(x, r, col / 8));
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(slot + x_off(x, r, col / 4));
      const f32x4 b = *reinterpret_cast<const f32x4*>(slot + x_off(x, r, col / 4 + 1));
      vec8<P> v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = a[j];
        v[j + 4] = b[j];
      }
      return v;
    }
  }
};

}  // namespace favor
