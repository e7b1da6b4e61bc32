// Device-side building blocks for the FAVOR+ kernels on gfx950 (CDNA4, wave64).
//
// MFMA fragment convention used by every kernel (lane l of a wave, c = l & 15, g = l >> 4):
//   * an A fragment of a 16 x 32 tile holds A[row c][k-slot (g, j)], j = 0..7;
//   * a B fragment of a 32 x 16 tile holds B[k-slot (g, j)][col c];
//   * a 16 x 16 fp32 accumulator (f32x4) holds C[row 4g + i][col c], i = 0..3.
// A product sums over all 32 k-slots; which logical index a slot stands for is
// chosen by the loader, and A and B only have to agree. Two slot maps are used:
//   * linear:  slot (g, j) <-> k = 8g + j       (contiguous loads along k from memory)
//   * paired:  slot (g, j) <-> k = 16(j >> 2) + 4g + (j & 3)
//     which is exactly what a lane already holds in two stacked accumulators
//     (rows 0..15 and 16..31 of a 32-row C tile), so an accumulator pair turns
//     into an operand without any data movement.
// bf16: one v_mfma_f32_16x16x32_bf16 per 16x16x32 step. fp32: eight
// v_mfma_f32_16x16x4_f32, the j-th one taking slot j of every lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace favor {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename T> struct VecT;
template <> struct VecT<bf16> { using v8 = bf16x8; using v4 = bf16x4; using v2 = bf16x2; };
template <> struct VecT<float> { using v8 = f32x8; using v4 = f32x4; using v2 = f32x2; };
template <> struct VecT<f16> { using v8 = f16x8; using v4 = f16x4; using v2 = f16x2; };
template <typename T> using vec8 = typename VecT<T>::v8;
template <typename T> using vec4 = typename VecT<T>::v4;
template <typename T> using vec2 = typename VecT<T>::v2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void mma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f16x8& a, const f16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
}

// A product whose A (or B) operand is a projection matrix held as hi + lo fragments: with LO the
// residual fragments are contracted too (one more MFMA), so the sum sees the matrix to about
// fp32 accuracy instead of its 16-bit rounding.
template <bool LO, typename V8>
__device__ __forceinline__ void mma16_split_a(f32x4& acc, const V8& a_hi, const V8& a_lo, const V8& b) {
  mma16(acc, a_hi, b);
  if constexpr (LO) mma16(acc, a_lo, b);
}
template <bool LO, typename V8>
__device__ __forceinline__ void mma16_split_b(f32x4& acc, const V8& a, const V8& b_hi, const V8& b_lo) {
  mma16(acc, a, b_hi);
  if constexpr (LO) mma16(acc, a, b_lo);
}

template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ float to_t<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to_t<bf16>(float x) { return static_cast<bf16>(x); }
template <> __device__ __forceinline__ f16 to_t<f16>(float x) { return static_cast<f16>(x); }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f(f16 x) { return static_cast<float>(x); }

// x as a value of the 16-bit type C and its remainder (x - that value, also rounded to C), for slots j and
// j + 1 of two operands at once: the pair is rounded in one packed conversion and widened back with a shift
// and a mask, which the per-element form cannot share. Same results as rounding each x on its own.
template <typename V>
__device__ __forceinline__ void split_pair(float x0, float x1, V& h, V& l, int j) {
  using C = std::remove_cv_t<std::remove_reference_t<decltype(h[0])>>;
  if constexpr (std::is_same_v<C, bf16>) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const bf16x2 hp = __builtin_convertvector(f32x2{x0, x1}, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, hp);
    const float h0 = __builtin_bit_cast(float, hb << 16), h1 = __builtin_bit_cast(float, hb & 0xffff0000u);
    const bf16x2 lp = __builtin_convertvector(f32x2{x0 - h0, x1 - h1}, bf16x2);
    h[j] = hp[0];
    h[j + 1] = hp[1];
    l[j] = lp[0];
    l[j + 1] = lp[1];
  } else {
    const C h0 = to_t<C>(x0), h1 = to_t<C>(x1);
    h[j] = h0;
    h[j + 1] = h1;
    l[j] = to_t<C>(x0 - to_f(h0));
    l[j + 1] = to_t<C>(x1 - to_f(h1));
  }
}
// every slot of h and l from f(slot), in pairs
template <int N, typename V, typename F>
__device__ __forceinline__ void split_all(V& h, V& l, F&& f) {
#pragma unroll
  for (int j = 0; j < N; j += 2) split_pair(f(j), f(j + 1), h, l, j);
}

// Inputs of a 16-bit projection: a chunk whose sum of squares reaches 65504^2 may hold a value beyond fp16's
// range; its fp16 copy is taken clamped to +-65504 (rarely taken; the norm keeps the true value, so a key of
// such a norm still gets the zero features exact arithmetic gives it, and nothing turns into inf or NaN).
constexpr float kF16Max = 65504.f;
constexpr float kF16MaxSq = 65504.f * 65504.f;
template <typename P, typename V8>
__device__ __forceinline__ void clamp_to_f16(const V8& x, vec8<P>& y) {
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = to_t<P>(__builtin_fminf(__builtin_fmaxf(to_f(x[j]), -kF16Max), kF16Max));
}

template <typename T> __device__ __forceinline__ vec8<T> zero8() {
  vec8<T> z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = to_t<T>(0.f);
  return z;
}

// Operand types per input type: the projection runs in fp16 for bf16 inputs (a bf16 value
// inside fp16's range converts exactly, and fp16's 11-bit significand keeps the rounding of
// the scaled Omega small enough for the exponent), the contraction with values in bf16;
// fp32 inputs use fp32 for both.
template <typename T> struct Ops;
template <> struct Ops<float> { using P = float; using C = float; };
template <> struct Ops<bf16> { using P = f16; using C = bf16; };

// 8 contiguous elements (16 B for 16-bit types, 32 B for fp32), 16-byte aligned.
template <typename T> __device__ __forceinline__ vec8<T> ld8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const vec8<T>*>(p);
  } else {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
    return r;
  }
}
template <typename T> __device__ __forceinline__ void st8(T* p, const vec8<T>& x) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<vec8<T>*>(p) = x;
  } else {
    f32x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = x[j]; b[j] = x[j + 4]; }
    reinterpret_cast<f32x4*>(p)[0] = a;
    reinterpret_cast<f32x4*>(p)[1] = b;
  }
}

// Eight stored sums (fp32, or bf16 where a partial sum is kept in half the bytes) as two fp32 quads, and back:
// element j of the eight is lo[j] for j < 4, hi[j - 4] otherwise. Stores round to nearest even.
template <typename S> __device__ __forceinline__ void ld8_f32(const S* p, f32x4& lo, f32x4& hi) {
  if constexpr (sizeof(S) == 4) {
    lo = reinterpret_cast<const f32x4*>(p)[0];
    hi = reinterpret_cast<const f32x4*>(p)[1];
  } else {
    const vec8<S> x = *reinterpret_cast<const vec8<S>*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = to_f(x[i]);
      hi[i] = to_f(x[i + 4]);
    }
  }
}
template <typename S> __device__ __forceinline__ void st8_f32(S* p, const f32x4& lo, const f32x4& hi) {
  if constexpr (sizeof(S) == 4) {
    reinterpret_cast<f32x4*>(p)[0] = lo;
    reinterpret_cast<f32x4*>(p)[1] = hi;
  } else {
    vec8<S> x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = to_t<S>(lo[i]);
      x[i + 4] = to_t<S>(hi[i]);
    }
    *reinterpret_cast<vec8<S>*>(p) = x;
  }
}
// Four stored sums as one fp32 quad, and back.
template <typename S> __device__ __forceinline__ f32x4 ld4_f32(const S* p) {
  if constexpr (sizeof(S) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    const vec4<S> x = *reinterpret_cast<const vec4<S>*>(p);
    return f32x4{to_f(x[0]), to_f(x[1]), to_f(x[2]), to_f(x[3])};
  }
}
template <typename S> __device__ __forceinline__ void st4_f32(S* p, const f32x4& v) {
  if constexpr (sizeof(S) == 4) {
    *reinterpret_cast<f32x4*>(p) = v;
  } else {
    vec4<S> x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_t<S>(v[i]);
    *reinterpret_cast<vec4<S>*>(p) = x;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Cross-lane exchanges on the VALU (no LDS round trip).
// permlane32_swap / permlane16_swap applied to (x, x) leave, in every lane, x and its
// partner across the 32-lane / 16-lane boundary in the two results (in some order), so a
// symmetric reduction of the pair is the xor-32 / xor-16 butterfly step.
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// DPP moves within a 16-lane row: row_ror:n rotates, quad_perm permutes inside quads.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppRor4 = 0x124, kDppRor8 = 0x128;

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppRor8>(x));
  x = fmaxf(x, dpp<kDppRor4>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppXor1>(x));
  return pair_max32(pair_max16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Reduce over the four lanes that share c (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_sum(float x) { return pair_sum32(pair_sum16(x)); }
__device__ __forceinline__ float group_max(float x) { return pair_max32(pair_max16(x)); }
// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, ..., 64).
template <int N> __device__ __forceinline__ float lanes_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRor8>(x);
  if constexpr (N >= 32) x = pair_sum16(x);
  if constexpr (N >= 64) x = pair_sum32(x);
  static_assert(N <= 64, "lanes_sum covers at most 64 lanes");
  return x;
}

template <int N> __device__ __forceinline__ float lanes_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kDppXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppRor8>(x));
  static_assert(N <= 16, "lanes_max covers at most 16 lanes");
  return x;
}

// Flattened work split: the B*H*ceil(L/32) token tiles, in (b,h)-major order, are cut
// into G contiguous pieces of nearly equal length. Piece i covers tiles
// [piece_start(i), piece_start(i+1)). A piece may span several (b,h); the part of
// piece i that lies in (b,h) bh is stored under index i + bh, which is unique because
// both indices only grow along the flattened order.
__host__ __device__ __forceinline__ long long piece_start(long long i, long long total, long long G) {
  return (i * total) / G;
}
__host__ __device__ __forceinline__ long long piece_of(long long t, long long total, long long G) {
  long long i = (t * G) / total;
  while (i + 1 < G && piece_start(i + 1, total, G) <= t) ++i;
  while (i > 0 && piece_start(i, total, G) > t) --i;
  return i;
}

// ---- asynchronous global -> LDS copies (gfx950 global_load_lds_dwordx4)
// Each active lane copies 16 bytes from its own global address to LDS byte address
// lds_base + 16 * lane (lds_base must be wave-uniform). The copy completes
// asynchronously and is counted by vmcnt like any vector memory load; the compiler
// does not track it, so the waits are placed explicitly with wait_vmcnt().
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  // an LDS DMA reading M0 right after an SALU write of M0 needs one wait state
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(base) : "memory");
}
// The same copy through a buffer resource: lane data = rsrc.base + voff, 16 bytes, and zero where the 16 bytes lie
// at or past rsrc's byte count (the hardware's range check), so the address arithmetic per copy is one offset that
// can stay fixed while the resource moves. rsrc must be the same across the wave's active lanes: the copy takes
// the first active lane's.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 raw_buffer(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);                                     // range in bytes
  r[3] = 0x00020000u;  // raw (unformatted) 32-bit data, no swizzle: the gfx9-family encoding
  return r;
}
__device__ __forceinline__ void lds_dma16_buf(const u32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(rsrc[0]);
  r[1] = __builtin_amdgcn_readfirstlane(rsrc[1]);
  r[2] = __builtin_amdgcn_readfirstlane(rsrc[2]);
  r[3] = __builtin_amdgcn_readfirstlane(rsrc[3]);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
               "s"(base)
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}
// Wait until at most n vector memory operations of this wave are outstanding (n < 64).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}
// Workgroup barrier that waits only for this wave's LDS traffic (no vector-memory drain),
// so asynchronous copies stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// gfx950 transposing LDS read: within each 16-lane group, lane r supplies the address of 4
// consecutive 16-bit elements M[r][0..3]; lane i receives M[i/4 + 4k][i%4] for k = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Map a launch-order block index so that consecutive logical indices land on
// the same XCD (the hardware deals workgroups to the 8 XCDs round robin), which
// keeps work that shares inputs inside one L2. Identity when n is not a
// multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if ((n & 7) != 0) return bid;
  return (bid & 7) * (n >> 3) + (bid >> 3);
}

}  // namespace favor
