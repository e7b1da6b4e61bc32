// Host-side launch plans and workspace layouts (shared by the size query and the launchers).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

// (d, dv, m) combinations with compiled kernels for the sequence entry points.
#define FAVOR_SHAPES(X) \
  X(16, 16, 16)         \
  X(16, 16, 32)         \
  X(16, 16, 64)         \
  X(16, 16, 128)        \
  X(16, 16, 256)        \
  X(32, 32, 64)         \
  X(32, 32, 128)        \
  X(64, 64, 64)         \
  X(64, 64, 128)        \
  X(64, 64, 256)

// Compiled (d, dv, m) of the general kernels (value columns in groups of 64, runtime feature count
// up to the capacity m), for the shapes FAVOR_SHAPES does not list (its shapes keep their exact
// kernels, without the general kernels' masking). At d = 128 the smallest capacity
// is 64 (two waves: one wave would have more tile copies in flight than it can count).
#define FAVOR_GENERAL_SHAPES(X) \
  X(16, 64, 32)                 \
  X(16, 64, 64)                 \
  X(16, 64, 128)                \
  X(16, 64, 256)                \
  X(16, 64, 512)                \
  X(32, 64, 32)                 \
  X(32, 64, 64)                 \
  X(32, 64, 128)                \
  X(32, 64, 256)                \
  X(32, 64, 512)                \
  X(64, 64, 32)                 \
  X(64, 64, 64)                 \
  X(64, 64, 128)                \
  X(64, 64, 256)                \
  X(64, 64, 512)                \
  X(128, 64, 64)                \
  X(128, 64, 128)               \
  X(128, 64, 256)               \
  X(128, 64, 512)

// (d, dv, m) combinations with compiled kernels for the bidirectional backward.
#define FAVOR_BWD_SHAPES(X) \
  X(16, 16, 32)             \
  X(32, 32, 64)             \
  X(64, 64, 128)            \
  X(64, 64, 256)

namespace favor {

struct Shape {
  int B, H, L, d, dv, m;
  long long bh() const { return (long long)B * H; }
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t elt(int dtype) { return dtype == 0 ? 4 : 2; }

// Waves of the key/value reduction for m features at projection width d (m: the compiled
// feature capacity); the device-side split (RedSplit) follows the same rule.
#ifndef FAVOR_REDUCE_WAVES
#define FAVOR_REDUCE_WAVES 4
#endif
inline int reduce_waves(int m, int d) {
  const int base = m < 32 ? 1 : ((m / 32) < FAVOR_REDUCE_WAVES ? (m / 32) : FAVOR_REDUCE_WAVES);
  const int fpw = d > 64 ? 32 : 64;
  return m / base > fpw ? (m / fpw < 8 ? m / fpw : 8) : base;
}

// Waves of the query-side kernels for m features at projection width d (the device-side FeatSplit): up to
// four waves of up to 64 features (32 at d = 128), then up to eight.
inline int output_waves(int m, int d) {
  const int base = (m / 16) < 4 ? (m / 16) : 4;
  const int fpw = d > 64 ? 32 : 64;
  return m / base > fpw ? (m / fpw < 8 ? m / fpw : 8) : base;
}

// Bidirectional path: omega fragments, per-segment partial (S, z) sums with their
// stabiliser maxima, and the combined S fragments.
// Both passes walk the B*H*ceil(L/32) token tiles split into G contiguous pieces (one
// workgroup each); partials are stored per (piece, b*h) intersection.
struct BidirPlan {
  int tpb = 0, G = 0, nw_reduce = 0;  // key side (the reduction)
  long long T_all = 0;
  int tpb_q = 0, G_q = 0;             // query side (the output)
  long long T_all_q = 0;
  size_t off_omf = 0, off_part = 0, off_zpart = 0, off_pmax = 0, off_sfr = 0, off_gmax = 0, total = 0;
};

// Causal path: Omega fragments, one partial (S, z) sum per (b*h, segment) in MFMA fragment
// layout with its stabiliser maxima, the exclusive prefix over segments (carries) in the same
// layout, and the carries' common key maxima.
struct CausalPlan {
  int nseg = 0, seg_len = 0, tpb = 0, G = 0, nw_reduce = 0;
  long long T_all = 0;
  size_t off_omf = 0, off_part = 0, off_zpart = 0, off_pmax = 0, off_cpart = 0, off_cz = 0, off_cmax = 0,
         total = 0;
};

// Bidirectional backward: Omega' fragments and their residuals (the projections run through both),
// the forward reduction's pieces and partials, S_aug rows, the backward's own pieces (G, one
// workgroup per CU) and their dS_aug partials, dS_aug rows.
struct BackwardPlan {
  int tpb = 0, G_red = 0, G = 0, nw_reduce = 0;
  long long T_all = 0;
  size_t off_omf = 0, off_omlo = 0, off_omt = 0, off_part = 0, off_zpart = 0, off_pmax = 0, off_srow = 0,
         off_gmax = 0, off_dpart = 0, off_dzpart = 0, off_dsrow = 0, total = 0;
};

// Causal backward: the forward's causal plan (Omega fragments, segment partials, carries and key
// maxima), the Omega' fragments' residuals, Omega'^T fragments (hi and lo parts), per-query l and
// gamma, and one [m][dv+16] fp32 block per segment (the query-side totals, then the suffix carries
// in place).
struct CausalBackwardPlan {
  CausalPlan f;
  size_t off_omlo = 0, off_omth = 0, off_omtl = 0, off_lg = 0, off_gam = 0, off_trow = 0, total = 0;
};

// The compiled kernels a call of the sequence entry points runs on: its own (d, dv, m) when FAVOR_SHAPES
// lists it (exact), else the general kernels (d, 64, mk) with mk the next of 32 (64 at d = 128), 64, 128,
// 256, 512 at or above m, dv covered by column groups of up to 64. Valid for d in {16, 32, 64, 128} and multiples of 16
// dv <= 256, m <= 512 (ok = false otherwise).
struct KShape {
  int dk = 0, dvk = 0, mk = 0;
  bool exact = false, ok = false;
};
KShape kernel_shape(int dtype, int d, int dv, int m);
// fp32 inputs on the general kernels: d <= 64 and a feature capacity of at most 256 (fp32 operands
// take twice the registers and LDS of the 16-bit ones; larger fp32 shapes are not built).
constexpr bool fp32_built(bool general, int d, int mk) { return !general || (d <= 64 && mk <= 256); }
bool shape_built(int dtype, int d, int dv, int m);
bool bwd_shape_built(int d, int dv, int m);
BackwardPlan plan_backward(const Shape& s, int dtype);
// s.L is the key length; Lq > 0 sets a different query length (cross attention).
BidirPlan plan_bidir(const Shape& s, int dtype, int Lq = 0);
CausalPlan plan_causal(const Shape& s, int dtype);
CausalBackwardPlan plan_causal_backward(const Shape& s, int dtype);

hipError_t launch_features(const void* x, const float* omega, const Shape& s, int dtype, int kind, float eps,
                           float* phi, float* logscale, hipStream_t st);
// prep: Omega' fragments written by launch_prepare_omega for the same (H, d, dv, m, dtype, kind), read in place
// of converting omega on the call (omega is then unused); null: convert omega into the workspace.
hipError_t launch_bidir(const void* q, const void* k, const void* v, const float* omega, const Shape& s, int Lq,
                        int renorm, int dtype, int kind, float eps, int out_f32, void* out, void* ws,
                        hipStream_t st, const void* prep = nullptr);
hipError_t launch_causal(const void* q, const void* k, const void* v, const float* omega, const Shape& s,
                         int dtype, int kind, float eps, int out_f32, void* out, float* S_final, float* z_final,
                         void* ws, hipStream_t st, const void* prep = nullptr);
// Bytes of the Omega' fragments of the compiled kernels for (H, d, dv, m) (Shape's B and L unused), the same
// area both plans reserve at offset 0 of their workspace; and their conversion from omega.
size_t omega_prepared_bytes(const Shape& s, int dtype);
hipError_t launch_prepare_omega(const float* omega, const Shape& s, int dtype, int kind, void* prep, hipStream_t st);
hipError_t launch_backward(const void* q, const void* k, const void* v, const float* omega, const void* dout,
                           const Shape& s, int dtype, int kind, float eps, int grad_f32, void* dq, void* dk, void* dv,
                           void* ws, hipStream_t st);
hipError_t launch_causal_backward(const void* q, const void* k, const void* v, const float* omega, const void* dout,
                                  const Shape& s, int dtype, int kind, float eps, int grad_f32, void* dq, void* dk,
                                  void* dv, void* ws, hipStream_t st);
// Device address of the library's own workspace array (FAVOR_BIDIR_NOALLOC_MAX_BYTES) on device `dev`, which
// must be the current device; resolved on the first call for that device.
hipError_t noalloc_scratch(int dev, void** ptr);
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* omega, float* S, float* z,
                         int N, int H, int d, int dv, int m, int dtype, int kind, float eps, const float* gate,
                         const float* inw, float* out, hipStream_t st);

}  // namespace favor
