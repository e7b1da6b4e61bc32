// C ABI of libfavor: argument checks, workspace sizing and dispatch to the HIP kernels.
// Every check runs before any launch; a failed check launches nothing.
#include "../../include/favor.h"
#include "favor_plan.hpp"

#include <cstdint>
#include <vector>

namespace favor_host {
void make_omega(uint64_t seed, int H, int m, int d, int mode, float* out);
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_dtype(favor_dtype t) { return t == FAVOR_F32 || t == FAVOR_BF16; }
bool valid_kind(favor_kind k) { return k == FAVOR_PRF || k == FAVOR_RELU || k == FAVOR_TRIG; }
bool valid_omega_mode(favor_omega_mode mode, int m) {
  if (mode == FAVOR_HYPERBOLIC || mode == FAVOR_TRIG_PAIRS) return m % 2 == 0;
  return mode == FAVOR_ORTHO_CHI || mode == FAVOR_IID || mode == FAVOR_ORTHO_SQRTD;
}

favor_status hip_status(hipError_t e) { return e == hipSuccess ? FAVOR_OK : FAVOR_ERR_HIP; }

// Shared checks for the sequence entry points (features / bidir / causal).
favor_status check_seq(const favor::Shape& s, favor_dtype dt, favor_kind kind, float eps) {
  if (s.B < 1 || s.H < 1 || s.L < 1 || s.d < 1 || s.dv < 1 || s.m < 1) return FAVOR_ERR_INVALID_ARG;
  if (!valid_dtype(dt) || !valid_kind(kind)) return FAVOR_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps != eps) return FAVOR_ERR_INVALID_ARG;
  if ((long long)s.B * s.H > (1LL << 24) || s.L > (1 << 28)) return FAVOR_ERR_INVALID_ARG;
  if ((long long)s.B * s.H * s.L * (s.d > s.dv ? s.d : s.dv) >= (1LL << 40)) return FAVOR_ERR_INVALID_ARG;
  return FAVOR_OK;
}

}  // namespace

extern "C" {

const char* favor_status_string(favor_status st) {
  switch (st) {
    case FAVOR_OK: return "ok";
    case FAVOR_ERR_INVALID_ARG: return "invalid argument";
    case FAVOR_ERR_UNSUPPORTED: return "unsupported shape (no kernel built for it)";
    case FAVOR_ERR_WORKSPACE: return "workspace too small";
    case FAVOR_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

favor_status favor_make_omega_host(uint64_t seed, int H, int m, int d, favor_omega_mode mode, float* omega_host) {
  if (!omega_host || H < 1 || H > 65536 || m < 1 || m > 4096 || d < 1 || d > 256) return FAVOR_ERR_INVALID_ARG;
  if (!valid_omega_mode(mode, m)) return FAVOR_ERR_INVALID_ARG;
  favor_host::make_omega(seed, H, m, d, static_cast<int>(mode), omega_host);
  return FAVOR_OK;
}

favor_status favor_make_omega(uint64_t seed, int H, int m, int d, favor_omega_mode mode, float* omega_dev,
                              hipStream_t stream) {
  if (!omega_dev || !aligned16(omega_dev)) return FAVOR_ERR_INVALID_ARG;
  if (H < 1 || H > 65536 || m < 1 || m > 4096 || d < 1 || d > 256) return FAVOR_ERR_INVALID_ARG;
  if (!valid_omega_mode(mode, m)) return FAVOR_ERR_INVALID_ARG;
  std::vector<float> host((size_t)H * m * d);
  favor_host::make_omega(seed, H, m, d, static_cast<int>(mode), host.data());
  hipError_t e = hipMemcpyAsync(omega_dev, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return FAVOR_ERR_HIP;
  return hip_status(hipStreamSynchronize(stream));
}

size_t favor_workspace_size(int causal, int B, int H, int L, int d, int dv, int m, favor_dtype dtype) {
  const favor::Shape s{B, H, L, d, dv, m};
  if (check_seq(s, dtype, FAVOR_PRF, 0.0f) != FAVOR_OK) return 0;
  if (!favor::shape_built(dtype, d, dv, m)) return 0;
  return causal ? favor::plan_causal(s, dtype).total : favor::plan_bidir(s, dtype).total;
}

favor_status favor_features(const void* x, const float* omega, int B, int H, int L, int d, int m, favor_dtype dtype,
                            favor_kind kind, float eps, float* phi, float* logscale, hipStream_t stream) {
  const favor::Shape s{B, H, L, d, 16, m};
  favor_status st = check_seq(s, dtype, kind, eps);
  if (st != FAVOR_OK) return st;
  if (!x || !omega || !phi || !logscale) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(omega) || !aligned16(phi) || !aligned16(logscale)) return FAVOR_ERR_INVALID_ARG;
  if (!(d == 16 || d == 32 || d == 64 || d == 128) || m % 16 != 0 || m > 512) return FAVOR_ERR_UNSUPPORTED;
  return hip_status(favor::launch_features(x, omega, s, dtype, kind, eps, phi, logscale, stream));
}

// Checks of the bidirectional entry points, everything but the workspace.
static favor_status check_bidir(const void* q, const void* k, const void* v, const float* omega,
                                const favor::Shape& s, int Lq, favor_dtype dtype, favor_kind kind, float eps,
                                int renormalize, void* out) {
  favor_status st = check_seq(s, dtype, kind, eps);
  if (st != FAVOR_OK) return st;
  if (Lq < 1 || Lq > (1 << 28)) return FAVOR_ERR_INVALID_ARG;
  if (!q || !k || !v || !omega || !out) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(omega) || !aligned16(out))
    return FAVOR_ERR_INVALID_ARG;
  const favor::KShape ks = favor::kernel_shape(dtype, s.d, s.dv, s.m);
  if (!ks.ok) return FAVOR_ERR_UNSUPPORTED;
  if (kind == FAVOR_TRIG && s.m % 2 != 0) return FAVOR_ERR_INVALID_ARG;
  if (kind == FAVOR_TRIG && (!renormalize || !ks.exact)) return FAVOR_ERR_UNSUPPORTED;
  return FAVOR_OK;
}

favor_status favor_bidir_cross(const void* q, const void* k, const void* v, const float* omega, int B, int H,
                               int Lq, int Lk, int d, int dv, int m, favor_dtype dtype, favor_kind kind, float eps,
                               int renormalize, int out_f32, void* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  const favor::Shape s{B, H, Lk, d, dv, m};
  favor_status st = check_bidir(q, k, v, omega, s, Lq, dtype, kind, eps, renormalize, out);
  if (st != FAVOR_OK) return st;
  if (!ws || !aligned16(ws)) return FAVOR_ERR_INVALID_ARG;
  if (ws_bytes < favor::plan_bidir(s, dtype).total) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_bidir(q, k, v, omega, s, Lq, renormalize ? 1 : 0, dtype, kind, eps,
                                        out_f32 ? 1 : 0, out, ws, stream));
}

favor_status favor_bidir_noalloc(const void* q, const void* k, const void* v, const float* omega, int B, int H,
                                 int L, int d, int dv, int m, favor_dtype dtype, favor_kind kind, float eps,
                                 int out_f32, void* out, hipStream_t stream) {
  const favor::Shape s{B, H, L, d, dv, m};
  favor_status st = check_bidir(q, k, v, omega, s, L, dtype, kind, eps, 1, out);
  if (st != FAVOR_OK) return st;
  if (favor::plan_bidir(s, dtype).total > FAVOR_BIDIR_NOALLOC_MAX_BYTES) return FAVOR_ERR_WORKSPACE;
  int dev = -1;
  hipDevice_t sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) return FAVOR_ERR_HIP;
  if (sdev != dev) return FAVOR_ERR_INVALID_ARG;  // the stream must belong to the current device
  void* ws = nullptr;
  if (favor::noalloc_scratch(dev, &ws) != hipSuccess) return FAVOR_ERR_HIP;
  return hip_status(favor::launch_bidir(q, k, v, omega, s, L, 1, dtype, kind, eps, out_f32 ? 1 : 0, out, ws, stream));
}

favor_status favor_bidir(const void* q, const void* k, const void* v, const float* omega, int B, int H, int L, int d,
                         int dv, int m, favor_dtype dtype, favor_kind kind, float eps, int out_f32, void* out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  return favor_bidir_cross(q, k, v, omega, B, H, L, L, d, dv, m, dtype, kind, eps, 1, out_f32, out, ws, ws_bytes,
                           stream);
}

size_t favor_omega_prepared_size(int H, int d, int dv, int m, favor_dtype dtype) {
  const favor::Shape s{1, H, 1, d, dv, m};
  if (check_seq(s, dtype, FAVOR_PRF, 0.0f) != FAVOR_OK) return 0;
  return favor::omega_prepared_bytes(s, dtype);
}

favor_status favor_omega_prepare(const float* omega, int H, int d, int dv, int m, favor_dtype dtype, favor_kind kind,
                                 void* prep, size_t prep_bytes, hipStream_t stream) {
  const favor::Shape s{1, H, 1, d, dv, m};
  favor_status st = check_seq(s, dtype, kind, 0.0f);
  if (st != FAVOR_OK) return st;
  if (!omega || !prep || !aligned16(omega) || !aligned16(prep)) return FAVOR_ERR_INVALID_ARG;
  const favor::KShape ks = favor::kernel_shape(dtype, d, dv, m);
  if (!ks.ok) return FAVOR_ERR_UNSUPPORTED;
  if (kind == FAVOR_TRIG && m % 2 != 0) return FAVOR_ERR_INVALID_ARG;
  if (kind == FAVOR_TRIG && !ks.exact) return FAVOR_ERR_UNSUPPORTED;
  if (prep_bytes < favor::omega_prepared_bytes(s, dtype)) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_prepare_omega(omega, s, dtype, kind, prep, stream));
}

favor_status favor_bidir_prepared(const void* q, const void* k, const void* v, const void* prep, int B, int H, int L,
                                  int d, int dv, int m, favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                                  void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const favor::Shape s{B, H, L, d, dv, m};
  favor_status st = check_bidir(q, k, v, static_cast<const float*>(prep), s, L, dtype, kind, eps, 1, out);
  if (st != FAVOR_OK) return st;
  if (!ws || !aligned16(ws)) return FAVOR_ERR_INVALID_ARG;
  if (ws_bytes < favor::plan_bidir(s, dtype).total) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_bidir(q, k, v, nullptr, s, L, 1, dtype, kind, eps, out_f32 ? 1 : 0, out, ws, stream,
                                        prep));
}

size_t favor_backward_workspace_size(int B, int H, int L, int d, int dv, int m, favor_dtype dtype) {
  const favor::Shape s{B, H, L, d, dv, m};
  if (check_seq(s, dtype, FAVOR_PRF, 0.f) != FAVOR_OK) return 0;
  return favor::plan_backward(s, dtype).total;
}

favor_status favor_bidir_backward(const void* q, const void* k, const void* v, const float* omega,
                                  const void* dout, int B, int H, int L, int d, int dv, int m, favor_dtype dtype,
                                  favor_kind kind, float eps, int grad_f32, void* dq, void* dk, void* dv_, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  const favor::Shape s{B, H, L, d, dv, m};
  favor_status st = check_seq(s, dtype, kind, eps);
  if (st != FAVOR_OK) return st;
  if (!q || !k || !v || !omega || !dout || !dq || !dk || !dv_ || !ws) return FAVOR_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, (const void*)omega, dout, (const void*)dq, (const void*)dk, (const void*)dv_,
                        (const void*)ws})
    if (!aligned16(p)) return FAVOR_ERR_INVALID_ARG;
  if (kind != FAVOR_PRF && kind != FAVOR_RELU) return FAVOR_ERR_UNSUPPORTED;
  if (!favor::bwd_shape_built(d, dv, m)) return FAVOR_ERR_UNSUPPORTED;
  if (ws_bytes < favor::plan_backward(s, dtype).total) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_backward(q, k, v, omega, dout, s, dtype, kind, eps, grad_f32 ? 1 : 0, dq, dk, dv_,
                                           ws, stream));
}

size_t favor_causal_backward_workspace_size(int B, int H, int L, int d, int dv, int m, favor_dtype dtype) {
  const favor::Shape s{B, H, L, d, dv, m};
  if (check_seq(s, dtype, FAVOR_PRF, 0.f) != FAVOR_OK) return 0;
  return favor::plan_causal_backward(s, dtype).total;
}

favor_status favor_causal_backward(const void* q, const void* k, const void* v, const float* omega,
                                   const void* dout, int B, int H, int L, int d, int dv, int m, favor_dtype dtype,
                                   favor_kind kind, float eps, int grad_f32, void* dq, void* dk, void* dv_, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  const favor::Shape s{B, H, L, d, dv, m};
  favor_status st = check_seq(s, dtype, kind, eps);
  if (st != FAVOR_OK) return st;
  if (!q || !k || !v || !omega || !dout || !dq || !dk || !dv_ || !ws) return FAVOR_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, (const void*)omega, dout, (const void*)dq, (const void*)dk, (const void*)dv_,
                        (const void*)ws})
    if (!aligned16(p)) return FAVOR_ERR_INVALID_ARG;
  if (kind != FAVOR_PRF && kind != FAVOR_RELU) return FAVOR_ERR_UNSUPPORTED;
  if (!favor::bwd_shape_built(d, dv, m)) return FAVOR_ERR_UNSUPPORTED;
  if (ws_bytes < favor::plan_causal_backward(s, dtype).total) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_causal_backward(q, k, v, omega, dout, s, dtype, kind, eps, grad_f32 ? 1 : 0, dq, dk, dv_,
                                                  ws, stream));
}

// favor_causal (omega) and favor_causal_prepared (prep): exactly one of the two is non-null.
static favor_status causal_common(const void* q, const void* k, const void* v, const float* omega, const void* prep,
                                  int B, int H, int L, int d, int dv, int m, favor_dtype dtype, favor_kind kind,
                                  float eps, int out_f32, void* out, float* S_final, float* z_final, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  if (!omega) omega = static_cast<const float*>(prep);  // checked like omega
  const favor::Shape s{B, H, L, d, dv, m};
  favor_status st = check_seq(s, dtype, kind, eps);
  if (st != FAVOR_OK) return st;
  if (!q || !k || !v || !omega || !out || !ws) return FAVOR_ERR_INVALID_ARG;
  if ((S_final == nullptr) != (z_final == nullptr)) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(omega) || !aligned16(out) || !aligned16(ws))
    return FAVOR_ERR_INVALID_ARG;
  if (S_final && (!aligned16(S_final) || !aligned16(z_final))) return FAVOR_ERR_INVALID_ARG;
  if (!favor::shape_built(dtype, d, dv, m)) return FAVOR_ERR_UNSUPPORTED;
  if (kind == FAVOR_TRIG && m % 2 != 0) return FAVOR_ERR_INVALID_ARG;
  if (kind == FAVOR_TRIG && !favor::kernel_shape(dtype, d, dv, m).exact) return FAVOR_ERR_UNSUPPORTED;
  if (S_final && (kind != FAVOR_PRF || d > 64)) return FAVOR_ERR_UNSUPPORTED;
  if (ws_bytes < favor::plan_causal(s, dtype).total) return FAVOR_ERR_WORKSPACE;
  return hip_status(favor::launch_causal(q, k, v, prep ? nullptr : omega, s, dtype, kind, eps, out_f32 ? 1 : 0, out,
                                         S_final, z_final, ws, stream, prep));
}

favor_status favor_causal(const void* q, const void* k, const void* v, const float* omega, int B, int H, int L, int d,
                          int dv, int m, favor_dtype dtype, favor_kind kind, float eps, int out_f32, void* out,
                          float* S_final, float* z_final, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!omega) return FAVOR_ERR_INVALID_ARG;
  return causal_common(q, k, v, omega, nullptr, B, H, L, d, dv, m, dtype, kind, eps, out_f32, out, S_final, z_final,
                       ws, ws_bytes, stream);
}

favor_status favor_causal_prepared(const void* q, const void* k, const void* v, const void* prep, int B, int H, int L,
                                   int d, int dv, int m, favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                                   void* out, float* S_final, float* z_final, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!prep) return FAVOR_ERR_INVALID_ARG;
  return causal_common(q, k, v, nullptr, prep, B, H, L, d, dv, m, dtype, kind, eps, out_f32, out, S_final, z_final,
                       ws, ws_bytes, stream);
}

static favor_status decode_common(const void* q, const void* k, const void* v, const float* omega, float* S,
                                  float* z, const float* gate, const float* inw, int N, int H, int d, int dv, int m,
                                  favor_dtype dtype, favor_kind kind, float eps, float* out, hipStream_t stream) {
  if (N < 1 || H < 1 || (long long)N * H > (1LL << 24)) return FAVOR_ERR_INVALID_ARG;
  if (!valid_dtype(dtype) || !valid_kind(kind) || !(eps >= 0.0f)) return FAVOR_ERR_INVALID_ARG;
  if (d < 1 || dv < 1 || m < 1) return FAVOR_ERR_INVALID_ARG;
  if (!q || !k || !v || !omega || !S || !z || !out) return FAVOR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(omega) || !aligned16(S) || !aligned16(z) ||
      !aligned16(out))
    return FAVOR_ERR_INVALID_ARG;
  if (!(d == 16 || d == 32 || d == 64)) return FAVOR_ERR_UNSUPPORTED;
  if (dv % 16 != 0 || dv < 16 || dv > 256) return FAVOR_ERR_UNSUPPORTED;
  if (m % 16 != 0 || m > 1024) return FAVOR_ERR_UNSUPPORTED;
  return hip_status(
      favor::launch_decode(q, k, v, omega, S, z, N, H, d, dv, m, dtype, kind, eps, gate, inw, out, stream));
}

favor_status favor_decode(const void* q, const void* k, const void* v, const float* omega, float* S, float* z, int N,
                          int H, int d, int dv, int m, favor_dtype dtype, favor_kind kind, float eps, float* out,
                          hipStream_t stream) {
  return decode_common(q, k, v, omega, S, z, nullptr, nullptr, N, H, d, dv, m, dtype, kind, eps, out, stream);
}

favor_status favor_decode_gated(const void* q, const void* k, const void* v, const float* omega, float* S, float* z,
                                const float* gate, const float* in_weight, int N, int H, int d, int dv, int m,
                                favor_dtype dtype, favor_kind kind, float eps, float* out, hipStream_t stream) {
  if (!gate || !aligned4(gate) || (in_weight && !aligned4(in_weight))) return FAVOR_ERR_INVALID_ARG;
  return decode_common(q, k, v, omega, S, z, gate, in_weight, N, H, d, dv, m, dtype, kind, eps, out, stream);
}

}  // extern "C"
