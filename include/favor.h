/*
 * favor.h — C ABI of libfavor, FAVOR+ random-feature attention on MI355X (gfx950).
 *
 * The method (Performer paper, "Rethinking Attention with Performers"):
 *   x = q * d^(-1/4), y = k * d^(-1/4)                      (section 2.3, under eq. 6)
 *   phi_r(x) = exp(omega_r . x - |x|^2 / 2) / sqrt(m)        (Lemma 1, eq. 7; eq. 5)
 *   bidirectional: out_i = phi(q_i) . S / phi(q_i) . z,      (eq. 4; Algorithm 1)
 *                  S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j)
 *   causal:        the same with the sums over j <= i        (appendix B.1, eq. 11)
 *   decode:        S += phi(k) v^T, z += phi(k), then out = phi(q).S / phi(q).z
 *                  (the recurrent form of the causal sums; linear-attention blog,
 *                  "Autoregressive Generation"; RFA summary page, appendix A.3)
 * A ReLU feature map phi_r(x) = max(omega_r . x, 0) / sqrt(m) + eps (eq. 5 with
 * f = ReLU; appendix A.4) is selectable.
 *
 * Conventions shared by every entry point
 *   - Layouts are dense row-major: q, k [B,H,L,d]; v [B,H,L,dv]; out [B,H,L,dv];
 *     omega [H,m,d] fp32 (one random-feature matrix per head).
 *   - Device pointers must be 16-byte aligned. The caller owns every buffer;
 *     the library allocates no device memory and keeps no state between calls
 *     (except favor_bidir_noalloc's workspace array, described there).
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and the call returns without waiting. FAVOR_ERR_HIP reports a launch
 *     error; errors inside kernels surface at the caller's next synchronisation.
 *   - Arguments are checked before anything is launched. Bad arguments return
 *     FAVOR_ERR_INVALID_ARG, a valid but unbuilt shape FAVOR_ERR_UNSUPPORTED,
 *     a short workspace FAVOR_ERR_WORKSPACE; nothing is launched in those cases
 *     and output buffers are untouched. There is no fallback path.
 *   - Non-finite inputs are not checked; they propagate.
 *   - q and k are raw: the d^(-1/4) scaling happens inside the library.
 *   - The stabilisers (a constant per query row: a norm bound max_r|omega_r||x|
 *     or the exact row maximum; one constant per (b,h) for keys, or per segment
 *     prefix in the causal form) cancel exactly in the ratio, so results equal
 *     the unstabilised definitions up to rounding.
 *   - bf16 inputs are projected in fp16 (exact for 2^-14 <= |x| < 65504). Components
 *     of magnitude 65504 or more are clamped to +-65504 for the projection only (the
 *     norm term keeps the true value): keys of such norms get the zero features exact
 *     arithmetic gives them, and such a query is projected along its clamped direction.
 */
#ifndef FAVOR_H
#define FAVOR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAVOR_OK = 0,
  FAVOR_ERR_INVALID_ARG = 1,
  FAVOR_ERR_UNSUPPORTED = 2,
  FAVOR_ERR_WORKSPACE = 3,
  FAVOR_ERR_HIP = 4
} favor_status;

/* Element type of q, k, v (and of out for favor_bidir / favor_causal unless out_f32).
 * Arithmetic: FAVOR_F32 projects and contracts in fp32 (fp32 MFMA);
 * FAVOR_BF16 projects and contracts on bf16 MFMA with fp32 accumulation. */
typedef enum { FAVOR_F32 = 0, FAVOR_BF16 = 1 } favor_dtype;

/* Feature map: positive softmax features (Lemma 1), ReLU features (appendix A.4) or
 * trigonometric features (equation 5 with h(x) = exp(|x|^2/2), f1 = sin, f2 = cos; section
 * 2.3's SM^trig). FAVOR_TRIG (m even): feature r < m/2 is sin(omega_r.x), feature r >= m/2 is
 * cos(omega_r.x), scaled by exp(|x|^2/2)/sqrt(m/2); with an Omega of FAVOR_TRIG_PAIRS (the
 * same m/2 vectors twice) these are the sine and cosine features of m/2 vectors. Supported by
 * favor_features and favor_bidir / favor_bidir_cross (renormalize = 1); the projection of
 * every token must stay within 1600 radians (the hardware cosine's range). Trigonometric
 * features can be negative, so the denominators of the ratio can vanish (section 2.3). */
typedef enum { FAVOR_PRF = 0, FAVOR_RELU = 1, FAVOR_TRIG = 2 } favor_kind;

/* Omega rows: orthogonal blocks with chi(d) lengths (section 2.4, appendix B.2/F.4),
 * independent Gaussian rows, or orthogonal rows of length sqrt(d) (SMREG, section 2.3).
 * FAVOR_HYPERBOLIC (m even): the m/2 rows of FAVOR_ORTHO_CHI, then their negatives; with
 * FAVOR_PRF every entry point then computes the hyperbolic positive features of Lemma 1
 * (second form): exp(-|x|^2/2)/sqrt(m) (exp(w_i.x), exp(-w_i.x)) for the m/2 vectors w_i.
 * FAVOR_TRIG_PAIRS (m even): the m/2 rows of FAVOR_ORTHO_CHI, then the same rows again, for
 * FAVOR_TRIG. */
typedef enum {
  FAVOR_ORTHO_CHI = 0,
  FAVOR_IID = 1,
  FAVOR_ORTHO_SQRTD = 2,
  FAVOR_HYPERBOLIC = 3,
  FAVOR_TRIG_PAIRS = 4
} favor_omega_mode;

/* favor_make_omega — random features omega [H,m,d] fp32 into device memory.
 * Section 2.4 and appendix B.2 of the Performer paper: for each head, ceil(m/d)
 * independent d x d Gaussian blocks, rows orthogonalised by Gram-Schmidt, row r
 * rescaled by an independent chi(d) length (marginally N(0, I_d), appendix F.4);
 * rows past m are dropped. Computed on the host in fp64 from a counter-based
 * SplitMix64 stream keyed by (seed, head, block) and rounded to fp32, so the
 * bits depend only on (seed, H, m, d, mode): head h's rows do not depend on H.
 * Then copied with hipMemcpyAsync on `stream` (the host buffer stays alive
 * until the copy completes: the call synchronises `stream` before returning).
 * Requires 1 <= d <= 256, 1 <= m <= 4096, 1 <= H <= 65536 (m even for FAVOR_HYPERBOLIC and
 * FAVOR_TRIG_PAIRS). */
favor_status favor_make_omega(uint64_t seed, int H, int m, int d, favor_omega_mode mode,
                              float* omega_dev, hipStream_t stream);

/* favor_make_omega_host — the same bits into caller-owned host memory [H,m,d]. No GPU needed. */
favor_status favor_make_omega_host(uint64_t seed, int H, int m, int d, favor_omega_mode mode,
                                   float* omega_host);

/* favor_features — the feature map alone (Lemma 1 / eq. 5) for x [B,H,L,d] (raw q or k).
 * Writes phi [B,H,L,m] fp32 and logscale [B,H,L] fp32 with the true feature
 *   phi_true[b,h,l,r] = phi[b,h,l,r] * exp(logscale[b,h,l]).
 * PRF: phi is exp(omega_r.x - max_r' omega_r'.x) / sqrt(m) (each row's largest
 * entry is 1/sqrt(m)) and logscale = max_r omega_r.x - |x|^2/2, so no row over- or
 * underflows. RELU: phi = max(omega_r.x, 0)/sqrt(m) + eps and logscale = 0. TRIG: phi is
 * sin or cos(omega_r.x) / sqrt(m/2) and logscale = |x|^2/2.
 * Supported: d in {16, 32, 64, 128}, m a multiple of 16 up to 512. */
favor_status favor_features(const void* x, const float* omega, int B, int H, int L, int d, int m,
                            favor_dtype dtype, favor_kind kind, float eps,
                            float* phi, float* logscale, hipStream_t stream);

/* favor_bidir — bidirectional FAVOR+ (eq. 4, Algorithm 1 with C = [V 1]).
 * out [B,H,L,dv] in the input dtype (bf16 rounded to nearest even), or fp32
 * when out_f32 != 0. ws: device scratch of at least
 * favor_workspace_size(0, B, H, L, d, dv, m, dtype) bytes; its contents on
 * entry do not matter and are garbage on exit.
 * Shapes: d in {16, 32, 64, 128}; dv a multiple of 16 with 16 <= dv <= 256 (independent of d);
 * m a multiple of 16 with 16 <= m <= 512. fp32 inputs: d <= 64 and m <= 256, besides the exact
 * shapes below. Others return FAVOR_ERR_UNSUPPORTED. Exact kernels exist for (d, dv, m) = (16,16,16)
 * (16,16,32) (16,16,64) (16,16,128) (16,16,256) (32,32,64) (32,32,128) (64,64,64) (64,64,128)
 * (64,64,256); every other shape runs on general kernels (m rounded up to 32, 64, ..., 512 inside
 * them with the extra features masked; v and out taken in column groups of 64), which cost more
 * per token. FAVOR_TRIG only on the exact shapes. */
favor_status favor_bidir(const void* q, const void* k, const void* v, const float* omega,
                         int B, int H, int L, int d, int dv, int m,
                         favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                         void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* favor_bidir_noalloc — favor_bidir without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, results, shapes and checks as favor_bidir, and the same kernels. The workspace is
 * an array of FAVOR_BIDIR_NOALLOC_MAX_BYTES inside the library, one per device, which each device holds from
 * the first call on it until the process ends. Calls whose workspace (favor_workspace_size(0, ...)) exceeds it
 * return FAVOR_ERR_WORKSPACE and launch nothing. `stream` must belong to the current device
 * (FAVOR_ERR_INVALID_ARG otherwise). Every call on one device shares that device's array: calls that overlap
 * on one device (on different streams, or from several threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe. The array needs no clearing between calls. */
#define FAVOR_BIDIR_NOALLOC_MAX_BYTES ((size_t)64 << 20)
favor_status favor_bidir_noalloc(const void* q, const void* k, const void* v, const float* omega,
                                 int B, int H, int L, int d, int dv, int m,
                                 favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                                 void* out, hipStream_t stream);

/* favor_bidir_cross — bidirectional FAVOR+ between Lq queries and Lk keys (the RFA
 * page's cross-attention procedure; Performer Algorithm 1 with Q' of Lq rows and K' of
 * Lk rows), with the renormaliser D^-1 optional (Performer appendices A.3 and D.3,
 * "renormalize"): q [B,H,Lq,d], k [B,H,Lk,d], v [B,H,Lk,dv], out [B,H,Lq,dv].
 *   renormalize != 0: out_i = phi(q_i).S / phi(q_i).z   (as favor_bidir)
 *   renormalize == 0: out_i = phi(q_i).S with S = sum_j phi(k_j) v_j^T and the features
 *     in canonical scale, phi = exp(omega.x - |x|^2/2)/sqrt(m) (PRF) or
 *     max(omega.x, 0)/sqrt(m) + eps (ReLU); the stabilisers are undone exactly
 *     (FAVOR_TRIG: FAVOR_ERR_UNSUPPORTED).
 * Workspace: favor_workspace_size(0, B, H, Lk, d, dv, m, dtype). Built shapes, dtypes,
 * errors as favor_bidir, and 1 <= Lq <= 2^28. favor_bidir(..., L, ...) is
 * favor_bidir_cross(..., L, L, ..., renormalize = 1, ...). */
favor_status favor_bidir_cross(const void* q, const void* k, const void* v, const float* omega,
                               int B, int H, int Lq, int Lk, int d, int dv, int m,
                               favor_dtype dtype, favor_kind kind, float eps, int renormalize,
                               int out_f32, void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* favor_causal — unidirectional FAVOR+ (appendix B.1 eq. 11: prefix sums including
 * the diagonal) as a chunked scan. Same arguments and shapes as favor_bidir
 * (workspace from favor_workspace_size(1, ...)). If S_final [B,H,m,dv] and
 * z_final [B,H,m] (fp32, both or neither) are non-NULL, the state after the last
 * token is written in canonical (unstabilised) scale: exactly what
 * favor_decode continues from. Canonical state needs PRF with d <= 64
 * (exp(omega.x - |x|^2/2) <= exp(|omega|^2/2) stays inside fp32). FAVOR_TRIG
 * (equation 5's sin/cos features over a FAVOR_TRIG_PAIRS Omega) as favor_bidir: m even,
 * exact shapes only, and no final state (FAVOR_ERR_UNSUPPORTED with S_final). */
favor_status favor_causal(const void* q, const void* k, const void* v, const float* omega,
                          int B, int H, int L, int d, int dv, int m,
                          favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                          void* out, float* S_final, float* z_final,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Prepared random features. Omega stays fixed over many calls (the Performer paper redraws it
 * only periodically, section 4.2 with Figure 5, appendix B.2), while favor_bidir and favor_causal convert it into
 * the kernels' scaled MFMA fragments on every call. favor_omega_prepare does that conversion
 * once into a caller buffer `prep` of at least favor_omega_prepared_size(H, d, dv, m, dtype)
 * bytes (0 for invalid or unbuilt sizes; the fragments depend on the compiled kernel, hence dv);
 * favor_bidir_prepared and favor_causal_prepared then read `prep` in place of omega and are
 * otherwise favor_bidir and favor_causal (same workspace, checks, errors and bit-identical
 * outputs). `prep` must come from favor_omega_prepare with the same H, d, dv, m, dtype and kind
 * (the library cannot check this; another one gives wrong outputs, not an error); it is only read,
 * so any number of calls may share it, and it stays valid until omega changes. Stream-ordered:
 * prepare on the stream of the calls, or synchronise first. prep_bytes too small:
 * FAVOR_ERR_WORKSPACE; FAVOR_TRIG as favor_bidir (exact shapes only). */
size_t favor_omega_prepared_size(int H, int d, int dv, int m, favor_dtype dtype);
favor_status favor_omega_prepare(const float* omega, int H, int d, int dv, int m, favor_dtype dtype,
                                 favor_kind kind, void* prep, size_t prep_bytes, hipStream_t stream);
favor_status favor_bidir_prepared(const void* q, const void* k, const void* v, const void* prep,
                                  int B, int H, int L, int d, int dv, int m,
                                  favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                                  void* out, void* ws, size_t ws_bytes, hipStream_t stream);
favor_status favor_causal_prepared(const void* q, const void* k, const void* v, const void* prep,
                                   int B, int H, int L, int d, int dv, int m,
                                   favor_dtype dtype, favor_kind kind, float eps, int out_f32,
                                   void* out, float* S_final, float* z_final,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* favor_decode — one recurrent step for N sequences x H heads (the causal sums
 * advanced by one token; token t's output reads the state that includes t).
 * q, k [N,H,d], v [N,H,dv] in `dtype`; S [N,H,m,dv] and z [N,H,m] fp32 in canonical
 * scale, updated in place; out [N,H,dv] fp32.
 * Requires d in {16, 32, 64}, dv a multiple of 16 in [16, 256], m a multiple of 16
 * with m <= 1024 (other values: FAVOR_ERR_UNSUPPORTED). FAVOR_TRIG (over a
 * FAVOR_TRIG_PAIRS Omega): the state holds the canonical features sin/cos(omega.k)
 * exp(|k|^2/2)/sqrt(m/2) (k scaled by d^-1/4), finite while |k|^2 d^-1/2 < 176. */
favor_status favor_decode(const void* q, const void* k, const void* v, const float* omega,
                          float* S, float* z, int N, int H, int d, int dv, int m,
                          favor_dtype dtype, favor_kind kind, float eps,
                          float* out, hipStream_t stream);

/* favor_decode_gated — the decode step with recency gating (RFA page, section 3.2,
 * RFA-GATE: the historical state decays by a scalar gate computed from the step's
 * input, in both the value state and the normalisation state). Per (sequence, head)
 * pair p = n*H + h, with g = gate[p] and w = in_weight[p] (w = 1 if in_weight is NULL):
 *   S = g*S + w*phi(k) v^T,  z = g*z + w*phi(k),  out = phi(q).S / phi(q).z
 * (RFA's own form uses w = 1 - g). gate and in_weight are fp32 device arrays [N,H],
 * 4-byte aligned, read once; the gate network itself is the caller's. Everything else
 * as favor_decode; gate == NULL is FAVOR_ERR_INVALID_ARG. With every g = w = 1 the
 * result equals favor_decode's. */
favor_status favor_decode_gated(const void* q, const void* k, const void* v, const float* omega,
                                float* S, float* z, const float* gate, const float* in_weight,
                                int N, int H, int d, int dv, int m,
                                favor_dtype dtype, favor_kind kind, float eps,
                                float* out, hipStream_t stream);

/* favor_bidir_backward — gradients of favor_bidir's output (Performer equation 4 /
 * Algorithm 1; the pages time forward and backward, section 4.1) with respect to the raw
 * q, k and v, for positive softmax features (FAVOR_PRF) or the ReLU features of appendix A.4
 * (FAVOR_RELU, with the forward's eps; FAVOR_TRIG returns FAVOR_ERR_UNSUPPORTED), given
 * dout [B,H,L,dv] = dLoss/dout in `dtype`. The forward's sums are recomputed. The chain rule
 * through out = (Phi_Q S)/(Phi_Q z), xs = d^-1/4 x:
 *   W_i = [dout_i, -(dout_i . out_i)] / (Phi_Q z)_i,  dPhi_Q = W [S z]^T,  [dS dz] = Phi_Q^T W,
 *   dPhi_K = [V 1] [dS dz]^T,  dv = Phi_K dS,
 * then through the feature map: PRF phi(x) = exp(w.xs - |xs|^2/2)/sqrt(m) gives
 *   dx = d^-1/4 (Omega^T (phi*dphi) - xs (phi.dphi)),
 * ReLU phi(x) = max(w.xs, 0)/sqrt(m) + eps gives dx = d^-1/4 Omega^T (1[w.xs > 0] dphi)/sqrt(m)
 * (a ReLU row whose features are all zero with eps = 0 has a zero denominator: NaN, as in the
 * forward). eps must be >= 0 (else FAVOR_ERR_INVALID_ARG); PRF ignores it.
 * dq, dk [B,H,L,d] and dv_grad [B,H,L,dv] are written in `dtype`, or fp32 when grad_f32 != 0.
 * ws: at least favor_backward_workspace_size(B, H, L, d, dv, m, dtype) bytes. Built shapes
 * (d, dv, m): (16,16,32) (32,32,64) (64,64,128) (64,64,256), both dtypes; others return
 * FAVOR_ERR_UNSUPPORTED. Checks and errors otherwise as favor_bidir. */
favor_status favor_bidir_backward(const void* q, const void* k, const void* v, const float* omega,
                                  const void* dout, int B, int H, int L, int d, int dv, int m,
                                  favor_dtype dtype, favor_kind kind, float eps, int grad_f32, void* dq,
                                  void* dk, void* dv_grad, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace favor_bidir_backward needs; 0 if the arguments are invalid. */
size_t favor_backward_workspace_size(int B, int H, int L, int d, int dv, int m, favor_dtype dtype);

/* favor_causal_backward — gradients of favor_causal's output (Performer appendix B.1,
 * equation 11: prefix sums S_i, z_i over j <= i, diagonal included) with respect to the raw q,
 * k and v, for positive softmax features (FAVOR_PRF) or the ReLU features (FAVOR_RELU, with the
 * forward's eps; trigonometric features return FAVOR_ERR_UNSUPPORTED), given dout [B,H,L,dv] in
 * `dtype`. The forward is recomputed. With W_i = [dout_i, -(dout_i . out_i)] / (Phi_Q z)_i:
 *   dPhi_Q,i = [S_i z_i] W_i,  R_j = sum_{i>=j} Phi_Q,i W_i^T,  dPhi_K,j = R_j [v_j 1],
 *   dv_j = R_j^T Phi_K,j (value columns),  then through the feature map as favor_bidir_backward.
 * dq, dk [B,H,L,d] and dv_grad [B,H,L,dv] are written in `dtype`, or fp32 when grad_f32 != 0.
 * ws: at least favor_causal_backward_workspace_size(B, H, L, d, dv, m, dtype) bytes. Built shapes
 * as favor_bidir_backward; checks and errors as favor_bidir_backward. */
favor_status favor_causal_backward(const void* q, const void* k, const void* v, const float* omega,
                                   const void* dout, int B, int H, int L, int d, int dv, int m,
                                   favor_dtype dtype, favor_kind kind, float eps, int grad_f32, void* dq,
                                   void* dk, void* dv_grad, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace favor_causal_backward needs; 0 if the arguments are invalid. */
size_t favor_causal_backward_workspace_size(int B, int H, int L, int d, int dv, int m, favor_dtype dtype);

/* Bytes of device workspace favor_bidir (causal = 0) or favor_causal (causal = 1)
 * needs for these sizes; 0 if the arguments are invalid. */
size_t favor_workspace_size(int causal, int B, int H, int L, int d, int dv, int m, favor_dtype dtype);

/* Opt-in launch timing for profiling. favor_timing_enable(1) clears the record list
 * and, from then on, brackets every kernel the library launches with two HIP events
 * recorded on that launch's stream; favor_timing_enable(0) clears and stops.
 * favor_timing_read synchronises the recorded events and fills up to `cap`
 * (kernel name, milliseconds) pairs in launch order (names are static strings);
 * it returns the total number of records. Either output pointer may be NULL.
 * The record list is process-wide and guarded by a mutex. */
favor_status favor_timing_enable(int on);
int favor_timing_read(const char** names, float* ms, int cap);

/* Static description of a status code. */
const char* favor_status_string(favor_status status);

#ifdef __cplusplus
}
#endif
#endif /* FAVOR_H */
