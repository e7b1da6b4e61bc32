"""FAVOR+ forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full pass of the selected path over one batch of synthetic,
seeded inputs already resident in device memory:
  bidir_bf16  (default, the headline workload) favor_bidir, B8 H12 L4096 d64 dv64 m256, bf16 in/out
  cross_bf16  favor_bidir_cross, B8 H12 Lq1024 Lk4096 d64 dv64 m256 (tokens = query tokens)
  causal_bf16 favor_causal, B4 H8 L8192 d64 dv64 m256
  decode_bf16 one favor_decode step for 256 sequences x 16 heads, d64 dv64 m256 (fp32 state)
  decode_gated_bf16 the same with favor_decode_gated (gates U[0.9,1), input weight 1 - g)
  backward_bf16 favor_bidir_backward (dq, dk, dv) at bidir_bf16's shape, bf16 gradients
  causal_backward_bf16 favor_causal_backward (dq, dk, dv) at causal_bf16's shape, bf16 gradients
  trig_bf16   favor_bidir with trigonometric features (FAVOR_TRIG) at bidir_bf16's shape
  features_bf16 favor_features alone on bidir_bf16's queries (phi written as fp32: 402 MB per step)
  bidir_fp32 / bidir_small  the fp32 parity workloads
For bidir and causal workloads the timed step reads Omega's fragments prepared once before
timing (favor_omega_prepare, then favor_bidir_prepared / favor_causal_prepared: Omega is a
fixed parameter between redraws); the same steps with Omega converted on every call
(favor_bidir / favor_causal) are timed too and reported as *_omega_per_call
(--omega-per-call makes those the timed step).
The step first runs untimed for --settle-ms (200 ms) so the GPU reaches its working
clock, then W warm-up steps, then K timed steps. Prints one JSON line with
whole-job throughput (tokens/s = B*H*L per second; for decode, head-tokens/s), the
dominant kernel's roofline fraction (per-launch durations from start and stop events
recorded in each kernel's own dispatch during a second pass of the same steps, right
after the timed one), and the fp64 oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "FAVOR+ fwd tokens/sec (B*H*L/s) + % MFMA/HBM roofline, L=4096 m=256 bf16"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3


def _kernel_work(w: workloads.Workload, name: str, out_bytes: int):
    """Algorithmic (flops, bytes) of one launch of kernel `name` for workload w.

    Per token-head: projection 2*m*d flops, contraction with [V 1] or [S z]
    2*m*(dv+1) flops; bytes are the inputs the step must read and the outputs it
    must write (q/k/v at the input width, out at the output width)."""
    eb = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.L          # keys (and queries unless cross attention)
    thq = w.B * w.H * w.Lq_eff    # queries
    proj = 2 * w.m * w.d
    contr = 2 * w.m * (w.dv + 1)
    if name == "reduce":
        return th * (proj + contr), th * (w.d + w.dv) * eb
    if name == "output":
        return thq * (proj + contr), thq * (w.d * eb + w.dv * out_bytes)
    if name == "sweep":       # queries and keys projected, inter+intra contractions, outputs
        return th * (2 * proj + 2 * contr), th * ((2 * w.d + w.dv) * eb + w.dv * out_bytes)
    if name == "bwd_q":       # projection, u = S g, dq = Omega^T (phi' . Delta), dS_aug += phi'^T W
        return thq * (2 * proj + 2 * w.m * w.dv + contr), thq * ((w.d + w.dv) * eb + w.d * out_bytes)
    if name == "bwd_k":       # projection, dPhi_K = dS_aug [v 1], dk = Omega^T P, dv = dS^T phi
        return th * (2 * proj + contr + 2 * w.m * w.dv), th * ((w.d + w.dv) * eb + (w.d + w.dv) * out_bytes)
    if name == "cbwd_fwd":    # the forward recomputed: phi_K, phi_Q, S update, output; l and gamma written
        return th * (2 * proj + 2 * contr), th * ((2 * w.d + 2 * w.dv) * eb + 8)
    if name == "cbwd_q":      # phi_K, phi~_Q, S update, dPhi_Q = [S z] W, dq = Omega^T P
        return th * (3 * proj + 2 * contr), th * ((2 * w.d + 2 * w.dv) * eb + 8 + w.d * out_bytes)
    if name == "cbwd_k":      # phi_K, phi~_Q, R update, dPhi_K = R [v 1], dk = Omega^T P
        return th * (3 * proj + 2 * contr), th * ((2 * w.d + 2 * w.dv) * eb + 8 + w.d * out_bytes)
    if name == "cbwd_v":      # phi_K, phi~_Q, R update (value columns), dv = R^T phi_K
        return th * (2 * proj + 4 * w.m * w.dv), th * ((2 * w.d + 2 * w.dv) * eb + 4 + w.dv * out_bytes)
    if name == "features":    # projection and map of every token-head; x read, phi (fp32, m) and logscale written
        return th * proj, th * (w.d * eb + w.m * 4 + 4)
    if name == "decode":      # per (sequence, head): q,k projections, state read+write, out (+ gate, weight)
        sb = (w.m * w.dv + w.m) * 4
        gb = 8 if w.kind == "decode_gated" else 0
        return th * (2 * proj + 2 * contr), th * (2 * sb + (2 * w.d + w.dv) * eb + w.dv * 4 + gb)
    return None, None


# the device sources each path's kernels are built from
_PATH_SOURCES = {
    "bidir": ["favor_bidir.hip", "favor_tiles.hpp", "favor_reduce.hpp", "favor_device.hpp", "favor_plan.hpp"],
    "cross": ["favor_bidir.hip", "favor_tiles.hpp", "favor_reduce.hpp", "favor_device.hpp", "favor_plan.hpp"],
    "causal": ["favor_causal.hip", "favor_segments.hpp", "favor_tiles.hpp", "favor_reduce.hpp", "favor_device.hpp",
               "favor_plan.hpp"],
    "decode": ["favor_decode.hip", "favor_device.hpp", "favor_plan.hpp"],
    "decode_gated": ["favor_decode.hip", "favor_device.hpp", "favor_plan.hpp"],
    "backward": ["favor_backward.hip", "favor_tiles.hpp", "favor_reduce.hpp", "favor_device.hpp", "favor_plan.hpp"],
    "causal_backward": ["favor_causal_bwd.hip", "favor_segments.hpp", "favor_tiles.hpp", "favor_reduce.hpp",
                        "favor_device.hpp", "favor_plan.hpp"],
    "features": ["favor_bidir.hip", "favor_tiles.hpp", "favor_reduce.hpp", "favor_device.hpp", "favor_plan.hpp"],
}


def _code_only(data: bytes) -> bytes:
    """The source without // comments, trailing blanks and empty lines (comments do not change a kernel)."""
    out = []
    for line in data.split(b"\n"):
        k = line.find(b"//")
        if k >= 0:
            line = line[:k]
        line = line.rstrip()
        if line:
            out.append(line)
    return b"\n".join(out)


def _src_hash(kind: str) -> str:
    """Digest of the code one path's kernels are built and launched from (the .hip files whole, launch
    plans and launchers included, and the headers; comments left out): a counter summary is valid while it
    matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "random_feature_amd", "csrc")
    for f in _PATH_SOURCES[kind]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(_code_only(fh.read()))
    return h.hexdigest()[:16]


def _traffic(kernel: str, workload: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if taken on the current sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("src_hash") != _src_hash(kind):
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(w: workloads.Workload, budget_s: float = 12.0, omega_mode: str = "ortho_chi"):
    """The fp64 oracle on the host, NumPy's BLAS on every core this process may use, on a bounded sample: the
    first pass runs (b,h) pairs (decode: steps of 8 sequences x all heads) until about budget_s / 3 seconds
    have passed, two more passes repeat that sample, and the median pass gives the rate in the metric's unit
    (a single pass when one pair already takes longer than budget_s)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    if w.feature == "trig":  # likewise for the sine and cosine features
        om, kind = oracle.make_omega(w.seed, w.H, w.m // 2, w.d), "trig"
    elif omega_mode == "hyperbolic":  # the oracle takes the m/2 vectors and builds the 2 x m/2 features itself
        om, kind = oracle.make_omega(w.seed, w.H, w.m // 2, w.d), "hyperbolic"
    else:
        om, kind = oracle.make_omega(w.seed, w.H, w.m, w.d, omega_mode), "prf"
    ncpu = len(os.sched_getaffinity(0))
    with threadpool_limits(ncpu):
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
        if w.kind in ("bidir", "cross", "causal", "backward", "causal_backward", "features"):
            q, k, v = workloads.make_qkv(w)
            if w.kind == "features":
                fn = lambda q_, k_, v_, o_, kd, sl: oracle.features(q_, o_, kd)  # noqa: E731
            elif w.kind in ("backward", "causal_backward"):
                dout = workloads.make_dout(w)
                fb = oracle.bidir_backward if w.kind == "backward" else oracle.causal_backward
                fn = lambda q_, k_, v_, o_, kd, sl: fb(q_, k_, v_, o_, dout[sl], kd)  # noqa: E731
            else:
                f0 = oracle.causal if w.kind == "causal" else oracle.bidir
                fn = lambda q_, k_, v_, o_, kd, sl: f0(q_, k_, v_, o_, kd)  # noqa: E731

            def run(pairs):
                for b, h in pairs:
                    sl = (slice(b, b + 1), slice(h, h + 1))
                    fn(q[sl], k[sl], v[sl], om[h:h + 1], kind, sl)
            sample, t0 = [], time.perf_counter()
            for b in range(w.B):
                for h in range(w.H):
                    run([(b, h)])
                    sample.append((b, h))
                    if time.perf_counter() - t0 > budget_s / 3:
                        break
                if time.perf_counter() - t0 > budget_s / 3:
                    break
            times = [time.perf_counter() - t0]
            if times[0] < budget_s:
                for _ in range(2):
                    t1 = time.perf_counter()
                    run(sample)
                    times.append(time.perf_counter() - t1)
            dt = sorted(times)[len(times) // 2]
            return dict(value=len(sample) * w.Lq_eff / dt, unit="tokens/s", cores=threads, kind="oracle",
                        sample=f"{len(sample)} of {w.B * w.H} (b,h) pairs x {w.Lq_eff} tokens, fp64 NumPy with "
                               f"{threads} BLAS threads, median of {len(times)} passes of {dt:.1f} s")
        # decode: steps of the fp64 recurrence for all heads of a few sequences
        n_seq = 8

        def steps_run(nsteps=None, limit=None):
            gen = torch.Generator().manual_seed(w.seed)
            S = np.zeros((n_seq, w.H, w.m, w.dv))
            z = np.ones((n_seq, w.H, w.m))
            done, t0 = 0, time.perf_counter()
            while (done < nsteps) if nsteps is not None else (time.perf_counter() - t0 < limit):
                qq = torch.randn(n_seq, w.H, w.d, generator=gen).bfloat16()
                kk = torch.randn(n_seq, w.H, w.d, generator=gen).bfloat16()
                vv = torch.randn(n_seq, w.H, w.dv, generator=gen).bfloat16()
                if w.kind == "decode_gated":
                    gg = 0.9 + 0.1 * torch.rand(n_seq, w.H, generator=gen).double().numpy()
                    S, z, _ = oracle.decode_gated_step(S, z, qq, kk, vv, om, gg, 1.0 - gg, kind)
                else:
                    S, z, _ = oracle.decode_step(S, z, qq, kk, vv, om, kind)
                done += 1
            return done, time.perf_counter() - t0
        nsteps, t_first = steps_run(limit=budget_s / 3)
        times = [t_first] + [steps_run(nsteps=nsteps)[1] for _ in range(2)]
        dt = sorted(times)[1]
        return dict(value=nsteps * n_seq * w.H / dt, unit="head-tokens/s", cores=threads, kind="oracle",
                    sample=f"{nsteps} decode steps x {n_seq} sequences x {w.H} heads, fp64 NumPy with {threads} "
                           f"BLAS threads, median of 3 passes of {dt:.1f} s")


def measure(a, wname: str, omega_mode: str = "ortho_chi") -> dict:
    """Time one workload (see the module docstring) and return its result fields."""
    import random_feature_amd as rf
    w = workloads.WORKLOADS[wname]
    steps = a.steps if a.steps is not None else (w.steps if w.kind in ("decode", "decode_gated") else 50)
    dev = "cuda:0"
    dt = w.torch_dtype
    fkind = w.feature
    om = rf.make_omega(w.seed, w.H, w.m, w.d, "trig_pairs" if fkind == "trig" else omega_mode, device=dev)

    prepared = False  # the timed step reads prepared Omega fragments (bidir and causal)
    if w.kind in ("decode", "decode_gated"):
        S = torch.empty((w.B, w.H, w.m, w.dv), dtype=torch.float32, device=dev)
        z = torch.empty((w.B, w.H, w.m), dtype=torch.float32, device=dev)
        # initial state: the canonical final state of a causal pass over `prior` tokens per sequence
        gen = torch.Generator(dev).manual_seed(w.seed + 1)
        for s0 in range(0, w.B, 64):
            n = min(64, w.B - s0)
            kp = (torch.randn(n, w.H, w.prior, w.d, generator=gen, device=dev) * w.k_scale).to(dt)
            vp = (torch.randn(n, w.H, w.prior, w.dv, generator=gen, device=dev) * w.v_scale).to(dt)
            _, S_, z_ = rf.causal(kp, kp, vp, om, return_state=True)
            S[s0:s0 + n] = S_
            z[s0:s0 + n] = z_
            del kp, vp
        n_steps = a.warmup + steps
        qs, ks, vs = workloads.make_decode_steps(w, dev, steps=n_steps)
        out = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)
        it = iter(range(10 ** 9))
        if w.kind == "decode_gated":
            gs = workloads.make_gates((n_steps, w.B, w.H), w.seed, device=dev)
            wts = 1.0 - gs

        def step():
            t = next(it) % n_steps
            if w.kind == "decode_gated":
                rf.decode_gated(qs[t], ks[t], vs[t], om, S, z, gs[t], wts[t], out=out)
            else:
                rf.decode(qs[t], ks[t], vs[t], om, S, z, out=out)
        tokens_per_step = w.B * w.H
        unit = "head-tokens/s"
        out_bytes = 4
        sets = None
    else:
        sets = []
        nset = 1 + (max(0, a.rotate - 1) if a.rotate else 0)
        for r in range(nset):
            q, k, v = workloads.make_qkv(w.with_(seed=w.seed + 1000 * r) if r else w, device=dev)
            sets.append((q, k, v))
        q, k, v = sets[0]
        cur = [0]
        if w.kind in ("backward", "causal_backward"):
            douts = [workloads.make_dout(w.with_(seed=w.seed + 1000 * r) if r else w, device=dev)
                     for r in range(nset)]
            wsfn, bfn = ((rf.backward_workspace, rf.bidir_backward) if w.kind == "backward"
                         else (rf.causal_backward_workspace, rf.causal_backward))
            ws = wsfn(q, v, om)
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))

            def step():
                qq, kk, vv = sets[cur[0]]
                bfn(qq, kk, vv, om, douts[cur[0]], ws=ws, out=grads)
        elif w.kind == "features":
            def step():
                rf.features(sets[cur[0]][0], om, kind=fkind)
        else:
            ws = rf.workspace(w.kind == "causal", k, v, om)
            out = torch.empty((w.B, w.H, w.Lq_eff, w.dv), dtype=dt, device=dev)
            fn = {"bidir": rf.bidir, "cross": rf.bidir_cross, "causal": rf.causal}[w.kind]
            # Omega's fragments prepared once (favor_omega_prepare; the timed calls read them), unless
            # --omega-per-call; the per-call figure is timed as well below
            if w.kind in ("bidir", "causal"):
                prep = rf.prepare_omega(om, w.dv, dt, fkind)
                torch.cuda.synchronize()
                prepared = not a.omega_per_call

            def step():
                qq, kk, vv = sets[cur[0]]
                if prepared:
                    fn(qq, kk, vv, om, kind=fkind, ws=ws, out=out, prep=prep)
                else:
                    fn(qq, kk, vv, om, kind=fkind, ws=ws, out=out)
        tokens_per_step = w.B * w.H * w.Lq_eff   # output (query) tokens
        unit = "tokens/s"
        out_bytes = 2 if dt == torch.bfloat16 else 4

    def rotate(i):
        if sets is not None:
            cur[0] = i % len(sets)

    if a.copy_calib:
        # a plain elementwise copy of known size: hardware counters of the same run are
        # calibrated against it (see random_feature_amd.profiling)
        # (a bitwise not over int32: no other kernel of any workload's setup has that name)
        n = a.copy_calib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # settle: the GPU raises its clocks over the first tens of milliseconds of load (a 5-step warm-up leaves
    # the timed steps 10-15 % slow), so the step runs untimed for settle_ms of wall-clock time first
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < a.settle_ms:
        for i in range(8):
            rotate(i)
            step()
        settle_steps += 8
        torch.cuda.synchronize()
    for i in range(a.warmup):
        rotate(i)
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the timed steps run uninstrumented, each on the next of the rotating input sets (together larger than
    # the 256 MB last-level cache, so every step reads its inputs from HBM); later passes are instrumented
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        rotate(i)
        step()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # the same rotating steps with Omega converted on every call (favor_bidir / favor_causal)
    per_call_ms = None
    if prepared:
        prepared = False
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            rotate(i)
            step()
        e1.record()
        torch.cuda.synchronize()
        per_call_ms = e0.elapsed_time(e1)
        prepared = True
    # the same steps on one input set only (it stays resident in the last-level cache): the warm figure
    warm_ms = None
    if sets is not None and len(sets) > 1:
        rotate(0)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        warm_ms = e0.elapsed_time(e1)
    # per-step distribution (a separate pass, an event pair around every step)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (p0, p1) in enumerate(pairs):
        rotate(i)
        p0.record()
        step()
        p1.record()
    torch.cuda.synchronize()
    per_step = sorted(p0.elapsed_time(p1) for p0, p1 in pairs)

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]
    rf.timing_enable(True)
    for i in range(steps):
        rotate(i)
        step()
    torch.cuda.synchronize()
    recs = rf.timing_read()
    rf.timing_enable(False)

    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    avg = {n: sum(v) / len(v) for n, v in per.items()}
    dominant = max(avg, key=lambda n: avg[n] * len(per[n]))
    flops, nbytes = _kernel_work(w, dominant, out_bytes)
    roofline = None
    if flops is not None:
        t_s = avg[dominant] * 1e-3
        gbs = nbytes / t_s / 1e9
        peak_f = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        tfl = flops / t_s / 1e12
        hbm_time, mfma_time = nbytes / (PEAK_HBM_GBS * 1e9), flops / (peak_f * 1e12)
        if hbm_time >= mfma_time:
            roofline = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                            frac=round(gbs / PEAK_HBM_GBS, 4), traffic=_traffic(dominant, w.name, w.kind))
        else:
            roofline = dict(bound="mfma", achieved=round(tfl, 2), peak=peak_f, unit="TFLOP/s",
                            frac=round(tfl / peak_f, 4), traffic=_traffic(dominant, w.name, w.kind))
        roofline.update(kernel=dominant, avg_launch_us=round(avg[dominant] * 1e3, 2),
                        mfma_tflops=round(tfl, 2), mfma_frac=round(tfl / peak_f, 4),
                        hbm_gbs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                        algorithmic_flops=flops, algorithmic_bytes=nbytes)
    # the whole step against the peaks: the workload's algorithmic flops and bytes (every token-head's work
    # once, as _kernel_work counts them) over the measured time per step
    step_flops = step_bytes = 0
    for name in {"bidir": ("reduce", "output"), "cross": ("reduce", "output"), "causal": ("sweep",),
                 "decode": ("decode",), "decode_gated": ("decode",), "features": ("features",)}.get(w.kind, ()):
        f_, b_ = _kernel_work(w, name, out_bytes)
        step_flops += f_
        step_bytes += b_
    whole = None
    if step_flops:
        t_step = total_ms * 1e-3 / steps
        peak_f = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        whole = dict(algorithmic_flops=step_flops, algorithmic_bytes=step_bytes,
                     mfma_frac=round(step_flops / t_step / 1e12 / peak_f, 4),
                     hbm_frac=round(step_bytes / t_step / 1e9 / PEAK_HBM_GBS, 4))

    res = {
        "metric": METRIC if w.name == "bidir_bf16" else f"FAVOR+ {w.kind} {unit}, workload {w.name}",
        "value": tokens_per_step * steps / (total_ms * 1e-3), "unit": unit, "n_gpus": 1, "steps": steps,
        "warmup": a.warmup, "settle": {"ms": a.settle_ms, "steps": settle_steps},
        "ms_per_step": total_ms / steps,
        "ms_per_step_p10_p50_p90": [round(pct(0.1), 5), round(pct(0.5), 5), round(pct(0.9), 5)],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "kind": w.kind, "B": w.B, "H": w.H, "L": w.L, "Lq": w.Lq_eff, "d": w.d,
                   "dv": w.dv, "m": w.m, "feature_map": fkind if omega_mode != "hyperbolic" else "prf_hyperbolic",
                   "omega": "trig_pairs" if fkind == "trig" else omega_mode,
                   "out_dtype": "fp32" if w.kind.startswith("decode") else w.dtype,
                   "omega_fragments": ("prepared once (favor_omega_prepare), read by every timed call" if prepared
                                       else "converted on every call")},
        "kernels_us": {n: round(v * 1e3, 2) for n, v in avg.items()},
        "roofline": roofline,
        "whole_step": whole,
    }
    if per_call_ms is not None:
        res["value_omega_per_call"] = tokens_per_step * steps / (per_call_ms * 1e-3)
        res["ms_per_step_omega_per_call"] = per_call_ms / steps
    if sets is not None:
        res["inputs"] = (f"{len(sets)} input sets in rotation, one per step"
                         if len(sets) > 1 else "one input set, reused every step")
        if warm_ms is not None:
            res["value_warm_inputs"] = tokens_per_step * steps / (warm_ms * 1e-3)
            res["ms_per_step_warm_inputs"] = warm_ms / steps
    else:
        res["inputs"] = f"{w.steps} decode steps' inputs pre-generated in device memory, the state updated in place"
    del sets
    torch.cuda.empty_cache()
    return res


# the workloads whose figures the default (headline) line also carries
COMPANIONS = ("causal_bf16", "decode_bf16")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; decode workloads: the workload's 1000 steps)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="bidir_bf16", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--omega-per-call", action="store_true",
                    help="bidir/causal: time the calls that convert Omega on every call (favor_bidir, favor_causal) "
                         "instead of the prepared-Omega calls")
    ap.add_argument("--no-companions", action="store_true",
                    help="headline workload only (without the causal and decode figures)")
    ap.add_argument("--omega-mode", default="ortho_chi", choices=["ortho_chi", "iid", "ortho_sqrtd", "hyperbolic"],
                    help="random features: hyperbolic gives Lemma 1's hyperbolic features (m/2 vectors)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps for this long before the warm-up, so the GPU reaches its working clock")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="launch one elementwise copy of this many MiB first (counter calibration)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="input sets in rotation, one per timed step (together larger than the 256 MB "
                         "last-level cache); 1 reuses one set")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {a.gpus} is not supported "
              f"(the path shards over (b,h) pairs with no communication between GPUs)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    res = measure(a, a.workload, a.omega_mode)
    if a.workload == "bidir_bf16" and not a.no_companions:
        for cname in COMPANIONS:
            a2 = argparse.Namespace(**vars(a))
            a2.steps = None  # each companion at its own default step count
            a2.copy_calib = 0
            c = measure(a2, cname)
            res[cname] = {k: c[k] for k in ("metric", "value", "unit", "steps", "ms_per_step",
                                            "ms_per_step_p10_p50_p90", "config", "kernels_us", "roofline",
                                            "whole_step", "inputs", "value_omega_per_call",
                                            "ms_per_step_omega_per_call") if k in c}
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(workloads.WORKLOADS[a.workload], omega_mode=a.omega_mode)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
