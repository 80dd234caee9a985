"""GCA throughput on one MI355X: frames/s per layer at 1004 tokens per frame.

One step = one pass of the whole GCA path over a synthetic frame stream of the
518x378 shape (1004 tokens, 16 heads x 64): reset, then for every frame
append (3D RoPE on K, paged scatter) -> evict/compact -> attend (pool
selection, paged MFMA attention with RoPE on Q, split merge); non-keyframes do
append -> attend -> rollback.  Inputs are resident in HBM before the timed
region.  Each frame is one gca_step call: one launch for the append, eviction,
query rotation and gather list, then the attention and the split merge.  The
attention kernel's duration comes from HIP events that the library records
around each of its launches on the stream it launches on; the roofline
uses the algorithmic FLOPs 4*T*H*D*n_ctx per frame.  Events at the start of
the last 10 % of each stream's frames give the steady-state rate.  After the
timed region the append and compaction launches (the individual calls) are timed in
back-to-back batches for their HBM roofline (`append_compact`).  MFMA busy and
HBM traffic come from the committed rocprofv3 counter summary of the same
kernel source; the other kernels' durations from a rocprofv3 kernel trace.

The headline line is the 64-frame stream at page size 16; `configs` holds the
same measurements for the three long streams (1,000 frames with a 64-frame
window, 10,000 drifting frames with keyframe interval 4, the 20,000-frame
12-frame ring), each with its own CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-configs] [--no-cpu-baseline] [--stream-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GCA frames/sec/layer at 1004 tok/frame + % bf16 MFMA peak (1 MI355X)"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="bf16_T1004_H16_P16_W16_64f")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=64)
    ap.add_argument("--stream-only", action="store_true",
                    help="skip the scale-phase, camera-head and long-stream measurements (counter runs "
                         "that average per stream launch)")
    ap.add_argument("--no-configs", action="store_true", help="skip the long-stream lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (counter calibration)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: read 256 MiB, write 256 MiB, five times."""
    import torch
    n = 256 << 20
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def kernel_hash() -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "paged_kv_cache_gca_amd", "csrc", "gca_kernels.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def counters_from_profiles(kh: str, workload: str) -> dict:
    """The committed counter summary of the attention kernel on `workload`, if
    it was taken from this kernel source."""
    p = os.path.join(ROOT, "profiles", "attn_traffic.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return {}
    if d.get("kernel_hash") != kh:
        return {}
    return d.get("workloads", {}).get(workload, {})


def stage_frames(w, fs, dt, n_stage):
    """Device copies of the stream's inputs, made before any timing: the
    n_stage distinct query frames, and the key/value frames -- the same
    n_stage for a cycled stream, every frame for a drifting one (the per-frame
    offsets of the random walk added in float32 to the float32 base draws on
    the device and rounded once, as the generator does on the host)."""
    import numpy as np
    import torch
    from paged_kv_cache_gca_amd.synth import TENSOR_K, TENSOR_V
    print(f"[bench] staging {n_stage} distinct frames of {w.name}", file=sys.stderr, flush=True)
    Q, K, V = [], [], []
    for f in range(n_stage):
        Q.append(torch.from_numpy(fs.q(f)).to(dt).cuda())
        if not w.drift_sigma:
            k, v = fs.kv(f)
            K.append(torch.from_numpy(k).to(dt).cuda())
            V.append(torch.from_numpy(v).to(dt).cuda())
    if w.drift_sigma:
        bk = [torch.from_numpy(fs.base(f, TENSOR_K)).cuda() for f in range(n_stage)]
        bv = [torch.from_numpy(fs.base(f, TENSOR_V)).cuda() for f in range(n_stage)]
        mu = np.stack([np.stack(fs.drift(f)) for f in range(w.n_frames)]).astype(np.float32)
        mu = torch.from_numpy(mu).cuda()                       # [n_frames][2][H][D]
        print(f"[bench] {w.n_frames} drifting key/value frames on the device", file=sys.stderr, flush=True)
        for f in range(w.n_frames):
            i = f % n_stage
            K.append((bk[i] + mu[f, 0][None]).to(dt))
            V.append((bv[i] + mu[f, 1][None]).to(dt))
        # the device rounding is the generator's: a few frames compared bit for bit
        for f in (0, 1, w.n_frames // 2, w.n_frames - 1):
            k, v = fs.kv(f)
            assert torch.equal(K[f].cpu(), torch.from_numpy(k).to(dt)), f
            assert torch.equal(V[f].cpu(), torch.from_numpy(v).to(dt)), f
        del bk, bv, mu
    torch.cuda.synchronize()
    return Q, K, V


def plan_n_ctx(w):
    """Context length of every frame of the stream (data independent), from the host planner."""
    from paged_kv_cache_gca_amd import gca
    plan = gca.Plan(gca.Config.from_workload(w))
    n_ctx = []
    for f in range(w.n_frames):
        key = w.is_keyframe(f)
        plan.append(f, temp=not key)
        if key:
            plan.evict()
        n_ctx.append(plan.query().n_ctx)
        if not key:
            plan.rollback(f)
    return n_ctx


def run_gpu(w, steps, warmup):
    import numpy as np
    import torch

    from paged_kv_cache_gca_amd import gca
    from paged_kv_cache_gca_amd.synth import FrameStream

    torch.cuda.set_device(0)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    fs = FrameStream(w.seed, w.T, w.H, w.D, w.dtype, n_base=w.n_base, drift_sigma=w.drift_sigma)
    n_stage = w.n_frames if w.n_base is None else min(w.n_frames, w.n_base)
    Q, K, V = stage_frames(w, fs, dt, n_stage)
    cache = gca.Cache(gca.Config.from_workload(w))
    out = torch.empty((w.T, w.H, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # the last 10 % of each stream (the longest contexts): events on the stream
    f_tail = w.n_frames - max(1, w.n_frames // 10)
    tail_ev = []

    def one_stream(mark_tail=False):
        if cache.reset(stream) != 0:
            raise RuntimeError("reset failed")
        for f in range(w.n_frames):
            if mark_tail and f == f_tail:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                tail_ev.append(e)
            i = f % n_stage
            # append (+ evict) + attend (+ rollback): one update launch, then attention
            rc = cache.step(f, K[f % len(K)], V[f % len(V)], Q[i], out, lse, keyframe=w.is_keyframe(f),
                            stream=stream)
            if rc != 0:
                raise RuntimeError(f"frame {f}: {gca.status_string(rc)}")
        if mark_tail:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            tail_ev.append(e)

    n_ctx = plan_n_ctx(w)
    flop_stream = float(sum(4.0 * w.T * w.H * w.D * n for n in n_ctx))

    print(f"[bench] warmup {warmup} streams", file=sys.stderr, flush=True)
    for _ in range(warmup):
        one_stream()
    torch.cuda.synchronize()
    # HIP events only around the attention kernel (the roofline kernel); the
    # other kernels' durations come from the rocprofv3 trace of this command
    cache.profile_enable(steps * w.n_frames + 16, kinds=("attn",))
    print(f"[bench] timing {steps} streams x {w.n_frames} frames", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_stream(mark_tail=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = {"attn": cache.profile_read("attn")}
    cache.profile_enable(0)
    assert torch.isfinite(out).all()
    tail_ms = sum(tail_ev[2 * i].elapsed_time(tail_ev[2 * i + 1]) for i in range(steps))
    tail_fps = steps * (w.n_frames - f_tail) / (tail_ms * 1e-3)


    # Append and compaction as their own launches (the individual calls), timed
    # in back-to-back batches with HIP events on the launch stream around each
    # batch: per-launch time = kernel plus the dispatch gap to the next one.  A
    # spin kernel ahead of the batch holds the stream until every launch is
    # queued, so host-side call overhead is not timed.
    def batch(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def appends():  # TEMP appends of frames 0..n-1 on an empty cache, each rolled back (host only)
        for f in range(w.n_frames):
            if cache.append_frame(f, K[f % len(K)], V[f % len(V)], temp=True, stream=stream) != 0 or \
                    cache.rollback_last_frame(f, stream) != 0:
                raise RuntimeError("append batch failed")

    for timed in (False, True):
        if cache.reset(stream) != 0:
            raise RuntimeError("reset failed")
        torch.cuda.synchronize()
        if timed:
            append_ms = batch(appends) / w.n_frames
        else:
            appends()
    fill = w.A + w.W  # keyframes that fit before the first eviction
    kf = [f for f in range(w.n_frames) if w.is_keyframe(f)]
    n_evict = 0
    if w.C > 0 and len(kf) > fill:
        if cache.reset(stream) != 0:
            raise RuntimeError("reset failed")
        for f in kf[:fill]:
            if cache.append_frame(f, K[f % len(K)], V[f % len(V)], stream=stream) != 0:
                raise RuntimeError("fill failed")

        def pairs():
            for f in kf[fill:]:
                if cache.append_frame(f, K[f % len(K)], V[f % len(V)], stream=stream) != 0 or \
                        cache.evict_compact(stream) != 0:
                    raise RuntimeError("eviction batch failed")
        torch.cuda.synchronize()
        n_evict = len(kf) - fill
        pair_ms = batch(pairs) / n_evict
    kern["append"] = (append_ms, 1)
    kern["evict"] = (pair_ms - append_ms, 1) if n_evict else (0.0, 0)
    cache.close()
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count, "hip": torch.version.hip}
    return dict(seconds=t1 - t0, kern=kern, flop_stream=flop_stream, n_ctx=n_ctx, tail_fps=tail_fps,
                tail_frames=(f_tail, w.n_frames), device=device)


def run_scale_phase(w, nf=8, reps=10, warmup=2):
    """The stream's first phase: nf scale frames appended as the anchor in one
    launch, then all of their queries in one joint (bidirectional) attention
    call.  HIP events from the library around the append and the attention
    launches; events on the stream around each whole phase."""
    import torch

    from paged_kv_cache_gca_amd import gca
    from paged_kv_cache_gca_amd.synth import FrameStream

    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    fs = FrameStream(w.seed, w.T, w.H, w.D, w.dtype, n_base=w.n_base)
    kv = [fs.kv(f) for f in range(nf)]
    K = torch.stack([torch.from_numpy(x[0]).to(dt) for x in kv]).cuda()
    V = torch.stack([torch.from_numpy(x[1]).to(dt) for x in kv]).cuda()
    Q = torch.stack([torch.from_numpy(fs.q(f)).to(dt) for f in range(nf)]).cuda()
    cache = gca.Cache(gca.Config.from_workload(w, num_anchor_frames=nf))
    out = torch.empty((nf, w.T, w.H, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((nf, w.T, w.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def phase():
        if cache.reset(stream) != 0:
            raise RuntimeError("reset failed")
        if cache.append_frames(0, K, V, stream=stream) != 0:
            raise RuntimeError("scale-frame append failed")
        if cache.attend_frames(0, Q, out, lse, stream=stream) != 0:
            raise RuntimeError("joint attention failed")

    for _ in range(warmup):
        phase()
    torch.cuda.synchronize()
    n_ctx = cache.query().n_ctx
    cache.profile_enable(reps + 4, kinds=("attn", "append"))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        phase()
        e1.record(stream)
    torch.cuda.synchronize()
    attn_ms, n = cache.profile_read("attn")
    app_ms, na = cache.profile_read("append")
    cache.profile_enable(0)
    cache.close()
    assert torch.isfinite(out).all()
    phase_ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps
    flop = 4.0 * nf * w.T * n_ctx * w.H * w.D
    us = attn_ms * 1e3 / max(n, 1)
    tflops = flop / (us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    esize = 2 if w.dtype == "bf16" else 4
    ppf = -(-w.T // w.P)
    # per frame: read K and V, write both into its pages (zero tail included)
    app_b = nf * (2 * w.T + 2 * ppf * w.P) * w.H * w.D * esize
    app_us = app_ms * 1e3 / max(na, 1)
    app_gbs = app_b / (app_us * 1e-6) / 1e9
    return {"frames": nf, "queries": nf * w.T, "n_ctx": n_ctx, "attn_us": round(us, 2),
            "attn_flop": flop, "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "append": {"us": round(app_us, 2), "bytes": app_b, "achieved": round(app_gbs, 1),
                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(app_gbs / PEAK_HBM_GBS, 4)},
            "phase_us": round(phase_ms * 1e3, 1),
            "timing": f"{reps} phases after {warmup} warm-up: library HIP events around the batched "
                      "append launch and the joint attention launch; stream events around each phase"}


def scale_phase_cpu(w, nf=8, n_rows=8):
    """The oracle on the scale phase (test infrastructure): nf appends, then the
    joint attention for n_rows of the T query rows of every frame (and 1 row,
    to separate the fixed cost), full-row time scaled linearly in rows."""
    import numpy as np

    import oracle
    from paged_kv_cache_gca_amd.synth import FrameStream

    threads = _cpu_threads()
    fs = FrameStream(w.seed, w.T, w.H, w.D, w.dtype, n_base=w.n_base)
    cfg = oracle.OracleConfig(T=w.T, H=w.H, D=w.D, P=w.P, dtype=w.dtype, A=nf, W=w.W, C=w.C,
                              rope=w.rope, num_special=w.num_special, grid_h=w.grid_h,
                              grid_w=w.grid_w, rope_theta=w.rope_theta, max_frames=w.n_frames)
    c = oracle.OracleCache(cfg)
    rows = np.linspace(0, w.T - 1, n_rows).astype(np.int32)
    a = time.perf_counter()
    for f in range(nf):
        k, v = fs.kv(f)
        c.append(f, k, v)
        c.evict()
    b = time.perf_counter()
    q = np.stack([fs.q(f) for f in range(nf)])
    c.attend_frames(0, q, rows=rows[:1], threads=threads)
    m = time.perf_counter()
    c.attend_frames(0, q, rows=rows, threads=threads)
    e = time.perf_counter()
    one = m - b
    per_row = max(0.0, (e - m) - one) / max(1, n_rows - 1)
    est = (b - a) + one + per_row * w.T
    return {"us": round(est * 1e6, 1), "cores": threads, "kind": "oracle",
            "sample": f"{nf} appends plus the joint attention for {n_rows} of {w.T} query rows per frame "
                      f"(and 1 row), full-row time scaled linearly in rows"}


def camera_line(wc, steps=3, warmup=1):
    """The causal camera head's cache: one token per frame, one query row per
    head; every step is launch-latency bound, so the figure is per frame."""
    r = run_gpu(wc, steps, warmup)
    attn_ms, n = r["kern"]["attn"]
    us = attn_ms * 1e3 / max(n, 1)
    esize = 2 if wc.dtype == "bf16" else 4
    mean_ctx = sum(r["n_ctx"]) / len(r["n_ctx"])
    kv = 2 * mean_ctx * wc.H * wc.D * esize  # K and V of the mean context, read once
    return {"workload": wc.name, "value": round(steps * wc.n_frames / r["seconds"], 1),
            "unit": "frames/s", "us_per_frame": round(r["seconds"] * 1e6 / (steps * wc.n_frames), 2),
            "attn_us": round(us, 2), "mean_n_ctx": round(mean_ctx, 1), "attn_bytes": round(kv),
            "attn_gbs": round(kv / (us * 1e-6) / 1e9, 1), "bound": "latency",
            "timing": f"{steps} streams of {wc.n_frames} frames after {warmup} warm-up (gca_step per frame); "
                      "library HIP events around each attention launch"}


def append_compact_line(w, kern):
    """HBM roofline of the append and compaction launches (algorithmic bytes per launch)."""
    esize = 2 if w.dtype == "bf16" else 4
    ppf = -(-w.T // w.P)
    row = w.H * w.D * esize
    # append: read the frame's K and V, write both into its pages (zero tail included)
    append_b = 2 * w.T * row + 2 * ppf * w.P * row
    # compaction: read C tokens' K and V from the evicted frame's pages, write them to trajectory pages
    evict_b = 4 * w.C * row
    out = {}
    for name, b in (("append", append_b), ("compact", evict_b)):
        ms, n = kern["append" if name == "append" else "evict"]
        if n == 0 or ms <= 0:
            continue
        us = ms * 1e3 / n
        gbs = b / (us * 1e-6) / 1e9
        out[name] = {"us_per_launch": round(us, 3), "bytes": b, "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    out["timing"] = ("back-to-back batches (one TEMP append per frame; append+evict pairs minus appends), "
                     "HIP events on the launch stream around each batch")
    return out


def _cpu_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_cpu_baseline(w, n_ctx):
    """The CPU oracle (test infrastructure, untuned) on a bounded sample of the
    same stream, on the host cores: bookkeeping (append, evict, rollback with
    the frame's data) for every frame up to the second sampled frame, timed per
    frame; attention for all T query rows and all heads at two sampled frames
    with different context lengths.  The oracle's attention cost per frame is
    linear in n_ctx (two passes over the context per row and head), so the two
    frames give a + b n_ctx, which is applied to every frame of the stream
    (n_ctx from the planner) together with the mean bookkeeping time."""
    import numpy as np

    import oracle
    from paged_kv_cache_gca_amd.synth import FrameStream

    threads = _cpu_threads()
    fs = FrameStream(w.seed, w.T, w.H, w.D, w.dtype, n_base=w.n_base, drift_sigma=w.drift_sigma)
    cfg = oracle.OracleConfig(T=w.T, H=w.H, D=w.D, P=w.P, dtype=w.dtype, A=w.A, W=w.W, C=w.C,
                              rope=w.rope, num_special=w.num_special, grid_h=w.grid_h,
                              grid_w=w.grid_w, rope_theta=w.rope_theta, max_frames=w.n_frames,
                              window=w.infer_window, overlap=w.infer_overlap)
    c = oracle.OracleCache(cfg)
    # sampled frames: one early, one once the window has filled (at most the stream's end)
    fb = min(w.n_frames - 1, (w.A + w.W + 1) * w.keyframe_interval)
    fa = min(fb // 4, w.n_frames - 1)
    t_book = 0.0
    timed = {}
    for f in range(fb + 1):
        key = w.is_keyframe(f)
        k, v = fs.kv(f)
        a = time.perf_counter()
        c.append(f, k, v, temp=not key)
        if key:
            c.evict()
        t_book += time.perf_counter() - a
        if f in (fa, fb):
            q = fs.q(f)
            # repeated until at least 50 ms have passed, so that small frames time reliably
            reps, a = 0, time.perf_counter()
            while True:
                c.attend(f, q, threads=threads)
                reps += 1
                el = time.perf_counter() - a
                if el >= 0.05:
                    break
            timed[f] = (el / reps, c.n_ctx())
        if not key:
            a = time.perf_counter()
            c.rollback(f)
            t_book += time.perf_counter() - a
    book = t_book / (fb + 1)
    (ta, na), (tb, nb) = timed[fa], timed[fb]
    # a + b*n_ctx through the two frames, neither part negative
    slope = max(0.0, (tb - ta) / (nb - na)) if nb != na else tb / nb
    icpt = max(0.0, tb - slope * nb)
    est = w.n_frames * book + sum(icpt + slope * n for n in n_ctx)
    return dict(value=w.n_frames / est, unit="frames/s/layer", cores=threads, kind="oracle",
                cpu_model=_cpu_model(),
                full_row_frames={str(fa): {"n_ctx": na, "s": round(ta, 6)},
                                 str(fb): {"n_ctx": nb, "s": round(tb, 6)}},
                bookkeeping_s_per_frame=round(book, 5),
                sample=(f"{w.name}: bookkeeping (append/evict/rollback with data) of frames 0..{fb}, "
                        f"attention for all {w.T} query rows x {w.H} heads at frames {fa} and {fb} "
                        f"(n_ctx {na} and {nb}); whole stream modelled as {w.n_frames} x the mean "
                        f"bookkeeping time plus a + b*n_ctx per frame from those two frames: "
                        f"{est:.1f} s for the {w.n_frames} frames"))


def stream_line(w, steps, warmup, cpu: bool):
    """frames/s/layer, attention roofline, steady state and append/compaction
    HBM fractions of one stream workload, plus its CPU baseline."""
    r = run_gpu(w, steps, warmup)
    attn_ms, attn_n = r["kern"]["attn"]
    flop_per_launch = r["flop_stream"] / w.n_frames
    avg_attn_s = attn_ms / 1e3 / max(attn_n, 1)
    achieved = flop_per_launch / avg_attn_s / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    # the attention together with its split merge: the merge's kernel duration from the committed
    # kernel trace of this kernel source (HIP events around a 7 us launch add several us), else null
    merge_us = counters_from_profiles(kernel_hash(), w.name).get("merge_us_per_frame")
    with_merge = None
    if merge_us is not None:
        t = avg_attn_s + merge_us * 1e-6
        with_merge = {"merge_us_per_frame": merge_us, "merge_source": "rocprofv3 kernel trace",
                      "achieved": round(flop_per_launch / t / 1e12, 2),
                      "frac": round(flop_per_launch / t / 1e12 / peak, 4), "unit": "TFLOP/s"}
    line = {
        "workload": w.name,
        "value": round(steps * w.n_frames / r["seconds"], 2),
        "unit": "frames/s/layer",
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["seconds"] * 1e3 / steps, 4),
        "config": {"tokens_per_frame": w.T, "heads": w.H, "head_dim": w.D, "page_size": w.P,
                   "frames_per_step": w.n_frames, "anchor": w.A, "window": w.W, "compact": w.C,
                   "keyframe_interval": w.keyframe_interval, "drift_sigma": w.drift_sigma,
                   **({"infer_window": w.infer_window, "infer_overlap": w.infer_overlap}
                      if w.infer_window else {})},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": counters_from_profiles(kernel_hash(), w.name).get("bytes_per_launch")},
        "with_merge": with_merge,
        "steady_state": {"frames": list(r["tail_frames"]), "value": round(r["tail_fps"], 2),
                         "unit": "frames/s/layer"},
        "append_compact": append_compact_line(w, r["kern"]),
        "attn_ms_avg": round(attn_ms / max(attn_n, 1), 5),
        "mean_n_ctx": round(sum(r["n_ctx"]) / len(r["n_ctx"]), 1),
        "attn_flop_per_launch": flop_per_launch,
    }
    if cpu:
        print(f"[bench] cpu baseline (oracle) {w.name}", file=sys.stderr, flush=True)
        line["cpu_baseline"] = run_cpu_baseline(w, r["n_ctx"])
    return line, r


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the GCA path runs on one GPU: --gpus must be 1"}))
        sys.exit(2)
    from paged_kv_cache_gca_amd import workloads as WL
    w = {x.name: x for x in WL.ALL}[args.workload]
    cpu = not args.no_cpu_baseline
    head, r = stream_line(w, args.steps, args.warmup, cpu=False)
    kh = kernel_hash()
    ctr = counters_from_profiles(kh, w.name)

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "frames/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, **{k: v for k, v in head["config"].items() if k != "drift_sigma"},
                   "rope": "3d" if w.rope else "none", "parallelism": "none (1 GPU)"},
        "roofline": head["roofline"],
        "attn_with_merge": head["with_merge"],
        "steady_state": head["steady_state"],
        "mfma_busy": ctr.get("mfma_busy"),
        "append_compact": head["append_compact"],
        "attn_ms_avg": head["attn_ms_avg"],
        "mean_n_ctx": head["mean_n_ctx"],
        "attn_flop_per_launch": head["attn_flop_per_launch"],
        "kernel_hash": kh,
        "device": r["device"],
    }
    if w.rope and w.dtype == "bf16" and not args.stream_only:
        print("[bench] scale phase", file=sys.stderr, flush=True)
        line["scale_phase"] = run_scale_phase(w)
        print("[bench] camera-head cache", file=sys.stderr, flush=True)
        line["camera_head"] = camera_line(WL.CAMERA_T1)
    if not args.stream_only and not args.no_configs and w is WL.FRAME1004_W16:
        # the long streams: fewer timed passes (each is 1,000 to 20,000 frames)
        line["configs"] = {}
        for wl, st, wu in ((WL.STREAM1000_W64, 3, 1), (WL.STREAM10K_KF4, 1, 1), (WL.RING20K_W12, 1, 1),
                           (WL.WINDOWED1200, 2, 1)):
            sub, _ = stream_line(wl, st, wu, cpu=cpu)
            line["configs"][wl.name] = sub
    if cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = run_cpu_baseline(w, r["n_ctx"])
        if "scale_phase" in line:
            line["scale_phase"]["cpu_baseline"] = scale_phase_cpu(w, line["scale_phase"]["frames"])
        if "camera_head" in line:
            line["camera_head"]["cpu_baseline"] = run_cpu_baseline(WL.CAMERA_T1, plan_n_ctx(WL.CAMERA_T1))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
