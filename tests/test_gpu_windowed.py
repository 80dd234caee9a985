"""GPU parity of windowed inference against the oracle, through the C ABI.

Windowed inference ("LingBot-Map runs 10,000 frames on monocular video",
section "Cloning and Installing"; the project summary's "Main features"
table): windows of a fixed frame span, overlapping by a few keyframes, with
window-relative temporal rotary positions.  The library keeps the raw K/V of
the last keyframes on the device and, at the first frame outside the window,
resets the ring and appends them again.  Bar as for every stream: ring, page
tables and gather lists bit-exact, K' and V pages bit-exact, attention within
the dtype's tolerance, at every step of the small streams and on sampled rows
of the 1,200-frame stream (ten window starts).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_gca_amd import workloads as WL
from tests.gpu_pair import DeviceFrames, Pair, dev, gca, host_frames, oracle_cfg
from tests.test_gpu_parity import _cmp_attention, _cmp_outputs, _rows

pytestmark = pytest.mark.gpu


def _origin_ok(p, f):
    assert p.gpu.query().window_origin == f - p.orc.rope_position(f)


@pytest.mark.parametrize("w", [WL.WINDOWED_SMALL_F32, WL.WINDOWED_SMALL_BF16], ids=lambda w: w.name)
def test_windowed_small_stream_full_parity(w):
    """Every step through the individual calls: the restarts inside
    gca_append_frame (with keyframes and non-keyframes arriving outside the
    window), page tables, pages and every output row against the oracle."""
    p = Pair(w)
    restarts = 0
    for f in range(w.n_frames):
        before = p.orc.rope_position(f) if f else 0
        key = p.step(f)
        restarts += f > 0 and before >= w.infer_window
        _origin_ok(p, f)
        gs = p.check_state()
        p.check_pages(gs)
        _cmp_attention(p, f)
        if not key:
            p.rollback(f)
            p.check_state(with_select=False)
    assert restarts >= 3


@pytest.mark.parametrize("w", [WL.WINDOWED_SMALL_F32, WL.WINDOWED_SMALL_BF16], ids=lambda w: w.name)
def test_windowed_step_matches_individual_calls_bitwise(w):
    """gca_step (restart, then the one update launch, the attention) gives
    bit for bit the outputs and state of the individual calls."""
    g = gca()
    a = g.Cache(g.Config.from_workload(w))
    b = g.Cache(g.Config.from_workload(w))
    p = Pair(w)
    shape = (w.T, w.H, w.D)
    for f in range(w.n_frames):
        key = w.is_keyframe(f)
        _, _, kd, vd = p.kv(f)
        qd = dev(p.fs.q(f), w.dtype)
        oa = torch.empty(shape, dtype=torch.float32, device="cuda")
        ob = torch.empty_like(oa)
        la = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
        lb = torch.empty_like(la)
        assert a.step(f, kd, vd, qd, oa, la, keyframe=key) == 0
        assert b.append_frame(f, kd, vd, temp=not key) == 0
        if key:
            assert b.evict_compact() == 0
        assert b.attend(f, qd, ob, lb) == 0
        if not key:
            assert b.rollback_last_frame(f) == 0
        assert torch.equal(oa, ob) and torch.equal(la, lb), f
        assert a.query().window_origin == b.query().window_origin
    sa, sb = a.export_state(), b.export_state()
    for k in ("free", "frame_idx", "frame_pages", "traj_pages"):
        np.testing.assert_array_equal(sa[k], sb[k])


def test_windowed1200_bookkeeping_every_step():
    """The 1,200-frame windowed stream (windows of 128 frames, 8 overlap
    keyframes): ring, page tables and gather list bit-exact at every step."""
    w = WL.WINDOWED1200
    p = Pair(w, data=False)
    restarts = 0
    for f in range(w.n_frames):
        restarts += f > 0 and p.orc.rope_position(f) >= w.infer_window
        key = p.step(f)
        p.check_state(with_select=True)
        if not key:
            p.rollback(f)
    assert restarts == 10
    assert p.gpu.query().window_origin == 1120


def test_windowed1200_stream_sampled():
    """The whole 1,200-frame stream on the GPU through gca_step; attention on
    sampled rows against the oracle around the first window start (frames 127
    to 129), around the last (1135 to 1137) and at the stream's end.  The
    oracle is fed every keyframe and every non-keyframe that starts a window
    (the others leave no trace)."""
    w = WL.WINDOWED1200
    p = Pair(w, data=False)
    p.orc = oracle.OracleCache(oracle_cfg(w))
    dfr = DeviceFrames(w, p.fs, check=(0, 1))
    rows = _rows(w.T, seed=7)
    samples = {127, 128, 129, 1135, 1136, 1137, 1197, 1198, 1199}
    out = torch.empty((w.T, w.H, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    oracle_frames = [f for f in range(w.n_frames) if w.is_keyframe(f) or f in samples]
    checked = 0
    nxt = 0          # the next frame the GPU has not stepped through
    for f, k, v in host_frames(p.fs, oracle_frames):
        for g_ in range(nxt, f):
            # a non-keyframe the oracle skips must not start a window
            assert w.is_keyframe(g_) or p.orc.rope_position(g_) < w.infer_window, g_
            kd, vd = dfr.kv(g_)
            assert p.gpu.step(g_, kd, vd, dfr.q[g_ % dfr.n], out, lse, keyframe=w.is_keyframe(g_)) == 0
        nxt = f + 1
        key = w.is_keyframe(f)
        kd, vd = dfr.kv(f)
        q = p.fs.q(f)
        assert p.gpu.step(f, kd, vd, dev(q, w.dtype), out, lse, keyframe=key) == 0
        assert p.orc.append(f, k, v, temp=not key) == 0
        if key:
            assert p.orc.evict() == 0
        if f in samples:
            _origin_ok(p, f)
            if key:
                st = p.gpu.export_state()
                page, ln, n_ctx = p.orc.select()
                np.testing.assert_array_equal(st["sel_page"], page)
                np.testing.assert_array_equal(st["sel_len"], ln)
                assert st["n_ctx"] == n_ctx
            _cmp_outputs(p, f, q, out, lse, rows)
            checked += 1
        if not key:
            assert p.orc.rollback(f) == 0
    assert checked == len(samples)
    gs = p.check_state(with_select=False)
    assert p.gpu.query().window_origin == 1120
    p.check_pages(gs)


def test_windowed_append_frames_and_errors():
    """A batched append may start a window but not cross into the next one
    (refused, nothing changed); the standalone rotation is limited to the
    window's positions."""
    g = gca()
    w = WL.Workload("win_batch", T=70, H=2, D=64, P=32, dtype="bf16", n_frames=20, A=1, W=8, C=5,
                    rope=1, num_special=6, grid_h=8, grid_w=8, seed=49, infer_window=6,
                    infer_overlap=2)
    p = Pair(w)
    for f in range(5):
        p.step(f)
    kv = [p.fs.kv(f) for f in (5, 6, 7)]
    k = dev(np.stack([x[0] for x in kv]), "bf16")
    v = dev(np.stack([x[1] for x in kv]), "bf16")
    before = p.gpu.export_state()
    # frames 5..7: frame 6 would start the next window inside the batch
    assert p.gpu.append_frames(5, k, v) == g.GCA_ERR_SEQUENCE
    after = p.gpu.export_state()
    for key in ("free", "frame_idx", "frame_pages", "traj_pages"):
        np.testing.assert_array_equal(before[key], after[key])
    assert p.gpu.append_frames(5, k[:1], v[:1]) == 0
    assert p.orc.append(5, *kv[0]) == 0
    # frames 6 and 7: the batch starts the next window (origin 4: keyframes 4
    # and 5 appended again), bit-exact against the oracle
    assert p.gpu.append_frames(6, k[1:], v[1:]) == 0
    assert p.orc.append(6, *kv[1]) == 0 and p.orc.append(7, *kv[2]) == 0
    assert p.gpu.query().window_origin == 4 and p.orc.rope_position(7) == 3
    gs = p.check_state()
    p.check_pages(gs)
    _cmp_attention(p, 7)
    x = torch.zeros((w.T, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    assert p.gpu.rope3d(w.infer_window - 1, x, torch.empty_like(x)) == 0
    assert p.gpu.rope3d(w.infer_window, x, torch.empty_like(x)) == g.GCA_ERR_CAPACITY


def test_windowed_step_static_matches_step_bitwise():
    """gca_step_static (scratch in the library's static array) starts the
    windows exactly as gca_step does: the same outputs bit for bit."""
    g = gca()
    w = WL.WINDOWED_SMALL_F32
    a = g.Cache(g.Config.from_workload(w))
    b = g.Cache(g.Config.from_workload(w))
    p = Pair(w)
    for f in range(w.n_frames):
        key = w.is_keyframe(f)
        _, _, kd, vd = p.kv(f)
        qd = dev(p.fs.q(f), w.dtype)
        oa = torch.empty((w.T, w.H, w.D), dtype=torch.float32, device="cuda")
        ob = torch.empty_like(oa)
        la = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
        lb = torch.empty_like(la)
        assert a.step(f, kd, vd, qd, oa, la, keyframe=key) == 0
        assert b.step_static(f, kd, vd, qd, ob, lb, keyframe=key) == 0
        assert torch.equal(oa, ob) and torch.equal(la, lb), f
    assert a.query().window_origin == b.query().window_origin > 0
