"""gca_step_static, the allocation-free variant of gca_step, against gca_step
through the C ABI: two caches fed the same frames, one stepping each way;
outputs and LSEs must agree to the attention bar (they are in fact bitwise
equal: same kernels, same split points), state and gather lists bit-exact.
Two calls in a row on different caches, the second with a smaller frame, so
the second reads the static array after the first left its data there; the
second cache is also checked against the oracle.  A step whose scratch
exceeds the array is refused and changes nothing."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_gca_amd import workloads as WL
from tests.gpu_pair import dev, gca, oracle_cfg, stream_of

pytestmark = pytest.mark.gpu

BIG = WL.Workload("static_big", T=1004, H=16, D=64, P=16, dtype="bf16", n_frames=24, A=1, W=8, C=13,
                  rope=1, num_special=5, grid_h=27, grid_w=37, keyframe_interval=3, seed=61)
SMALL = WL.Workload("static_small", T=300, H=4, D=64, P=32, dtype="bf16", n_frames=12, A=1, W=3, C=5,
                    rope=1, num_special=3, grid_h=9, grid_w=33, keyframe_interval=2, seed=62)


def _twin_stream(w, frames, check_oracle=False):
    g = gca()
    cfg = g.Config.from_workload(w)
    ca, cb = g.Cache(cfg), g.Cache(cfg)
    orc = oracle.OracleCache(oracle_cfg(w)) if check_oracle else None
    fs = stream_of(w)
    for f in frames:
        k, v = fs.kv(f)
        q = fs.q(f)
        kd, vd, qd = dev(k, w.dtype), dev(v, w.dtype), dev(q, w.dtype)
        key = w.is_keyframe(f)
        oa = torch.empty((w.T, w.H, w.D), dtype=torch.float32, device="cuda")
        ob = torch.full_like(oa, float("nan"))
        la = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
        lb = torch.full_like(la, float("nan"))
        assert ca.step(f, kd, vd, qd, oa, la, keyframe=key) == 0
        assert cb.step_static(f, kd, vd, qd, ob, lb, keyframe=key) == 0
        torch.cuda.synchronize()
        err = float((oa - ob).abs().max())
        lerr = float((la - lb).abs().max())
        assert torch.isfinite(ob).all() and err <= 2e-2 and lerr <= 2.0 ** -8, (w.name, f, err, lerr)
        assert torch.equal(oa, ob) and torch.equal(la, lb), (w.name, f, err, lerr)
        sa, sb = ca.export_state(), cb.export_state()
        for name in ("free", "frame_idx", "frame_pages", "traj_pages"):
            np.testing.assert_array_equal(sa[name], sb[name], err_msg=f"{name} frame {f}")
        if orc is not None:
            assert orc.append(f, k, v, temp=not key) == 0
            if key:
                assert orc.evict() == 0
            o_ref, lse_ref = orc.attend(f, q)
            assert np.abs(ob.cpu().numpy().astype(np.float64) - o_ref).max() <= 2e-2, f
            if not key:
                assert orc.rollback(f) == 0
    ca.close()
    cb.close()


def test_static_step_two_calls_second_smaller():
    # the bench shape (split context: partials in the array), then a smaller frame
    _twin_stream(BIG, range(BIG.n_frames))
    _twin_stream(SMALL, range(SMALL.n_frames), check_oracle=True)


def test_static_step_refuses_a_step_beyond_the_array():
    """H = 256 heads of 2100 tokens: the prepared queries alone (65.6 MiB) exceed
    the 64 MiB array; refused with GCA_ERR_CAPACITY before anything is enqueued."""
    g = gca()
    w = WL.Workload("static_huge", T=2100, H=256, D=64, P=64, dtype="bf16", n_frames=2, A=0, W=1, C=0,
                    rope=0, num_special=0, grid_h=42, grid_w=50, seed=63)
    c = g.Cache(g.Config.from_workload(w))
    x = torch.zeros((w.T, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((w.T, w.H, w.D), dtype=torch.float32, device="cuda")
    info = c.query()
    assert c.step_static(0, x, x, x, out) == g.GCA_ERR_CAPACITY
    assert "scratch" in g.last_error()
    after = c.query()
    assert after.last_frame == info.last_frame and after.free_pages == info.free_pages
    assert c.step(0, x, x, x, out) == 0   # the cache's own workspace still serves it
    c.close()
