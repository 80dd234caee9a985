"""Host-side tests (no GPU): the C ABI library loads and exports every symbol
declared in include/gca.h, and the host planner (the occupancy state machine
the cache runs before enqueuing kernels) validates configs and call sequences
and reports the same occupancy as the oracle's allocator model."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle
from paged_kv_cache_gca_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gca.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gca_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from paged_kv_cache_gca_amd import gca
    names = _declared()
    assert len(names) >= 24
    lib = ctypes.CDLL(gca.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    from paged_kv_cache_gca_amd import gca
    assert gca.status_string(0) == "ok"
    for code in range(-6, 0):
        assert gca.status_string(code) != "unknown status"


def cfg_of(w, **kw):
    from paged_kv_cache_gca_amd import gca
    return gca.Config.from_workload(w, **kw)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 128, -6),
    ("head_dim", 0, -1),
    ("page_size", 24, -1),
    ("page_size", 128, -6),
    ("window_frames", 0, -1),
    ("num_compact", 70, -1),
    ("num_anchor_frames", -1, -1),
    ("sm_scale", -0.125, -1),
    ("max_frames", 0, -1),
    ("compact_idx", [3, 3], -1),
    ("compact_idx", [64], -1),
])
def test_plan_rejects_bad_configs(field, value, code):
    from paged_kv_cache_gca_amd import gca
    c = cfg_of(WL.TINY_F32)
    setattr(c, field, value)
    if field == "compact_idx":
        c.num_compact = len(value)
    with pytest.raises(gca.GCAError) as ei:
        gca.Plan(c)
    assert ei.value.code == code


@pytest.mark.parametrize("window,overlap,A,W,code", [
    (8, 0, 1, 3, -1),     # a window needs at least one overlap keyframe
    (8, 8, 4, 8, -1),     # overlap below the window
    (8, 5, 1, 3, -1),     # at most A + W keyframes carried over
    (40, 17, 8, 16, -1),  # at most 16 (one re-append launch)
    (-1, 0, 1, 3, -1),
    (8, 3, 1, 3, 0),
    (40, 16, 8, 16, 0),
])
def test_plan_windowed_config_rules(window, overlap, A, W, code):
    from paged_kv_cache_gca_amd import gca
    c = cfg_of(WL.TINY_F32, infer_window=window, infer_overlap=overlap, num_anchor_frames=A,
               window_frames=W)
    if code:
        with pytest.raises(gca.GCAError) as e:
            gca.Plan(c)
        assert e.value.code == code
    else:
        gca.Plan(c)


def test_plan_rejects_rope_grid_mismatch_and_bad_ring():
    from paged_kv_cache_gca_amd import gca
    c = cfg_of(WL.FRAME1004_W16, grid_w=36)
    with pytest.raises(gca.GCAError):
        gca.Plan(c)
    c = cfg_of(WL.TINY_F32, ring_init=list(range(16)) + [0])
    with pytest.raises(gca.GCAError):
        gca.Plan(c)


def test_plan_sequence_errors():
    from paged_kv_cache_gca_amd import gca
    p = gca.Plan(cfg_of(WL.TINY_F32))
    assert p.attend(0) == gca.GCA_ERR_SEQUENCE          # nothing appended
    assert p.append(-1) == gca.GCA_ERR_INVALID_ARGUMENT
    assert p.append(0) == 0
    assert p.append(0) == gca.GCA_ERR_SEQUENCE          # not increasing
    assert p.attend(1) == gca.GCA_ERR_SEQUENCE          # not the last frame
    assert p.attend(0) == 0
    assert p.rollback(0) == gca.GCA_ERR_SEQUENCE        # not a TEMP frame
    assert p.append(1) == 0 and p.append(2) == 0 and p.append(3) == 0
    assert p.append(4) == gca.GCA_ERR_SEQUENCE          # W+1 window frames: evict first
    assert p.evict() == 0
    assert p.append(4, temp=True) == 0
    assert p.evict() == gca.GCA_ERR_SEQUENCE            # TEMP pending
    assert p.append(5) == gca.GCA_ERR_SEQUENCE
    before = p.query()
    assert p.rollback(4) == 0
    assert p.append(6) == gca.GCA_ERR_CAPACITY          # max_frames = 6
    info = p.query()
    assert info.temp_pending == 0 and before.temp_pending == 1
    assert info.free_pages == before.free_pages + info.pages_per_frame


def test_plan_out_of_pages_changes_nothing():
    from paged_kv_cache_gca_amd import gca
    p = gca.Plan(cfg_of(WL.TINY_F32, num_pages=9))
    assert p.append(0) == 0 and p.append(1) == 0
    before = p.query()
    assert p.append(2) == gca.GCA_ERR_OUT_OF_PAGES
    after = p.query()
    for f, _ in gca.gca_info._fields_:
        assert getattr(before, f) == getattr(after, f)


@pytest.mark.parametrize("w,expected", [
    (WL.TINY_F32, [0]),
    (WL.FRAME1004_W16, [0, 1, 2, 3, 4, 5, 129, 254, 379, 504, 629, 754, 879]),
    (WL.STREAM1000_W64, [0, 1, 2, 3, 4, 5, 129, 254, 379, 504, 629, 754, 879]),
    (WL.STREAM10K_KF4, [0, 1, 2, 3, 4, 5, 129, 254, 379, 504, 629, 754, 879]),
    (WL.RING20K_W12, []),
    (WL.CAMERA_T1, [0]),
], ids=lambda x: getattr(x, "name", ""))
def test_library_compact_offsets_pinned(w, expected):
    """The library's default compact list, read from its planner: the
    hand-derived lists of the compact-token reading (special tokens first,
    then evenly spaced patches), and a given list is kept as given."""
    from paged_kv_cache_gca_amd import gca
    assert gca.Plan(cfg_of(w)).compact() == expected
    assert gca.Plan(cfg_of(WL.TINY_F32, num_compact=3, compact_idx=[7, 2, 63])).compact() == [7, 2, 63]


def test_default_num_pages_matches_oracle_rule():
    from paged_kv_cache_gca_amd import gca
    for w in WL.ALL:
        p = gca.Plan(cfg_of(w))
        assert p.query().num_pages == oracle.default_num_pages(
            oracle.OracleConfig(T=w.T, H=w.H, D=w.D, P=w.P, A=w.A, W=w.W, C=w.C,
                                max_frames=w.n_frames, window=w.infer_window,
                                overlap=w.infer_overlap))


@pytest.mark.parametrize("w", WL.ALL, ids=lambda w: w.name)
def test_plan_occupancy_matches_oracle_every_step(w):
    from paged_kv_cache_gca_amd import gca
    p = gca.Plan(cfg_of(w))
    o = oracle.OracleCache(oracle.OracleConfig(T=w.T, H=w.H, D=w.D, P=w.P, A=w.A, W=w.W, C=w.C,
                                               num_special=w.num_special, max_frames=w.n_frames,
                                               window=w.infer_window, overlap=w.infer_overlap))
    n = min(w.n_frames, 3000)
    for f in range(n):
        key = w.is_keyframe(f)
        assert p.append(f, temp=not key) == 0
        assert o.append(f, None, None, temp=not key) == 0
        if key:
            assert p.evict() == 0 and o.evict() == 0
        assert p.attend(f) == 0
        info = p.query()
        assert info.n_ctx == o.n_ctx()
        if w.infer_window:
            assert info.window_origin == f - o.rope_position(f)
        if f % 97 == 0 or f == n - 1:
            page, ln, n_ctx = o.select()
            st = o.state()
            assert info.n_sel == len(page)
            assert info.free_pages == len(st["free"])
            assert info.traj_pages == len(st["traj_pages"])
            assert info.traj_tokens == st["traj_len"]
        if not key:
            assert p.rollback(f) == 0 and o.rollback(f) == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus 2 exits with a message, before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_bench_cpu_baseline_model_is_positive():
    """The CPU baseline's per-frame model (bookkeeping plus a + b*n_ctx through
    two timed frames) stays positive on tiny frames, where timing noise can
    make the later frame time shorter than the earlier one."""
    import bench
    for w in (WL.TINY_F32, WL.CAMERA_T1):
        r = bench.run_cpu_baseline(w, bench.plan_n_ctx(w))
        assert r["value"] > 0 and r["kind"] == "oracle" and r["cores"] >= 1


def test_committed_counter_summary_fields():
    """profiles/attn_traffic.json carries what the bench line reads from it."""
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    d = json.load(open(os.path.join(root, "profiles", "attn_traffic.json")))
    for key in ("kernel_hash", "fetch_scale", "write_scale", "workloads"):
        assert key in d
    assert len(d["kernel_hash"]) == 16
    from paged_kv_cache_gca_amd import workloads as WL
    assert WL.FRAME1004_W16.name in d["workloads"]
    for name, e in d["workloads"].items():
        assert name in {w.name for w in WL.ALL}
        assert e["bytes_per_launch"] > 0 and e["merge_us_per_frame"] > 0
        if "mfma_busy" in e:
            assert 0 < e["mfma_busy"] < 1
    # shader counters are taken for the two workloads with counter summaries
    for w in (WL.FRAME1004_W16, WL.STREAM1000_W64):
        assert 0 < d["workloads"][w.name]["mfma_busy"] < 1


def test_binding_refuses_bad_tensors_before_the_library():
    """Tensors the kernels would read or write out of bounds never reach the C
    ABI: wrong dtype, strided, short, or not on the GPU (checked in that order,
    so every rule shows on the CPU).  The cache handle is null here, so a
    tensor that got through would come back as GCA_ERR_INVALID_ARGUMENT from
    the library instead of raising."""
    import torch
    from paged_kv_cache_gca_amd import gca
    w = WL.TINY_F32
    c = object.__new__(gca.Cache)
    c.cfg = cfg_of(w)
    c.h = None
    c.device = 0
    shape = (w.T, w.H, w.D)
    good = torch.zeros(shape, dtype=torch.float32)
    bad = {
        "dtype": torch.zeros(shape, dtype=torch.bfloat16),
        "contiguous": torch.zeros((w.H, w.T, w.D), dtype=torch.float32).transpose(0, 1),
        "elements": torch.zeros((w.T - 1, w.H, w.D), dtype=torch.float32),
        "GPU": good,
    }
    calls = [
        lambda t: c.append_frame(0, t, good),
        lambda t: c.append_frame(0, good, t),
        lambda t: c.attend(0, t, good),
        lambda t: c.attend(0, good, t),
        lambda t: c.step(0, good, good, good, t),
        lambda t: c.rope3d(0, t, good),
        lambda t: c.append_frames(0, t[None], good[None]),
        lambda t: c.attend_frames(0, t[None], good[None]),
    ]
    for rule, t in bad.items():
        for call in calls:
            with pytest.raises(gca.GCAError) as ei:
                call(t)
            assert ei.value.code == gca.GCA_ERR_INVALID_ARGUMENT
            assert rule in str(ei.value) or rule == "elements" and "elements" in str(ei.value)
    # lse: float32 [T][H]
    with pytest.raises(gca.GCAError):
        c.attend(0, good, good, torch.zeros((w.T, w.H), dtype=torch.float64))
    # frame counts of the batched calls must agree
    with pytest.raises(gca.GCAError):
        c.append_frames(0, torch.stack([good, good]), good[None])
    c.h = None
