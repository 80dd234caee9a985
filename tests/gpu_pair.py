"""Drive the HIP library and the CPU oracle through the same frame stream.

Used by the GPU parity tests.  Both sides get the same seeded inputs from
paged_kv_cache_gca_amd.synth; the oracle never sees a value produced by the
HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_cache_gca_amd import workloads as WL
from paged_kv_cache_gca_amd.synth import FrameStream

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def gca():
    from paged_kv_cache_gca_amd import gca as g
    return g


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact copy of float32 values (bf16-representable for bf16) to the GPU."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dtype]).cuda()


def stream_of(w: WL.Workload) -> FrameStream:
    return FrameStream(w.seed, w.T, w.H, w.D, w.dtype, n_base=w.n_base, drift_sigma=w.drift_sigma)


def oracle_cfg(w: WL.Workload, **kw) -> oracle.OracleConfig:
    d = dict(T=w.T, H=w.H, D=w.D, P=w.P, dtype=w.dtype, A=w.A, W=w.W, C=w.C, rope=w.rope,
             num_special=w.num_special, grid_h=w.grid_h, grid_w=w.grid_w, rope_theta=w.rope_theta,
             max_frames=w.n_frames, window=w.infer_window, overlap=w.infer_overlap)
    d.update(kw)
    return oracle.OracleConfig(**d)


class Pair:
    """A GPU cache and an oracle cache fed the same frames."""

    def __init__(self, w: WL.Workload, data: bool = True, out_dtype: str = "f32",
                 ring_init=None, compact_idx=None, num_pages: int = 0):
        g = gca()
        self.w = w
        self.data = data
        kw = {}
        okw = {}
        if ring_init is not None:
            kw["ring_init"] = list(ring_init)
            okw["ring_init"] = list(ring_init)
        if compact_idx is not None:
            kw["compact_idx"] = list(compact_idx)
            okw["compact_idx"] = list(compact_idx)
        if num_pages:
            kw["num_pages"] = num_pages
            okw["num_pages"] = num_pages
        self.cfg = g.Config.from_workload(w, out_dtype=out_dtype, **kw)
        self.gpu = g.Cache(self.cfg)
        self.orc = oracle.OracleCache(oracle_cfg(w, **okw))
        assert self.gpu.info.num_pages == self.orc.N
        self.fs = stream_of(w)
        self._dummy = None

    def kv(self, f):
        if self.data:
            k, v = self.fs.kv(f)
            return k, v, dev(k, self.w.dtype), dev(v, self.w.dtype)
        if self._dummy is None:
            z = torch.zeros((self.w.T, self.w.H, self.w.D), dtype=TORCH_DT[self.w.dtype], device="cuda")
            self._dummy = z
        return None, None, self._dummy, self._dummy

    def append(self, f, temp=False):
        k, v, kd, vd = self.kv(f)
        rc = self.gpu.append_frame(f, kd, vd, temp=temp)
        ro = self.orc.append(f, k, v, temp=temp)
        assert rc == ro == 0, (rc, ro)

    def evict(self):
        rc = self.gpu.evict_compact()
        ro = self.orc.evict()
        assert rc == ro == 0, (rc, ro)

    def rollback(self, f):
        rc = self.gpu.rollback_last_frame(f)
        ro = self.orc.rollback(f)
        assert rc == ro == 0, (rc, ro)

    def step(self, f):
        """append (+ evict for keyframes); returns whether f is a keyframe."""
        key = self.w.is_keyframe(f)
        self.append(f, temp=not key)
        if key:
            self.evict()
        return key

    def attend_gpu(self, f, q=None):
        if q is None:
            q = self.fs.q(f)
        qd = dev(q, self.w.dtype)
        out = torch.empty((self.w.T, self.w.H, self.w.D), dtype=TORCH_DT[self.cfg.out_dtype],
                          device="cuda")
        lse = torch.empty((self.w.T, self.w.H), dtype=torch.float32, device="cuda")
        assert self.gpu.attend(f, qd, out, lse) == 0
        return q, out, lse

    def check_state(self, with_select=True):
        """Bit-exact comparison of ring, page tables and gather list."""
        if with_select:
            assert self.gpu.select() == 0
        gs = self.gpu.export_state()
        os_ = self.orc.state()
        np.testing.assert_array_equal(gs["free"], os_["free"])
        np.testing.assert_array_equal(gs["frame_idx"], os_["frame_idx"])
        np.testing.assert_array_equal(gs["frame_pages"], os_["frame_pages"])
        np.testing.assert_array_equal(gs["traj_pages"], os_["traj_pages"])
        assert gs["traj_len"] == os_["traj_len"]
        if with_select:
            page, ln, n_ctx = self.orc.select()
            np.testing.assert_array_equal(gs["sel_page"], page)
            np.testing.assert_array_equal(gs["sel_len"], ln)
            assert gs["n_ctx"] == n_ctx
        return gs

    def check_pages(self, gs):
        """Live page contents bit for bit: V as given, K' as the oracle rotates
        and rounds it (the library evaluates the rotation in float64 with the
        same operations and rounds once, as the oracle does).  Returns the
        number of key values compared."""
        pages = np.concatenate([gs["frame_pages"].ravel(), gs["traj_pages"]])
        ktot = 0
        for p in pages:
            exp = self.orc.page(int(p))
            assert exp is not None
            ek, ev, valid = exp
            gk, gv = self.gpu.read_page(int(p))
            np.testing.assert_array_equal(gv[:, valid], ev[:, valid])
            np.testing.assert_array_equal(gk[:, valid], ek[:, valid])
            ktot += int(gk[:, valid].size)
        return ktot


class DeviceFrames:
    """A stream's frames on the device, made on demand (no copy per frame from
    the host): the distinct base frames are staged once; a drifting stream's
    key/value frames are made on the device from the float32 base draws plus
    the walk's float32 offsets, rounded once to the storage type (the
    generator's own recipe), and checked bit for bit against the generator on
    a few frames."""

    def __init__(self, w: WL.Workload, fs: FrameStream, check=(0, 1)):
        from paged_kv_cache_gca_amd.synth import TENSOR_K, TENSOR_V
        self.w, self.fs = w, fs
        self.n = w.n_frames if w.n_base is None else min(w.n_frames, w.n_base)
        dt = TORCH_DT[w.dtype]
        self.q = [dev(fs.q(f), w.dtype) for f in range(self.n)]
        if w.drift_sigma:
            fs.prefetch_drift(w.n_frames)
            self.bk = [torch.from_numpy(fs.base(f, TENSOR_K)).cuda() for f in range(self.n)]
            self.bv = [torch.from_numpy(fs.base(f, TENSOR_V)).cuda() for f in range(self.n)]
            mu = np.stack([np.stack(fs.drift(f)) for f in range(w.n_frames)]).astype(np.float32)
            self.mu = torch.from_numpy(mu).cuda()
        else:
            kv = [fs.kv(f) for f in range(self.n)]
            self.k = [dev(x[0], w.dtype) for x in kv]
            self.v = [dev(x[1], w.dtype) for x in kv]
        for f in check:
            k, v = fs.kv(f)
            kd, vd = self.kv(f)
            assert torch.equal(kd.cpu(), torch.from_numpy(k).to(dt)) and \
                torch.equal(vd.cpu(), torch.from_numpy(v).to(dt)), f

    def kv(self, f):
        i = f % self.n
        if self.w.drift_sigma:
            dt = TORCH_DT[self.w.dtype]
            return (self.bk[i] + self.mu[f, 0][None]).to(dt), (self.bv[i] + self.mu[f, 1][None]).to(dt)
        return self.k[i], self.v[i]


def host_frames(fs: FrameStream, frames, threads: int = 8):
    """(f, k, v) from the generator for `frames` in order, computed a few ahead
    in threads (numpy releases the interpreter lock in its array work)."""
    from concurrent.futures import ThreadPoolExecutor
    frames = list(frames)
    with ThreadPoolExecutor(threads) as ex:
        futs = {}
        for i, f in enumerate(frames):
            for j in range(i, min(i + 2 * threads, len(frames))):
                if frames[j] not in futs:
                    futs[frames[j]] = ex.submit(fs.kv, frames[j])
            k, v = futs.pop(f).result()
            yield f, k, v
