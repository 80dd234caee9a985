"""ctypes wrapper of the CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The product path (the HIP library and its
binding) never does.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgca_oracle.so")


class _Cfg(C.Structure):
    _fields_ = [
        ("T", C.c_int32), ("H", C.c_int32), ("D", C.c_int32), ("P", C.c_int32),
        ("bf16", C.c_int32),
        ("A", C.c_int32), ("W", C.c_int32), ("C", C.c_int32),
        ("compact_idx", C.POINTER(C.c_int32)),
        ("num_special", C.c_int32), ("grid_h", C.c_int32), ("grid_w", C.c_int32),
        ("rope", C.c_int32),
        ("rope_theta", C.c_double),
        ("sm_scale", C.c_double),
        ("max_frames", C.c_int64),
        ("num_pages", C.c_int32),
        ("ring_init", C.POINTER(C.c_int32)),
        ("window", C.c_int32),
        ("overlap", C.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        i32p, i64p, f32p, f64p = (C.POINTER(C.c_int32), C.POINTER(C.c_int64),
                                  C.POINTER(C.c_float), C.POINTER(C.c_double))
        L.orc_create.restype = C.c_void_p
        L.orc_create.argtypes = [C.POINTER(_Cfg)]
        L.orc_destroy.argtypes = [C.c_void_p]
        L.orc_reset.argtypes = [C.c_void_p]
        L.orc_num_pages.argtypes = [C.c_void_p]
        L.orc_pages_per_frame.argtypes = [C.c_void_p]
        L.orc_append.argtypes = [C.c_void_p, C.c_int64, f32p, f32p, C.c_int32]
        L.orc_evict.argtypes = [C.c_void_p]
        L.orc_rollback.argtypes = [C.c_void_p, C.c_int64]
        L.orc_n_ctx.restype = C.c_int64
        L.orc_n_ctx.argtypes = [C.c_void_p]
        L.orc_select.argtypes = [C.c_void_p, i32p, i32p, C.c_int32, i32p, i64p]
        L.orc_state.argtypes = [C.c_void_p, i32p, i32p, i64p, i32p, i32p, i32p, i32p, i64p]
        L.orc_context.argtypes = [C.c_void_p, f32p, f32p, i64p, i32p, C.c_int64]
        L.orc_page.argtypes = [C.c_void_p, C.c_int32, f32p, f32p, C.POINTER(C.c_uint8)]
        L.orc_rope.argtypes = [C.POINTER(_Cfg), C.c_int64, f32p, f64p]
        L.orc_rope_angle.restype = C.c_double
        L.orc_rope_angle.argtypes = [C.POINTER(_Cfg), C.c_int64, C.c_int32, C.c_int32]
        L.orc_round_bf16.restype = C.c_double
        L.orc_round_bf16.argtypes = [C.c_double]
        L.orc_attend.argtypes = [C.c_void_p, C.c_int64, f32p, i32p, C.c_int32, f64p, f64p, C.c_int32]
        L.orc_attend_frames.argtypes = [C.c_void_p, C.c_int64, C.c_int32, f32p, i32p, C.c_int32, f64p, f64p,
                                        C.c_int32]
        L.orc_default_compact.argtypes = [C.c_int32, C.c_int32, C.c_int32, i32p]
        L.orc_default_num_pages.restype = C.c_int64
        L.orc_default_num_pages.argtypes = [C.POINTER(_Cfg)]
        L.orc_rope_position.restype = C.c_int64
        L.orc_rope_position.argtypes = [C.c_void_p, C.c_int64]
        _lib = L
    return _lib


def _p(a, ct):
    return a.ctypes.data_as(C.POINTER(ct))


@dataclass
class OracleConfig:
    T: int
    H: int
    D: int = 64
    P: int = 16
    dtype: str = "bf16"
    A: int = 1
    W: int = 2
    C: int = 1
    compact_idx: list | None = None
    num_special: int = 0
    grid_h: int = 8
    grid_w: int = 8
    rope: int = 0
    rope_theta: float = 10000.0
    sm_scale: float | None = None
    max_frames: int = 64
    num_pages: int = 0
    ring_init: list | None = None
    window: int = 0      # windowed inference: frames per window (0 = off)
    overlap: int = 0     # keyframes carried into the next window
    _keep: list = field(default_factory=list, repr=False)

    def to_c(self) -> _Cfg:
        c = _Cfg()
        c.T, c.H, c.D, c.P = self.T, self.H, self.D, self.P
        c.bf16 = 1 if self.dtype == "bf16" else 0
        c.A, c.W, c.C = self.A, self.W, self.C
        self._keep = []
        if self.compact_idx is not None:
            arr = np.asarray(self.compact_idx, dtype=np.int32)
            self._keep.append(arr)
            c.compact_idx = _p(arr, C.c_int32)
        c.num_special, c.grid_h, c.grid_w = self.num_special, self.grid_h, self.grid_w
        c.rope = self.rope
        c.rope_theta = self.rope_theta
        c.sm_scale = self.sm_scale if self.sm_scale is not None else self.D ** -0.5
        c.max_frames = self.max_frames
        c.num_pages = self.num_pages
        if self.ring_init is not None:
            arr = np.asarray(self.ring_init, dtype=np.int32)
            self._keep.append(arr)
            c.ring_init = _p(arr, C.c_int32)
        c.window, c.overlap = self.window, self.overlap
        return c


def default_compact(T: int, num_special: int, C_: int) -> list[int]:
    out = np.zeros(max(C_, 1), dtype=np.int32)
    lib().orc_default_compact(T, num_special, C_, _p(out, C.c_int32))
    return out[:C_].tolist()


def default_num_pages(cfg: OracleConfig) -> int:
    c = cfg.to_c()
    return int(lib().orc_default_num_pages(C.byref(c)))


def rope(cfg: OracleConfig, frame: int, x: np.ndarray) -> np.ndarray:
    """float64 rotary embedding of x [T][H][D] at global frame index `frame`."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.float64)
    c = cfg.to_c()
    lib().orc_rope(C.byref(c), frame, _p(x, C.c_float), _p(y, C.c_double))
    return y


def rope_angle(cfg: OracleConfig, frame: int, tok: int, pair: int) -> float:
    c = cfg.to_c()
    return float(lib().orc_rope_angle(C.byref(c), frame, tok, pair))


def round_bf16(x: float) -> float:
    return float(lib().orc_round_bf16(float(x)))


class OracleCache:
    """The oracle's non-paged three-pool cache plus its allocator model."""

    def __init__(self, cfg: OracleConfig):
        self.cfg = cfg
        self._c = cfg.to_c()
        self.h = lib().orc_create(C.byref(self._c))
        if not self.h:
            raise ValueError("oracle rejected config")
        self.N = lib().orc_num_pages(self.h)
        self.ppf = lib().orc_pages_per_frame(self.h)

    def __del__(self):
        if getattr(self, "h", None):
            lib().orc_destroy(self.h)
            self.h = None

    def reset(self):
        lib().orc_reset(self.h)

    def append(self, frame: int, k: np.ndarray | None, v: np.ndarray | None, temp: bool = False) -> int:
        """Append raw K/V [T][H][D]; k = v = None appends for bookkeeping only."""
        if k is None and v is None:
            return lib().orc_append(self.h, frame, None, None, int(temp))
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        return lib().orc_append(self.h, frame, _p(k, C.c_float), _p(v, C.c_float), int(temp))

    def evict(self) -> int:
        return lib().orc_evict(self.h)

    def rollback(self, frame: int) -> int:
        return lib().orc_rollback(self.h, frame)

    def n_ctx(self) -> int:
        return int(lib().orc_n_ctx(self.h))

    def rope_position(self, frame: int) -> int:
        """temporal rotary position of `frame` (window-relative in windowed mode)"""
        return int(lib().orc_rope_position(self.h, frame))

    def select(self):
        cap = self.N + 8
        page = np.zeros(cap, np.int32)
        ln = np.zeros(cap, np.int32)
        n_sel = C.c_int32()
        n_ctx = C.c_int64()
        rc = lib().orc_select(self.h, _p(page, C.c_int32), _p(ln, C.c_int32), cap,
                              C.byref(n_sel), C.byref(n_ctx))
        assert rc == 0, rc
        return page[:n_sel.value].copy(), ln[:n_sel.value].copy(), n_ctx.value

    def state(self):
        N, ppf = self.N, self.ppf
        free = np.zeros(N, np.int32)
        n_free = C.c_int32()
        fidx = np.zeros(N, np.int64)
        fpages = np.zeros(N * ppf, np.int32)
        n_frames = C.c_int32()
        tp = np.zeros(N, np.int32)
        ntp = C.c_int32()
        tl = C.c_int64()
        lib().orc_state(self.h, _p(free, C.c_int32), C.byref(n_free), _p(fidx, C.c_int64),
                        _p(fpages, C.c_int32), C.byref(n_frames), _p(tp, C.c_int32),
                        C.byref(ntp), C.byref(tl))
        nf = n_frames.value
        return dict(free=free[:n_free.value].copy(), frame_idx=fidx[:nf].copy(),
                    frame_pages=fpages[:nf * ppf].reshape(nf, ppf).copy(),
                    traj_pages=tp[:ntp.value].copy(), traj_len=tl.value)

    def context(self):
        n = self.n_ctx()
        H, D = self.cfg.H, self.cfg.D
        k = np.zeros((n, H, D), np.float32)
        v = np.zeros((n, H, D), np.float32)
        tf = np.zeros(n, np.int64)
        tt = np.zeros(n, np.int32)
        rc = lib().orc_context(self.h, _p(k, C.c_float), _p(v, C.c_float), _p(tf, C.c_int64),
                               _p(tt, C.c_int32), n)
        assert rc == 0
        return k, v, tf, tt

    def page(self, page_id: int):
        H, P, D = self.cfg.H, self.cfg.P, self.cfg.D
        k = np.zeros((H, P, D), np.float32)
        v = np.zeros((H, P, D), np.float32)
        valid = np.zeros(P, np.uint8)
        rc = lib().orc_page(self.h, page_id, _p(k, C.c_float), _p(v, C.c_float),
                            valid.ctypes.data_as(C.POINTER(C.c_uint8)))
        if rc != 0:
            return None
        return k, v, valid.astype(bool)

    def attend(self, frame: int, q: np.ndarray, rows=None, threads: int = 0):
        T, H, D = self.cfg.T, self.cfg.H, self.cfg.D
        q = np.ascontiguousarray(q, dtype=np.float32)
        rows = np.arange(T, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
        out = np.zeros((len(rows), H, D), np.float64)
        lse = np.zeros((len(rows), H), np.float64)
        if threads <= 0:
            threads = os.cpu_count() or 1
        rc = lib().orc_attend(self.h, frame, _p(q, C.c_float), _p(rows, C.c_int32), len(rows),
                              _p(out, C.c_double), _p(lse, C.c_double), threads)
        if rc != 0:
            raise RuntimeError(f"oracle attend failed: {rc}")
        return out, lse

    def attend_frames(self, first: int, q: np.ndarray, rows=None, threads: int = 0):
        """Scale frames together: q [nf][T][H][D] of frames first .. first+nf-1
        (the last the newest appended frame), each rotated at its own frame
        index, over the one current context.  Returns out [nf][rows][H][D] and
        lse [nf][rows][H]."""
        T, H, D = self.cfg.T, self.cfg.H, self.cfg.D
        q = np.ascontiguousarray(q, dtype=np.float32)
        nf = q.shape[0]
        assert q.shape == (nf, T, H, D)
        rows = np.arange(T, dtype=np.int32) if rows is None else np.asarray(rows, dtype=np.int32)
        out = np.zeros((nf, len(rows), H, D), np.float64)
        lse = np.zeros((nf, len(rows), H), np.float64)
        if threads <= 0:
            threads = os.cpu_count() or 1
        rc = lib().orc_attend_frames(self.h, first, nf, _p(q, C.c_float), _p(rows, C.c_int32), len(rows),
                                     _p(out, C.c_double), _p(lse, C.c_double), threads)
        if rc != 0:
            raise RuntimeError(f"oracle attend_frames failed: {rc}")
        return out, lse
