"""Python binding of libgca.so (the C ABI in include/gca.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch provides device memory
and the stream); the binding passes their data pointers and the current
stream's handle.  If the library is not built, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgca.so")

GCA_OK = 0
GCA_ERR_INVALID_ARGUMENT = -1
GCA_ERR_SEQUENCE = -2
GCA_ERR_OUT_OF_PAGES = -3
GCA_ERR_CAPACITY = -4
GCA_ERR_HIP = -5
GCA_ERR_UNSUPPORTED = -6
GCA_F32, GCA_BF16 = 0, 1
GCA_APPEND_TEMP = 1
STEP_KEYFRAME = 1
STATIC_SCRATCH_BYTES = 64 << 20  # GCA_STATIC_SCRATCH_BYTES
KIND = {"append": 0, "evict": 1, "select": 2, "attn": 3, "merge": 4, "rope": 5, "update": 6}


class GCAError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {code} ({status_string(code)})")


class gca_config(C.Structure):
    _fields_ = [
        ("tokens_per_frame", C.c_int32), ("num_heads", C.c_int32), ("head_dim", C.c_int32),
        ("page_size", C.c_int32), ("dtype", C.c_int32), ("out_dtype", C.c_int32),
        ("num_anchor_frames", C.c_int32), ("window_frames", C.c_int32), ("num_compact", C.c_int32),
        ("compact_idx", C.POINTER(C.c_int32)),
        ("num_special", C.c_int32), ("grid_h", C.c_int32), ("grid_w", C.c_int32),
        ("rope", C.c_int32), ("rope_theta", C.c_float), ("sm_scale", C.c_float),
        ("max_frames", C.c_int64), ("num_pages", C.c_int32),
        ("ring_init", C.POINTER(C.c_int32)),
        ("infer_window", C.c_int32), ("infer_overlap", C.c_int32),
    ]


class gca_info(C.Structure):
    _fields_ = [
        ("pages_per_frame", C.c_int32), ("num_pages", C.c_int32), ("free_pages", C.c_int32),
        ("anchor_frames", C.c_int32), ("window_frames", C.c_int32), ("temp_pending", C.c_int32),
        ("traj_pages", C.c_int32), ("n_sel", C.c_int32), ("traj_tokens", C.c_int64),
        ("n_ctx", C.c_int64), ("last_frame", C.c_int64), ("max_splits", C.c_int32),
        ("reserved", C.c_int32), ("window_origin", C.c_int64),
    ]


class gca_state_view(C.Structure):
    _fields_ = [
        ("free_ring", C.POINTER(C.c_int32)), ("frame_idx", C.POINTER(C.c_int64)),
        ("frame_pages", C.POINTER(C.c_int32)), ("traj_pages", C.POINTER(C.c_int32)),
        ("sel_page", C.POINTER(C.c_int32)), ("sel_len", C.POINTER(C.c_int32)),
        ("n_free", C.c_int32), ("n_frames", C.c_int32), ("n_traj_pages", C.c_int32),
        ("n_sel", C.c_int32), ("traj_tokens", C.c_int64), ("n_ctx", C.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python paged_kv_cache_gca_amd/build.py")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, u32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32
    sigs = {
        "gca_cache_create": [C.POINTER(gca_config), C.POINTER(vp)],
        "gca_cache_destroy": [vp],
        "gca_cache_reset": [vp, vp],
        "gca_append_frame": [vp, i64, vp, vp, u32, vp],
        "gca_evict_compact": [vp, vp],
        "gca_attend": [vp, i64, vp, vp, vp, vp],
        "gca_attend_frames": [vp, i64, i32, vp, vp, vp, vp],
        "gca_append_frames": [vp, i64, i32, vp, vp, vp],
        "gca_rollback_last_frame": [vp, i64, vp],
        "gca_step": [vp, i64, vp, vp, vp, vp, vp, u32, vp],
        "gca_step_static": [vp, i64, vp, vp, vp, vp, vp, u32, vp],
        "gca_select": [vp, vp],
        "gca_rope3d": [vp, i64, vp, vp, vp],
        "gca_query": [vp, C.POINTER(gca_info)],
        "gca_export_state": [vp, C.POINTER(gca_state_view), vp],
        "gca_read_page": [vp, i32, vp, vp, vp],
        "gca_profile_enable": [vp, i32, u32],
        "gca_profile_read": [vp, i32, C.POINTER(C.c_double), C.POINTER(i32)],
        "gca_plan_create": [C.POINTER(gca_config), C.POINTER(vp)],
        "gca_plan_destroy": [vp],
        "gca_plan_reset": [vp],
        "gca_plan_append": [vp, i64, u32],
        "gca_plan_evict": [vp],
        "gca_plan_attend": [vp, i64],
        "gca_plan_rollback": [vp, i64],
        "gca_plan_query": [vp, C.POINTER(gca_info)],
        "gca_plan_compact": [vp, C.POINTER(i32), i32, C.POINTER(i32)],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = C.c_int
    L.gca_status_string.argtypes = [C.c_int]
    L.gca_status_string.restype = C.c_char_p
    L.gca_last_error.argtypes = []
    L.gca_last_error.restype = C.c_char_p
    return L


_lib = _load()


def lib():
    return _lib


def status_string(code: int) -> str:
    return _lib.gca_status_string(code).decode()


def last_error() -> str:
    return _lib.gca_last_error().decode()


def _check(rc: int, what: str):
    if rc != GCA_OK:
        extra = f" [{last_error()}]" if rc == GCA_ERR_HIP else ""
        raise GCAError(rc, what + extra)


@dataclass
class Config:
    tokens_per_frame: int
    num_heads: int
    head_dim: int = 64
    page_size: int = 16
    dtype: str = "bf16"
    out_dtype: str = "f32"
    num_anchor_frames: int = 1
    window_frames: int = 16
    num_compact: int = 13
    compact_idx: list | None = None
    num_special: int = 0
    grid_h: int = 1
    grid_w: int = 1
    rope: int = 0
    rope_theta: float = 10000.0
    sm_scale: float | None = None
    max_frames: int = 64
    num_pages: int = 0
    ring_init: list | None = None
    infer_window: int = 0   # windowed inference: frames per window (0 = off)
    infer_overlap: int = 0  # keyframes carried into the next window

    def to_c(self):
        keep = []
        c = gca_config()
        c.tokens_per_frame, c.num_heads, c.head_dim = self.tokens_per_frame, self.num_heads, self.head_dim
        c.page_size = self.page_size
        c.dtype = GCA_BF16 if self.dtype == "bf16" else GCA_F32
        c.out_dtype = GCA_BF16 if self.out_dtype == "bf16" else GCA_F32
        c.num_anchor_frames, c.window_frames, c.num_compact = (self.num_anchor_frames,
                                                               self.window_frames, self.num_compact)
        if self.compact_idx is not None:
            arr = (C.c_int32 * len(self.compact_idx))(*self.compact_idx)
            keep.append(arr)
            c.compact_idx = C.cast(arr, C.POINTER(C.c_int32))
        c.num_special, c.grid_h, c.grid_w = self.num_special, self.grid_h, self.grid_w
        c.rope, c.rope_theta = self.rope, self.rope_theta
        c.sm_scale = (self.sm_scale if self.sm_scale is not None
                      else (self.head_dim ** -0.5 if self.head_dim > 0 else 1.0))
        c.max_frames, c.num_pages = self.max_frames, self.num_pages
        if self.ring_init is not None:
            arr = (C.c_int32 * len(self.ring_init))(*self.ring_init)
            keep.append(arr)
            c.ring_init = C.cast(arr, C.POINTER(C.c_int32))
        c.infer_window, c.infer_overlap = self.infer_window, self.infer_overlap
        return c, keep

    @staticmethod
    def from_workload(w, **kw) -> "Config":
        d = dict(tokens_per_frame=w.T, num_heads=w.H, head_dim=w.D, page_size=w.P, dtype=w.dtype,
                 num_anchor_frames=w.A, window_frames=w.W, num_compact=w.C, rope=w.rope,
                 num_special=w.num_special, grid_h=w.grid_h, grid_w=w.grid_w, rope_theta=w.rope_theta,
                 max_frames=w.n_frames, infer_window=w.infer_window, infer_overlap=w.infer_overlap)
        d.update(kw)
        return Config(**d)


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def check_tensors(specs, device: int | None = None):
    """Refuse tensors the kernels would read or write out of bounds.  `specs`
    lists (tensor, name, dtype, numel): each must be a torch tensor of `dtype`
    ("bf16" | "f32"), contiguous, with `numel` elements; then every one must be
    on the GPU (device index `device` when given).  Raises GCAError
    (GCA_ERR_INVALID_ARGUMENT) before anything reaches the library."""
    import torch
    for t, what, dtype, numel in specs:
        want = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
        why = None
        if not isinstance(t, torch.Tensor):
            why = f"not a torch tensor ({type(t).__name__})"
        elif t.dtype != want:
            why = f"dtype {t.dtype}, expected {want}"
        elif not t.is_contiguous():
            why = "not contiguous"
        elif t.numel() != numel:
            why = f"{t.numel()} elements, expected {numel}"
        if why is not None:
            raise GCAError(GCA_ERR_INVALID_ARGUMENT, f"{what}: {why}")
    for t, what, _, _ in specs:
        why = None
        if t.device.type != "cuda":
            why = f"on {t.device}, expected a GPU tensor"
        elif device is not None and t.device.index != device:
            why = f"on {t.device}, the cache lives on cuda:{device}"
        if why is not None:
            raise GCAError(GCA_ERR_INVALID_ARGUMENT, f"{what}: {why}")


class Plan:
    """Host-only occupancy planner (no device)."""

    def __init__(self, cfg: Config):
        c, self._keep = cfg.to_c()
        h = C.c_void_p()
        _check(_lib.gca_plan_create(C.byref(c), C.byref(h)), "gca_plan_create")
        self.h = h

    def __del__(self):
        if getattr(self, "h", None):
            _lib.gca_plan_destroy(self.h)
            self.h = None

    def reset(self):
        return _lib.gca_plan_reset(self.h)

    def append(self, frame: int, temp: bool = False) -> int:
        return _lib.gca_plan_append(self.h, frame, GCA_APPEND_TEMP if temp else 0)

    def evict(self) -> int:
        return _lib.gca_plan_evict(self.h)

    def attend(self, frame: int) -> int:
        return _lib.gca_plan_attend(self.h, frame)

    def rollback(self, frame: int) -> int:
        return _lib.gca_plan_rollback(self.h, frame)

    def query(self) -> gca_info:
        inf = gca_info()
        _check(_lib.gca_plan_query(self.h, C.byref(inf)), "gca_plan_query")
        return inf

    def compact(self) -> list[int]:
        """The compact token offsets the config resolves to."""
        n = C.c_int32()
        _lib.gca_plan_compact(self.h, None, 0, C.byref(n))
        buf = (C.c_int32 * max(n.value, 1))()
        _check(_lib.gca_plan_compact(self.h, buf, n.value, C.byref(n)), "gca_plan_compact")
        return list(buf[:n.value])


class Cache:
    """A GCA paged KV cache on the current HIP device."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        c, self._keep = cfg.to_c()
        h = C.c_void_p()
        _check(_lib.gca_cache_create(C.byref(c), C.byref(h)), "gca_cache_create")
        self.h = h
        self.info = self.query()
        import torch
        self.device = torch.cuda.current_device()

    def close(self):
        if getattr(self, "h", None):
            _check(_lib.gca_cache_destroy(self.h), "gca_cache_destroy")
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # raw calls return the status code; the checked wrappers raise GCAError
    def reset(self, stream=None) -> int:
        return _lib.gca_cache_reset(self.h, _stream(stream))

    # shapes the kernels read and write: one frame is [T][H][D] of the cache
    # dtype (queries, keys, values) or of out_dtype (outputs); lse is [T][H] f32
    def _validate(self, n: int = 1, out=None, lse=None, **inputs):
        c = self.cfg
        rows = n * c.tokens_per_frame * c.num_heads
        specs = [(t, name, c.dtype, rows * c.head_dim) for name, t in inputs.items()]
        if out is not None:
            specs.append((out, "out", c.out_dtype, rows * c.head_dim))
        if lse is not None:
            specs.append((lse, "lse", "f32", rows))
        check_tensors(specs, self.device)

    def append_frame(self, frame: int, k, v, temp: bool = False, stream=None) -> int:
        self._validate(k=k, v=v)
        return _lib.gca_append_frame(self.h, frame, _ptr(k), _ptr(v),
                                     GCA_APPEND_TEMP if temp else 0, _stream(stream))

    def evict_compact(self, stream=None) -> int:
        return _lib.gca_evict_compact(self.h, _stream(stream))

    def attend(self, frame: int, q, out, lse=None, stream=None) -> int:
        self._validate(out=out, lse=lse, q=q)
        return _lib.gca_attend(self.h, frame, _ptr(q), _ptr(out), _ptr(lse), _stream(stream))

    def append_frames(self, first: int, k, v, stream=None) -> int:
        """keyframes first .. first+n-1 in one launch: k, v [n][T][H][D]"""
        n = int(k.shape[0]) if hasattr(k, "shape") and len(k.shape) else 0
        if n < 1 or not hasattr(v, "shape") or int(v.shape[0]) != n:
            raise GCAError(GCA_ERR_INVALID_ARGUMENT, "append_frames: k and v need the same leading frame count")
        self._validate(n, k=k, v=v)
        return _lib.gca_append_frames(self.h, first, int(k.shape[0]), _ptr(k), _ptr(v), _stream(stream))

    def attend_frames(self, first: int, q, out, lse=None, stream=None) -> int:
        """scale frames together: q [n][T][H][D] of frames first .. first+n-1"""
        n = int(q.shape[0]) if hasattr(q, "shape") and len(q.shape) else 0
        if n < 1:
            raise GCAError(GCA_ERR_INVALID_ARGUMENT, "attend_frames: q needs a leading frame count")
        self._validate(n, out=out, lse=lse, q=q)
        return _lib.gca_attend_frames(self.h, first, int(q.shape[0]), _ptr(q), _ptr(out), _ptr(lse),
                                      _stream(stream))

    def rollback_last_frame(self, frame: int, stream=None) -> int:
        return _lib.gca_rollback_last_frame(self.h, frame, _stream(stream))

    def step(self, frame: int, k, v, q, out, lse=None, keyframe: bool = True, stream=None) -> int:
        """append (+ evict) + attend (+ rollback for a non-keyframe) in one call"""
        self._validate(out=out, lse=lse, k=k, v=v, q=q)
        return _lib.gca_step(self.h, frame, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(lse),
                             STEP_KEYFRAME if keyframe else 0, _stream(stream))

    def step_static(self, frame: int, k, v, q, out, lse=None, keyframe: bool = True, stream=None) -> int:
        """step() with its scratch in the library's fixed device array (no allocation)"""
        self._validate(out=out, lse=lse, k=k, v=v, q=q)
        return _lib.gca_step_static(self.h, frame, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(lse),
                                    STEP_KEYFRAME if keyframe else 0, _stream(stream))

    def select(self, stream=None) -> int:
        return _lib.gca_select(self.h, _stream(stream))

    def rope3d(self, frame: int, x, y, stream=None) -> int:
        self._validate(x=x, y=y)
        return _lib.gca_rope3d(self.h, frame, _ptr(x), _ptr(y), _stream(stream))

    def query(self) -> gca_info:
        inf = gca_info()
        _check(_lib.gca_query(self.h, C.byref(inf)), "gca_query")
        return inf

    def export_state(self, stream=None) -> dict:
        import numpy as np
        inf = self.query()
        n_live = inf.anchor_frames + inf.window_frames
        free = np.zeros(max(inf.num_pages, 1), np.int32)
        fidx = np.zeros(max(n_live, 1), np.int64)
        fpages = np.zeros(max(n_live * inf.pages_per_frame, 1), np.int32)
        tp = np.zeros(max(inf.traj_pages, 1), np.int32)
        sp = np.zeros(max(inf.n_sel, 1), np.int32)
        sl = np.zeros(max(inf.n_sel, 1), np.int32)
        v = gca_state_view()
        v.free_ring = free.ctypes.data_as(C.POINTER(C.c_int32))
        v.frame_idx = fidx.ctypes.data_as(C.POINTER(C.c_int64))
        v.frame_pages = fpages.ctypes.data_as(C.POINTER(C.c_int32))
        v.traj_pages = tp.ctypes.data_as(C.POINTER(C.c_int32))
        v.sel_page = sp.ctypes.data_as(C.POINTER(C.c_int32))
        v.sel_len = sl.ctypes.data_as(C.POINTER(C.c_int32))
        _check(_lib.gca_export_state(self.h, C.byref(v), _stream(stream)), "gca_export_state")
        return dict(free=free[:v.n_free].copy(), frame_idx=fidx[:v.n_frames].copy(),
                    frame_pages=fpages[:v.n_frames * inf.pages_per_frame]
                    .reshape(v.n_frames, inf.pages_per_frame).copy(),
                    traj_pages=tp[:v.n_traj_pages].copy(), traj_len=v.traj_tokens,
                    sel_page=sp[:v.n_sel].copy(), sel_len=sl[:v.n_sel].copy(), n_ctx=v.n_ctx)

    def read_page(self, page: int, stream=None):
        """(K, V) of one page as numpy float32 arrays [H][P][D]."""
        import numpy as np
        cfg = self.cfg
        n = cfg.num_heads * cfg.page_size * cfg.head_dim
        if cfg.dtype == "bf16":
            kb = np.zeros(n, np.uint16)
            vb = np.zeros(n, np.uint16)
        else:
            kb = np.zeros(n, np.float32)
            vb = np.zeros(n, np.float32)
        _check(_lib.gca_read_page(self.h, page, kb.ctypes.data_as(C.c_void_p),
                                  vb.ctypes.data_as(C.c_void_p), _stream(stream)), "gca_read_page")
        shape = (cfg.num_heads, cfg.page_size, cfg.head_dim)
        if cfg.dtype == "bf16":
            kf = (kb.astype(np.uint32) << 16).view(np.float32)
            vf = (vb.astype(np.uint32) << 16).view(np.float32)
            return kf.reshape(shape), vf.reshape(shape)
        return kb.reshape(shape), vb.reshape(shape)

    def profile_enable(self, capacity: int, kinds=("append", "evict", "select", "attn", "merge", "rope")):
        mask = 0
        for k in kinds:
            mask |= 1 << KIND[k]
        _check(_lib.gca_profile_enable(self.h, capacity, mask), "gca_profile_enable")

    def profile_read(self, kind: str):
        ms = C.c_double()
        n = C.c_int32()
        _check(_lib.gca_profile_read(self.h, KIND[kind], C.byref(ms), C.byref(n)), "gca_profile_read")
        return ms.value, n.value
