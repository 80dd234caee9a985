"""Seeded synthetic frame streams for GCA (inputs only, no attention arithmetic).

Every tensor handed to either the HIP library or the CPU oracle comes from here,
so both sides always see the same bits.  Nothing in this module rotates, caches,
selects or attends; it only draws numbers.

Generator (counter based, so any element can be drawn independently):

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as
  published by Vigna): ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31``.
* a stream key is ``mix64(mix64(seed + G) ^ (4 * slot + tensor))`` with
  ``G = 0x9E3779B97F4A7C15`` and ``tensor`` 0 for Q, 1 for K, 2 for V,
  3 for the drift increments;
* element ``e`` draws ``u1 = mix64(key + (2e + 1) G)`` and
  ``u2 = mix64(key + (2e + 2) G)``, maps each to a uniform in (0, 1] as
  ``((u >> 11) + 1) * 2**-53`` and returns the Box-Muller normal
  ``sqrt(-2 ln u1) cos(2 pi u2)`` computed in float64, then rounded to float32
  and, for bf16 streams, rounded to bfloat16 (round to nearest even).

Frame streams follow the workloads of the lingbot-map pages: frames of
``T`` tokens, ``H`` heads of width ``D``, Q/K/V ~ N(0, 1); long streams cycle a
set of ``n_base`` distinct base frames (frames stay distinct through their
global frame index, which drives the temporal rotary angle).  The optional
drift adds a per-(head, dim) random walk to K and V:
``mu_f = mu_{f-1} + sigma * z_f`` with ``mu_0 = 0``.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DRIFT = 0, 1, 2, 3


def mix64(z):
    """SplitMix64 output function on uint64 scalars or arrays (wrapping)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, slot: int, tensor: int) -> np.uint64:
    with np.errstate(over="ignore"):
        a = mix64(np.uint64(seed) + GOLDEN)
        return mix64(a ^ np.uint64(4 * slot + tensor))


def normals(seed: int, slot: int, tensor: int, n: int, start: int = 0) -> np.ndarray:
    """float64 N(0,1) draws for elements [start, start + n) of one stream."""
    key = stream_key(seed, slot, tensor)
    e = np.arange(start, start + n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        u1 = mix64(key + (np.uint64(2) * e + np.uint64(1)) * GOLDEN)
        u2 = mix64(key + (np.uint64(2) * e + np.uint64(2)) * GOLDEN)
    a = ((u1 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    b = ((u2 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    return np.sqrt(-2.0 * np.log(a)) * np.cos(2.0 * np.pi * b)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # 32-bit arithmetic: the sum wraps only for NaN bit patterns, replaced below
    with np.errstate(over="ignore"):
        r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    out = r.view(np.float32)
    nan = np.isnan(x32)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x.astype(np.float32)
    if dtype == "bf16":
        return round_bf16(x32)
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


class FrameStream:
    """Deterministic Q/K/V frames of shape [T, H, D] (values exactly representable in `dtype`)."""

    def __init__(self, seed: int, T: int, H: int, D: int, dtype: str,
                 n_base: int | None = None, drift_sigma: float = 0.0):
        self.seed, self.T, self.H, self.D, self.dtype = seed, T, H, D, dtype
        self.n_base = n_base
        self.drift_sigma = drift_sigma
        self._drift_cache: dict[int, tuple[np.ndarray, np.ndarray]] = {0: (np.zeros((H, D)), np.zeros((H, D)))}
        self._base_cache: dict[tuple[int, int], np.ndarray] = {}

    def slot(self, frame: int) -> int:
        return frame if self.n_base is None else frame % self.n_base

    def base(self, frame: int, tensor: int) -> np.ndarray:
        """float32 draws (before any bf16 rounding) of one frame tensor [T, H, D]."""
        key = (self.slot(frame), tensor)
        hit = self._base_cache.get(key)
        if hit is not None:
            return hit
        n = self.T * self.H * self.D
        x = normals(self.seed, key[0], tensor, n).reshape(self.T, self.H, self.D).astype(np.float32)
        if self.n_base is not None:  # cycled streams: at most 3 * n_base tensors
            self._base_cache[key] = x
        return x

    def drift(self, frame: int) -> tuple[np.ndarray, np.ndarray]:
        """(mu_K, mu_V) of shape [H, D] after `frame` steps of the random walk."""
        if frame in self._drift_cache:
            return self._drift_cache[frame]
        f0 = max(k for k in self._drift_cache if k <= frame)
        mk, mv = self._drift_cache[f0]
        for f in range(f0 + 1, frame + 1):
            # one draw per (frame, tensor K|V, head, dim); slot = frame index itself
            z = normals(self.seed, f, TENSOR_DRIFT, 2 * self.H * self.D).reshape(2, self.H, self.D)
            mk = mk + self.drift_sigma * z[0]
            mv = mv + self.drift_sigma * z[1]
            if f % 64 == 0 or f == frame:
                self._drift_cache[f] = (mk, mv)
        return mk, mv

    def prefetch_drift(self, n_frames: int) -> None:
        """Walk the drift through frames 0 .. n_frames - 1 once and keep every
        frame's offsets, so later kv() calls only read (and may run in threads)."""
        mk, mv = self._drift_cache[0]
        for f in range(1, n_frames):
            if f in self._drift_cache:
                mk, mv = self._drift_cache[f]
                continue
            z = normals(self.seed, f, TENSOR_DRIFT, 2 * self.H * self.D).reshape(2, self.H, self.D)
            mk = mk + self.drift_sigma * z[0]
            mv = mv + self.drift_sigma * z[1]
            self._drift_cache[f] = (mk, mv)

    def q(self, frame: int) -> np.ndarray:
        return to_dtype(self.base(frame, TENSOR_Q), self.dtype)

    def kv(self, frame: int) -> tuple[np.ndarray, np.ndarray]:
        k = self.base(frame, TENSOR_K)
        v = self.base(frame, TENSOR_V)
        if self.drift_sigma:
            mk, mv = self.drift(frame)
            # the offset is added in float32 to the float32 base draw, then rounded
            k32 = k + mk.astype(np.float32)[None]
            v32 = v + mv.astype(np.float32)[None]
            if self.dtype == "bf16":
                return round_bf16(k32), round_bf16(v32)
            return k32, v32
        return to_dtype(k, self.dtype), to_dtype(v, self.dtype)

