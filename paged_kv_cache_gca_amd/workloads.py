"""Synthetic GCA workloads shaped like the lingbot-map pages' streaming runs.

Frames are 518x378 images cut into 14x14 patches (37 x 27 = 999 patch tokens)
plus 5 special tokens, i.e. 1004 tokens per frame; the global attention uses
16 heads of width 64 (embed_dim 1024).  Stream lengths, window sizes and
keyframe intervals follow the runs the pages describe: 1,000-frame sequences
with a 64-frame window, 10,000-frame streams with keyframe-only caching, and
a strict 12-frame sliding window (current frame + 11 cached frames), and
windowed inference past the video rotary range (windows of 128 frames
overlapping by 8 keyframes).

Only parameters live here; no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens per frame
    H: int              # heads
    D: int              # head dim
    P: int              # page size (tokens)
    dtype: str          # "f32" | "bf16"
    n_frames: int       # frames in the stream
    A: int              # anchor frames
    W: int              # window keyframes (incl. the newest)
    C: int              # compact tokens kept per evicted frame
    rope: int           # 0 none, 1 3D (t, h, w)
    num_special: int
    grid_h: int
    grid_w: int
    keyframe_interval: int = 1
    n_base: int | None = None      # distinct base frames cycled (None: every frame distinct)
    drift_sigma: float = 0.0
    seed: int = 1
    rope_theta: float = 10000.0
    infer_window: int = 0          # windowed inference: frames per window (0 = off)
    infer_overlap: int = 0         # keyframes carried into the next window

    @property
    def n_keyframes(self) -> int:
        return (self.n_frames + self.keyframe_interval - 1) // self.keyframe_interval

    def is_keyframe(self, f: int) -> bool:
        return f % self.keyframe_interval == 0


TINY_F32 = Workload("tiny_f32_T64_H2", T=64, H=2, D=64, P=16, dtype="f32", n_frames=6,
                    A=1, W=2, C=1, rope=0, num_special=0, grid_h=8, grid_w=8, seed=1)

FRAME1004_W16 = Workload("bf16_T1004_H16_P16_W16_64f", T=1004, H=16, D=64, P=16, dtype="bf16",
                         n_frames=64, A=1, W=16, C=13, rope=1, num_special=5,
                         grid_h=27, grid_w=37, seed=2)

STREAM1000_W64 = Workload("bf16_T1004_H16_P64_W64_1000f", T=1004, H=16, D=64, P=64, dtype="bf16",
                          n_frames=1000, A=1, W=64, C=13, rope=1, num_special=5,
                          grid_h=27, grid_w=37, n_base=64, seed=3)

STREAM10K_KF4 = Workload("bf16_T1004_H16_P64_W32_10000f_kf4", T=1004, H=16, D=64, P=64,
                         dtype="bf16", n_frames=10000, A=1, W=32, C=13, rope=1, num_special=5,
                         grid_h=27, grid_w=37, keyframe_interval=4, n_base=64,
                         drift_sigma=0.1, seed=4)

RING20K_W12 = Workload("bf16_T1004_H16_P64_ring12_20000f", T=1004, H=16, D=64, P=64,
                       dtype="bf16", n_frames=20000, A=0, W=12, C=0, rope=1, num_special=5,
                       grid_h=27, grid_w=37, n_base=64, seed=5)

# The causal camera head's own cache: one camera token per frame under the same
# pool policy (anchor, sliding window, kept tokens of evicted frames) with its
# own rotary base; a decode-shaped attention (one query row per head).
CAMERA_T1 = Workload("bf16_T1_H16_P16_W32_camera_1000f", T=1, H=16, D=64, P=16, dtype="bf16",
                     n_frames=1000, A=1, W=32, C=1, rope=1, num_special=0, grid_h=1, grid_w=1,
                     n_base=64, seed=6, rope_theta=100.0)

# Windowed inference: windows of 128 frames overlapping by 8 keyframes, the
# documented setting for streams past the 320 views the video rotary embedding
# was trained on; every second frame a keyframe.
WINDOWED1200 = Workload("bf16_T1004_H16_P64_W32_win128_ov8_1200f_kf2", T=1004, H=16, D=64, P=64,
                        dtype="bf16", n_frames=1200, A=1, W=32, C=13, rope=1, num_special=5,
                        grid_h=27, grid_w=37, keyframe_interval=2, n_base=64, seed=7,
                        infer_window=128, infer_overlap=8)

# Small windowed streams: every third frame a keyframe, so that the oldest
# overlap keyframe sometimes falls outside the next window (f32), and every
# frame a keyframe with a ragged last page (bf16).
WINDOWED_SMALL_F32 = Workload("f32_T66_H2_P16_W3_win8_ov3_40f_kf3", T=66, H=2, D=64, P=16,
                              dtype="f32", n_frames=40, A=1, W=3, C=3, rope=1, num_special=2,
                              grid_h=8, grid_w=8, keyframe_interval=3, seed=8,
                              infer_window=8, infer_overlap=3)
WINDOWED_SMALL_BF16 = Workload("bf16_T70_H2_P32_W2_win6_ov2_30f", T=70, H=2, D=64, P=32,
                               dtype="bf16", n_frames=30, A=1, W=2, C=5, rope=1, num_special=6,
                               grid_h=8, grid_w=8, seed=9, infer_window=6, infer_overlap=2)

ALL = [TINY_F32, FRAME1004_W16, STREAM1000_W64, STREAM10K_KF4, RING20K_W12, CAMERA_T1,
       WINDOWED1200, WINDOWED_SMALL_F32, WINDOWED_SMALL_BF16]
