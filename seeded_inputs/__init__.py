"""Seeded synthetic inputs for masked attention forward + JVP.

This module is the one piece shared by the oracle side (tests, the CPU
baseline) and the GPU side (tests, bench, smoke).  It holds the workload
recipe only -- shapes, seeds, value distributions and the bf16 input
rounding -- and none of the attention arithmetic.

Recipe (stand-in for Wan2.1 DiT self-attention activations at 480p with
21 latent frames; Causal-rCM, arXiv 2606.25473, section 4 "Experiments"):

* one PCG64 stream per (workload seed, config id, tensor, b, h), from
  ``np.random.SeedSequence([20261203, cfg_id, tensor_id, b, h])`` with
  tensor ids q=0, k=1, v=2, tq=3, tk=4, tv=5 and, for the backward, the
  output gradient do=6, so that any (b, h) slice can be regenerated on its
  own;
* every slice is ``standard_normal((N, d), float32)``;
* q and k are RMS-normalised per token over the head dimension when the
  workload asks for it: x / sqrt(mean(x^2) + 1e-6), computed in float32;
* tangents are multiplied by their standard deviation;
* bf16 workloads round every value to bf16 with round-to-nearest-even; the
  oracle receives exactly these rounded values (widened to float64), so
  input rounding is never counted as error.
"""
from __future__ import annotations

from dataclasses import dataclass
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

TENSORS = ("q", "k", "v", "tq", "tk", "tv")
# The output gradient of the backward (dL/do): its own stream, id 6.
GRAD_TENSORS = ("do",)
_TENSOR_IDS = {t: i for i, t in enumerate(TENSORS + GRAD_TENSORS)}
ROOT_SEED = 20261203


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: geometry, mask descriptor and value recipe."""

    name: str
    cfg_id: int
    batch: int
    heads: int
    head_dim: int
    tokens_per_frame: int
    n_frames: int
    frames_per_chunk: int
    tf_layout: int
    dtype: str  # "bf16" or "fp32"
    tangent_std: float
    rms_norm_qk: bool
    # chunk sizes in frames, first to last, when the chunks are not all equal
    # (a cA-B pattern); empty: n_frames / frames_per_chunk chunks of equal size
    chunk_frames: tuple = ()

    @property
    def tokens_per_side(self) -> int:
        return self.tokens_per_frame * self.n_frames

    @property
    def seq_len(self) -> int:
        return self.tokens_per_side * (2 if self.tf_layout else 1)

    @property
    def shape(self):
        return (self.batch, self.heads, self.seq_len, self.head_dim)

    @property
    def desc(self):
        return (self.tokens_per_frame, self.n_frames, self.frames_per_chunk, self.tf_layout)

    @property
    def chunks(self) -> tuple:
        """Chunk sizes in frames."""
        if self.chunk_frames:
            return tuple(self.chunk_frames)
        return (self.frames_per_chunk,) * (self.n_frames // self.frames_per_chunk)

    def mask_ranges(self):
        """The workload's mask as (seq_len, query groups x key intervals)."""
        return chunked_mask_ranges(self.tokens_per_frame, self.chunks, self.tf_layout)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads: tiny fp32 teacher forcing; frame-wise block-causal
# (21 x 1560 tokens); frame-wise teacher forcing; chunk-wise teacher forcing
# (7 chunks of 3 frames); wide-head frame-wise teacher forcing.
WORKLOADS = {
    1: Workload("tf_framewise_tiny_fp32", 1, 1, 2, 64, 16, 3, 1, 1, "fp32", 0.1, False),
    2: Workload("blockcausal_framewise_32760", 2, 1, 12, 128, 1560, 21, 1, 0, "bf16", 0.1, True),
    3: Workload("tf_framewise_65520", 3, 1, 12, 128, 1560, 21, 1, 1, "bf16", 0.1, True),
    4: Workload("tf_chunkwise_65520_b2", 4, 2, 12, 128, 1560, 21, 3, 1, "bf16", 0.1, True),
    5: Workload("tf_framewise_65520_h40", 5, 1, 40, 128, 1560, 21, 1, 1, "bf16", 0.05, True),
}


# Workloads whose mask is given as a range list: frame-wise teacher forcing
# with a one-frame first chunk followed by four-frame chunks (c1-4, 21 frames).
RANGE_WORKLOADS = {
    6: Workload("tf_c1_4_65520", 6, 1, 12, 128, 1560, 21, 1, 1, "bf16", 0.1, True, (1, 4, 4, 4, 4, 4)),
}


def chunked_mask_ranges(tokens_per_frame: int, chunk_frames, tf_layout: int):
    """Structure of a chunked teacher-forcing / block-causal mask as query
    groups x key intervals: one group per chunk and side.  Clean chunk c sees
    the clean tokens of chunks 0..c; noisy chunk c sees the clean tokens of
    chunks 0..c-1 and its own noisy tokens (section 3.1.1); a block-causal
    mask is the clean side alone.  Returns (seq_len, groups) with groups =
    ((row_lo, row_hi, ((key_lo, key_hi), ...)), ...), half-open."""
    lens = [tokens_per_frame * int(c) for c in chunk_frames]
    nh = sum(lens)
    groups = []
    start = 0
    for t in lens:
        groups.append((start, start + t, ((0, start + t),)))
        start += t
    if tf_layout:
        start = 0
        for t in lens:
            own = (nh + start, nh + start + t)
            groups.append((own[0], own[1], (((0, start), own) if start > 0 else (own,))))
            start += t
    return nh * (2 if tf_layout else 1), tuple(groups)


def und_gen_ranges(n_und: int, n_frames: int, tokens_per_frame: int):
    """Structure of an understanding / generation layout [UND | GEN] as query
    groups x key intervals (section 4.2.2, Figure 9): UND tokens attend
    causally (one group per UND token); a GEN token of frame f attends to
    every UND token and to the GEN tokens of frames 0..f (one group per
    frame).  Returns (seq_len, groups)."""
    groups = [(i, i + 1, ((0, i + 1),)) for i in range(n_und)]
    for f in range(n_frames):
        lo = n_und + f * tokens_per_frame
        groups.append((lo, lo + tokens_per_frame, ((0, lo + tokens_per_frame),)))
    return n_und + n_frames * tokens_per_frame, tuple(groups)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.

    NaN inputs are not expected in synthetic data and are not special-cased.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_float32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stream(w: Workload, tensor_id: int, b: int, h: int) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, w.cfg_id, tensor_id, b, h])
    return np.random.Generator(np.random.PCG64(ss))


def slice_f32(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One (b, h) slice [N, d] as float32, before any bf16 rounding."""
    tid = _TENSOR_IDS[tensor]
    x = _stream(w, tid, b, h).standard_normal((w.seq_len, w.head_dim), dtype=np.float32)
    if tensor in ("q", "k") and w.rms_norm_qk:
        ms = np.mean(x * x, axis=1, keepdims=True, dtype=np.float32)
        x = x / np.sqrt(ms + np.float32(1e-6))
    if tensor in ("tq", "tk", "tv"):
        x = x * np.float32(w.tangent_std)
    return x.astype(np.float32, copy=False)


def slice_values(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One (b, h) slice as the exact values the kernel sees, in float64."""
    x = slice_f32(w, tensor, b, h)
    if w.dtype == "bf16":
        x = bf16_bits_to_float32(round_to_bf16_bits(x))
    return x.astype(np.float64)


def slice_device_bits(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One (b, h) slice in the device storage format: uint16 bf16 bits or float32."""
    x = slice_f32(w, tensor, b, h)
    return round_to_bf16_bits(x) if w.dtype == "bf16" else x


def full_tensor_bits(w: Workload, tensor: str, workers: int | None = None) -> np.ndarray:
    """The whole [B, H, N, d] tensor in device storage format (uint16 or float32)."""
    out = np.empty(w.shape, dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    jobs = [(b, h) for b in range(w.batch) for h in range(w.heads)]

    def fill(bh):
        b, h = bh
        out[b, h] = slice_device_bits(w, tensor, b, h)

    n = workers or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        list(ex.map(fill, jobs))
    return out


def full_values(w: Workload, tensor: str) -> np.ndarray:
    """The whole tensor as float64 values (small workloads only)."""
    out = np.empty(w.shape, dtype=np.float64)
    for b in range(w.batch):
        for h in range(w.heads):
            out[b, h] = slice_values(w, tensor, b, h)
    return out
