"""Seeded synthetic inputs for the packed joint-attention path.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and describes pack geometry (text length and latent grid
per sample). It holds none of the method's arithmetic: no normalisation, no
rotary embedding, no attention. Both the fp64 CPU oracle and the HIP path are
fed the arrays produced here.

Geometry follows the Mage-Flow pages (picx.dev summary, section "Native-Resolution
MMDiT"; the findtube.ai transcript at [00:03:16]-[00:04:03]): each sample is a
text segment followed by a flattened image-latent grid of its own height and
width, 16 pixels per latent token (picx.dev, section "Mage-VAE"), resolutions
512-2048 and aspect ratios up to 4:1.

Draw order for every workload (one ``numpy.random.default_rng(seed)`` stream):
  1. text lengths, ``rng.integers(lo, hi + 1, S)`` (only where they are random);
  2. gains ``1 + 0.1 * N(0,1)`` of shape [4, d], rows q_text, q_image, k_text, k_image;
  3. Q, K, V, each ``rng.standard_normal((N, H, d), dtype=float32)``;
  4. dO, the same way (only for workloads with a backward pass).
bf16 workloads round every tensor to bf16 with round-to-nearest-even; the oracle
receives exactly those rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "draw", "bf16_round", "bf16_bits",
    "random_pack", "Inputs", "draw_adaln", "geometry",
]


@dataclass(frozen=True)
class Workload:
    name: str
    title: str
    grids: Tuple[Tuple[int, int], ...]          # (h, w) per sample; (0, 0) = no image
    text: Optional[Tuple[int, ...]]             # fixed text lengths, or None = drawn
    text_range: Optional[Tuple[int, int]]       # inclusive range when drawn
    heads: int
    head_dim: int
    dtype: str                                  # "f32" or "bf16"
    backward: bool
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    src: Optional[Tuple[Tuple[int, int], ...]] = None   # editing: source grid per sample


def _rep(x, n):
    return tuple([x] * n)


WORKLOADS = {
    # Tiny two-sample pack, fp32, forward only.
    "tiny_fp32": Workload(
        "tiny_fp32", "tiny 2-sample pack, fp32 (440 tokens, H=4, d=64)",
        grids=((16, 16), (16, 8)), text=(32, 24), text_range=None,
        heads=4, head_dim=64, dtype="f32", backward=False),
    # One 1024x1024 generation step: 512 text + 64x64 latents.
    "gen1024": Workload(
        "gen1024", "1024^2 generation step, bf16 (512 text + 64x64 grid = 4,608 tokens, H=24, d=128)",
        grids=((64, 64),), text=(512,), text_range=None,
        heads=24, head_dim=128, dtype="bf16", backward=False),
    # Mixed-resolution packed training batch: six grids, text drawn from 64..512.
    "mixed6": Workload(
        "mixed6", "mixed-resolution packed training batch, bf16 (6 samples, 20,436 tokens, H=24, d=128)",
        grids=((32, 32), (48, 84), (64, 64), (32, 128), (84, 48), (40, 40)),
        text=None, text_range=(64, 512),
        heads=24, head_dim=128, dtype="bf16", backward=True),
    # One 2048x2048 sample: 512 text + 128x128 latents.
    "gen2048": Workload(
        "gen2048", "2048^2 single sample, bf16 (512 text + 128x128 grid = 16,896 tokens, H=24, d=128)",
        grids=((128, 128),), text=(512,), text_range=None,
        heads=24, head_dim=128, dtype="bf16", backward=True),
    # 64 small samples: 32x32 grids, text drawn from 32..256.
    "small64": Workload(
        "small64", "many-small-segments pack, bf16 (64 x (32x32 + text 32..256), 74,894 tokens, H=24, d=128)",
        grids=_rep((32, 32), 64), text=None, text_range=(32, 256),
        heads=24, head_dim=128, dtype="bf16", backward=True),
    # One 1024x1024 editing step: 512 text + 64x64 target latents + 64x64
    # source latents on a second RoPE frame.
    "edit1024": Workload(
        "edit1024", "1024^2 editing step, bf16 (512 text + 64x64 target + 64x64 source = 8,704 tokens, "
        "H=24, d=128)",
        grids=((64, 64),), text=(512,), text_range=None,
        heads=24, head_dim=128, dtype="bf16", backward=True, src=((64, 64),)),
}

# The workloads in their canonical order.
ORDER = ["tiny_fp32", "gen1024", "mixed6", "gen2048", "small64", "edit1024"]


def get(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the
    raw 16-bit patterns as uint16. Inputs are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    bias = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + bias) >> 16).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 value (RNE), returned as fp32."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """One seeded draw. Floating tensors are fp32 arrays holding exactly the
    values the device receives (already bf16-rounded for bf16 workloads)."""
    text_len: np.ndarray      # int32 [S]
    grid_h: np.ndarray        # int32 [S]
    grid_w: np.ndarray        # int32 [S]
    gains: np.ndarray         # fp32 [4, d]: q_text, q_image, k_text, k_image
    q: np.ndarray             # fp32 [N, H, d]
    k: np.ndarray
    v: np.ndarray
    dout: Optional[np.ndarray]
    heads: int
    head_dim: int
    dtype: str
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    src_h: Optional[np.ndarray] = None   # int32 [S]: source grids of an editing pack
    src_w: Optional[np.ndarray] = None

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def edit(self) -> bool:
        return self.src_h is not None

    def seqlens(self) -> np.ndarray:
        L = (self.text_len.astype(np.int64)
             + self.grid_h.astype(np.int64) * self.grid_w.astype(np.int64))
        if self.edit:
            L = L + self.src_h.astype(np.int64) * self.src_w.astype(np.int64)
        return L


def _finish(rng, text, hs, ws, H, d, dtype, backward, theta, eps, src=None) -> Inputs:
    text = np.asarray(text, dtype=np.int32)
    hs = np.asarray(hs, dtype=np.int32)
    ws = np.asarray(ws, dtype=np.int32)
    N = int((text.astype(np.int64) + hs.astype(np.int64) * ws.astype(np.int64)).sum())
    sh = sw = None
    if src is not None:
        sh = np.asarray([g[0] for g in src], dtype=np.int32)
        sw = np.asarray([g[1] for g in src], dtype=np.int32)
        N += int((sh.astype(np.int64) * sw.astype(np.int64)).sum())
    gains = (1.0 + 0.1 * rng.standard_normal((4, d))).astype(np.float32)
    tens = []
    for _ in range(4 if backward else 3):
        tens.append(rng.standard_normal((N, H, d), dtype=np.float32))
    if dtype == "bf16":
        tens = [bf16_round(t) for t in tens]
    q, k, v = tens[:3]
    dout = tens[3] if backward else None
    return Inputs(text, hs, ws, gains, q, k, v, dout, H, d, dtype, theta, eps, sh, sw)


def draw(w: Workload | str, seed: int = 0, backward: Optional[bool] = None) -> Inputs:
    """Draw the inputs of a named workload (seed 0 unless told otherwise)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    S = len(w.grids)
    if w.text is None:
        lo, hi = w.text_range
        text = rng.integers(lo, hi + 1, S)
    else:
        text = np.asarray(w.text)
    hs = [g[0] for g in w.grids]
    ws = [g[1] for g in w.grids]
    bw = w.backward if backward is None else backward
    return _finish(rng, text, hs, ws, w.heads, w.head_dim, w.dtype, bw,
                   w.rope_theta, w.rms_eps, w.src)


def geometry(w: Workload | str, seed: int = 0):
    """Pack geometry of a named workload without drawing its tensors: (text
    lengths, grids, source grids or None), the text lengths being the first
    draw of ``draw``'s stream (so they equal the ones ``draw`` makes)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.text is None:
        lo, hi = w.text_range
        text = np.random.default_rng(seed).integers(lo, hi + 1, len(w.grids))
    else:
        text = np.asarray(w.text)
    return [int(t) for t in text], list(w.grids), None if w.src is None else list(w.src)


def draw_adaln(seed: int, num_tokens: int, num_samples: int, dim: int, dtype: str = "bf16",
               residual: bool = True) -> dict:
    """Inputs of the adaLN modulation / gated residual op for a pack of
    num_tokens tokens and num_samples samples at model width dim, from one
    ``default_rng(seed)`` stream in this order: per-row offsets N(0,1) and
    scales U(0.5, 2) of x, then x, y, dh, dz ~ N(0,1) [N, dim] (x scaled and
    offset per row), then shift, scale ~ 0.3 N(0,1) and gate ~ N(0,1)
    [S, 2, dim]. Token tensors are rounded to bf16 for bf16 packs; the
    modulation tables stay fp32."""
    rng = np.random.default_rng(seed)
    N, S, D = num_tokens, num_samples, dim
    off = rng.standard_normal((N, 1)).astype(np.float32)
    sc = rng.uniform(0.5, 2.0, (N, 1)).astype(np.float32)
    t = lambda: rng.standard_normal((N, D), dtype=np.float32)
    x = t() * sc + off
    y, dh, dz = t(), t(), t()
    if dtype == "bf16":
        x, y, dh, dz = (bf16_round(a) for a in (x, y, dh, dz))
    m = lambda k: (k * rng.standard_normal((S, 2, D))).astype(np.float32)
    out = dict(x=x, dh=dh, dz=dz, shift=m(0.3), scale=m(0.3))
    gate = m(1.0)
    if residual:
        out.update(y=y, gate=gate)
    return out


def random_pack(seed: int, *, max_samples: int = 4, max_text: int = 40,
                max_side: int = 9, heads: int = 2, head_dim: int = 64,
                dtype: str = "f32", backward: bool = True,
                allow_empty_text: bool = True, allow_empty_image: bool = True,
                text: Optional[Sequence[int]] = None,
                grids: Optional[Sequence[Tuple[int, int]]] = None,
                edit: bool = False,
                src: Optional[Sequence[Tuple[int, int]]] = None) -> Inputs:
    """A small random pack for property tests: random sample count, text
    lengths and grids (each sample keeps at least one token). ``text`` and
    ``grids`` override the random geometry. ``edit`` makes an editing pack:
    each sample with a target grid gets a source grid (a fifth of them none,
    i.e. generation samples in the editing pack), drawn after everything
    else; ``src`` gives the source grids instead."""
    rng = np.random.default_rng(seed)
    if text is None or grids is None:
        S = int(rng.integers(1, max_samples + 1))
        t_lo = 0 if allow_empty_text else 1
        tl, hs, ws = [], [], []
        for _ in range(S):
            t = int(rng.integers(t_lo, max_text + 1))
            if allow_empty_image and rng.random() < 0.2:
                h = w = 0
            else:
                h = int(rng.integers(1, max_side + 1))
                w = int(rng.integers(1, max_side + 1))
            if t + h * w == 0:
                t = 1
            tl.append(t); hs.append(h); ws.append(w)
    else:
        tl = list(text)
        hs = [g[0] for g in grids]
        ws = [g[1] for g in grids]
    if edit and src is None:
        src = []
        for h in hs:
            if h == 0 or rng.random() < 0.2:
                src.append((0, 0))
            else:
                src.append((int(rng.integers(1, max_side + 1)), int(rng.integers(1, max_side + 1))))
    return _finish(rng, tl, hs, ws, heads, head_dim, dtype, backward, 10000.0, 1e-6, src)
