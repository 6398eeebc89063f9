"""fp64 CPU oracle for packed native-resolution joint attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module. The library (``packed_attention_nr_amd``) never imports it
and this module imports nothing from the library: the two share no code.

What it computes is the plain definition of one NR-MMDiT attention core, as the
Mage-Flow pages describe it:

* packing: every sample's text tokens and flattened latent-grid tokens sit back
  to back in one contiguous batch, with per-sample cumulative offsets
  (findtube.ai transcript "Mage-Flow: Efficient Native-Resolution Image
  Generation and Editing" at [00:03:16] and [00:04:03]; picx.dev summary
  "Mage-Flow: An Efficient Native-Resolution Foundation Model ...", section
  "Native-Resolution MMDiT (NR-MMDiT)", bullet "Native-resolution packing");
* modality-specific normalisation of the joint-attention inputs (picx.dev,
  section "Native-Resolution MMDiT (NR-MMDiT)", first bullet; transcript at
  [00:00:00]), taken here as RMSNorm of Q and K per head with one gain vector
  per (Q or K, text or image);
* a per-sample 2D rotary embedding of image tokens by their own (row, col)
  (transcript at [00:03:16]; aiany.app entry, "Key Capabilities");
* for editing, the source image's latents joined to the target latents in
  the same sample and told apart by the frame dimension of a 3D rotary
  embedding (picx.dev, section "Native-Resolution MMDiT (NR-MMDiT)",
  conditioning bullet);
* joint text+image self-attention restricted to each sample, i.e. block
  diagonal over the cumulative offsets (picx.dev, same section: FlashAttention
  with per-sample cumulative offsets).

The method (variable-length flash attention) reaches exactly this definition up
to rounding, so the oracle is the definition written out in float64 with
numpy; matrix products use numpy's BLAS matmul. Readings taken where the pages
are silent:

* token order inside a sample: text first, then the image grid row-major;
* RMSNorm: over the d elements of one (token, head); eps inside the square
  root, added to the mean square; gain applied after normalisation; no bias;
  V is not normalised;
* order: RMSNorm, then gain, then RoPE;
* RoPE: the first d/2 dimensions rotate by the row index and the last d/2 by
  the column index, 0-based; inside each half, adjacent pairs (2j, 2j+1)
  rotate by angle pos * theta^(-4j/d), j < d/4; text tokens are not rotated;
* editing packs: a sample's source grid follows its target grid (text,
  target, source), the target on frame 0 and the source on frame 1; every
  image token of such a pack turns by three axes, the first d/8 pairs by the
  frame, the next 3d/16 by the row and the last 3d/16 by the column; pair j of
  a section of n pairs turns by pos * theta^(-j/n) (which for n = d/4 is the
  2D rule);
* softmax scale 1/sqrt(d), no causal mask, no dropout, natural-log lse;
* the adaptive-LayerNorm modulation and gated residual around the attention
  (see ``adaln_forward``).

Parity status of each function (how it is pinned by tests other than itself):
``layout`` (pure-Python enumeration, token counts, editing order),
``rms_norm`` (closed forms), ``rope_apply`` (hand values at d=4 and d=8,
norm preservation, relative-position property), ``rope_angles`` (hand
values of the 2D and 3D schedules, 3D relative-position property, frame-0
tokens unrotated on the frame pairs), ``attention_forward`` (pure-Python brute force,
torch fp64 library attention, closed forms, packing invariants),
``attention_backward`` / ``rope_backward`` / ``rms_norm_backward``
(central finite differences, torch fp64 autograd, closed forms),
``adaln_forward`` (hand values, torch fp64 ``layer_norm``, per-sample and
per-stream selection), ``adaln_backward`` (central finite differences, torch
fp64 autograd, closed forms).
The RoPE pair layout, frequency schedule, position origin and the 3D split
themselves are readings, not statements of the pages: against the pages they are parity
unpinned; the code is pinned only against that written reading.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Layout", "layout", "rope_frequencies", "rope_section_frequencies", "rope_sections",
    "rope_angles", "rope_apply",
    "rope_backward", "rms_norm", "rms_norm_backward", "token_gains",
    "prologue", "attention_forward", "attention_backward", "forward",
    "backward", "modulation_index", "adaln_forward", "adaln_backward",
]

QUERY_BLOCK = 2048  # rows of the score matrix formed at once (memory bound only)


# --------------------------------------------------------------------------
# Packing layout
# --------------------------------------------------------------------------
@dataclass
class Layout:
    cu_seqlens: np.ndarray   # int64 [S+1], cu[0] = 0, cu[S] = N
    segment: np.ndarray      # int64 [N], sample index of each token
    is_image: np.ndarray     # bool  [N]
    row: np.ndarray          # int64 [N], 0 for text tokens
    col: np.ndarray          # int64 [N], 0 for text tokens
    frame: Optional[np.ndarray] = None  # int64 [N]: 1 for source-image tokens, else 0
    three_axes: bool = False            # editing pack: RoPE over (frame, row, col)

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def layout(text_len: Sequence[int], grid_h: Sequence[int], grid_w: Sequence[int],
           src_h: Optional[Sequence[int]] = None, src_w: Optional[Sequence[int]] = None) -> Layout:
    """Packing of samples into one contiguous token batch.

    Sample i occupies tokens cu[i] .. cu[i+1]-1 where cu[i+1] = cu[i] + T_i + h_i*w_i:
    first its T_i text tokens, then its h_i x w_i latent grid flattened row-major,
    the grid token at (r, c) being token cu[i] + T_i + r*w_i + c.
    (picx.dev, "Native-Resolution MMDiT (NR-MMDiT)": each image becomes a
    variable-length token sequence by flattening and is packed together with
    its text under cumulative offsets; transcript [00:03:16]: all samples share
    one contiguous batch.)

    With src_h, src_w (an editing pack; picx.dev, same section, conditioning
    bullet: the source latents are concatenated with the target latents), the
    sample's sh_i x sw_i source grid follows its target grid, row-major, with
    frame index 1; the target grid keeps frame 0, and the pack's RoPE runs over
    three axes.
    """
    T = np.asarray(text_len, dtype=np.int64)
    h = np.asarray(grid_h, dtype=np.int64)
    w = np.asarray(grid_w, dtype=np.int64)
    edit = src_h is not None
    sh = np.asarray(src_h if edit else np.zeros_like(h), dtype=np.int64)
    sw = np.asarray(src_w if edit else np.zeros_like(h), dtype=np.int64)
    L = T + h * w + sh * sw
    cu = np.zeros(len(L) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(L)
    N = int(cu[-1])
    segment = np.zeros(N, dtype=np.int64)
    is_image = np.zeros(N, dtype=bool)
    row = np.zeros(N, dtype=np.int64)
    col = np.zeros(N, dtype=np.int64)
    frame = np.zeros(N, dtype=np.int64)
    for i in range(len(L)):
        segment[cu[i]:cu[i + 1]] = i
        start = cu[i] + T[i]
        for f, (gh, gw) in enumerate(((h[i], w[i]), (sh[i], sw[i]))):
            n_img = int(gh * gw)
            if n_img:
                idx = start + np.arange(n_img)
                is_image[idx] = True
                row[idx] = np.arange(n_img) // gw
                col[idx] = np.arange(n_img) % gw
                frame[idx] = f
                start += n_img
    return Layout(cu, segment, is_image, row, col, frame, edit)


# --------------------------------------------------------------------------
# 2D rotary embedding (image tokens only)
# --------------------------------------------------------------------------
def rope_section_frequencies(n: int, theta: float = 10000.0) -> np.ndarray:
    """omega_j = theta^(-j/n) for the n pairs of one axis: a 1D rotary
    embedding of 2n dimensions (frequencies theta^(-2j/(2n)))."""
    return np.power(float(theta), -np.arange(n, dtype=np.float64) / n)


def rope_frequencies(d: int, theta: float = 10000.0) -> np.ndarray:
    """2D: omega_j = theta^(-4j/d) for j < d/4, each half of the head dimension
    being a 1D rotary embedding of size d/2."""
    if d % 4:
        raise ValueError("head_dim must be a multiple of 4 for 2D RoPE")
    return rope_section_frequencies(d // 4, theta)


def rope_sections(d: int, three_axes: bool = False):
    """The axes of the d/2 dimension pairs, in pair order, as (axis, count):
    2D: row on d/4 pairs, then column on d/4; 3D (editing): frame on d/8,
    row on 3d/16, column on 3d/16."""
    if not three_axes:
        return [("row", d // 4), ("col", d // 4)]
    if d % 16:
        raise ValueError("head_dim must be a multiple of 16 for 3D RoPE")
    return [("frame", d // 8), ("row", 3 * d // 16), ("col", 3 * d // 16)]


def rope_angles(lay: Layout, d: int, theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of each of the d/2 dimension pairs of each token, [N, d/2].

    The pairs are split into consecutive sections, one per axis
    (``rope_sections``); pair j of a section of n pairs turns by
    pos * theta^(-j/n), pos the token's index on that axis. 2D: pair p < d/4
    (dimensions 2p, 2p+1) turns by row * theta^(-4p/d) and pair d/4 + j by
    col * theta^(-4j/d). Text tokens get angle 0, i.e. no rotation.
    (Transcript [00:03:16]: per-sample 2D rotary positional embeddings keeping
    each sample's own pixel layout; picx.dev, "Native-Resolution MMDiT
    (NR-MMDiT)", conditioning bullet: a third, frame axis for editing.)
    """
    frame = lay.frame if lay.frame is not None else np.zeros_like(lay.row)
    pos = {"frame": frame, "row": lay.row, "col": lay.col}
    parts = []
    for axis, n in rope_sections(d, lay.three_axes):
        om = rope_section_frequencies(n, theta)
        x = np.where(lay.is_image, pos[axis], 0).astype(np.float64)
        parts.append(x[:, None] * om[None, :])
    return np.concatenate(parts, axis=1)


def rope_apply(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each pair (x[2p], x[2p+1]) of every head by angles[t, p]:
    (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi). x is [N, H, d]."""
    cos = np.cos(angles)[:, None, :]
    sin = np.sin(angles)[:, None, :]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def rope_backward(dy: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Gradient through ``rope_apply``: the transpose of a rotation, i.e. the
    rotation by -phi applied to the incoming gradient."""
    return rope_apply(dy, -angles)


# --------------------------------------------------------------------------
# Per-modality RMSNorm of Q and K
# --------------------------------------------------------------------------
def token_gains(gains: np.ndarray, lay: Layout, which: str) -> np.ndarray:
    """Per-token gain vector [N, d] from the four gain rows
    (0 q_text, 1 q_image, 2 k_text, 3 k_image)."""
    g = np.asarray(gains, dtype=np.float64)
    base = 0 if which == "q" else 2
    return np.where(lay.is_image[:, None], g[base + 1][None, :], g[base][None, :])


def rms_norm(x: np.ndarray, g_tok: np.ndarray, eps: float):
    """y = x * rho * g with rho = (mean over the d elements of x^2 + eps)^(-1/2),
    per (token, head). Returns (y, rho) with rho of shape [N, H]."""
    ms = np.mean(x * x, axis=-1)
    rho = 1.0 / np.sqrt(ms + eps)
    return x * rho[..., None] * g_tok[:, None, :], rho


def rms_norm_backward(x: np.ndarray, g_tok: np.ndarray, rho: np.ndarray, dy: np.ndarray):
    """Gradients of y = x * rho(x) * g.

    dx = rho * g * dy - (rho^3 / d) * x * sum_k g_k dy_k x_k
    dg (per token and head) = dy * x * rho, left unsummed: [N, H, d].
    """
    d = x.shape[-1]
    gdy = g_tok[:, None, :] * dy
    dot = np.sum(gdy * x, axis=-1)
    dx = rho[..., None] * gdy - (rho ** 3 / d)[..., None] * x * dot[..., None]
    dg = dy * x * rho[..., None]
    return dx, dg


def prologue(q, k, gains, lay: Layout, eps: float = 1e-6, theta: float = 10000.0):
    """Q-hat and K-hat: RMSNorm with the modality's gain, then 2D RoPE."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    ang = rope_angles(lay, d, theta)
    yq, rq = rms_norm(q, token_gains(gains, lay, "q"), eps)
    yk, rk = rms_norm(k, token_gains(gains, lay, "k"), eps)
    return rope_apply(yq, ang), rope_apply(yk, ang), rq, rk


# --------------------------------------------------------------------------
# Block-diagonal joint attention
# --------------------------------------------------------------------------
def _heads_first(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).transpose(1, 0, 2))


def attention_forward(qh, kh, v, cu_seqlens, q_block: int = QUERY_BLOCK):
    """Per sample i and head h: O = softmax(Q_i K_i^T / sqrt(d)) V_i over that
    sample's tokens only (text and image jointly, no mask inside a sample), and
    lse = ln sum_j exp(S_tj). Returns O [N, H, d] and lse [N, H]."""
    Q, K, V = _heads_first(qh), _heads_first(kh), _heads_first(v)
    H, N, d = Q.shape
    scale = 1.0 / np.sqrt(d)
    O = np.zeros((H, N, d))
    lse = np.zeros((H, N))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for h in range(H):
            Kh, Vh = K[h, a:b], V[h, a:b]
            for q0 in range(a, b, q_block):
                q1 = min(q0 + q_block, b)
                s = (Q[h, q0:q1] @ Kh.T) * scale
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                O[h, q0:q1] = (p @ Vh) / l
                lse[h, q0:q1] = (m + np.log(l))[:, 0]
    return O.transpose(1, 0, 2).copy(), lse.T.copy()


def attention_backward(qh, kh, v, dout, cu_seqlens, q_block: int = QUERY_BLOCK):
    """Gradients of sum(dO * O) for the attention above, per sample and head:
    P = softmax(S), S = Q K^T / sqrt(d);  dV = P^T dO;  dP = dO V^T;
    dS = P * (dP - rowsum(P * dP));  dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
    Returns dQ-hat, dK-hat, dV, each [N, H, d]."""
    Q, K, V, dO = (_heads_first(t) for t in (qh, kh, v, dout))
    H, N, d = Q.shape
    scale = 1.0 / np.sqrt(d)
    dQ = np.zeros((H, N, d))
    dK = np.zeros((H, N, d))
    dV = np.zeros((H, N, d))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for h in range(H):
            Kh, Vh = K[h, a:b], V[h, a:b]
            for q0 in range(a, b, q_block):
                q1 = min(q0 + q_block, b)
                Qb, dOb = Q[h, q0:q1], dO[h, q0:q1]
                s = (Qb @ Kh.T) * scale
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dV[h, a:b] += p.T @ dOb
                dp = dOb @ Vh.T
                ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
                dQ[h, q0:q1] = (ds @ Kh) * scale
                dK[h, a:b] += (ds.T @ Qb) * scale
    back = lambda t: t.transpose(1, 0, 2).copy()
    return back(dQ), back(dK), back(dV)


# --------------------------------------------------------------------------
# Whole forward / backward of the attention core
# --------------------------------------------------------------------------
def forward(text_len, grid_h, grid_w, q, k, v, gains, eps=1e-6, theta=10000.0,
            lay: Optional[Layout] = None):
    """Pre-norm Q, K, V [N, H, d] -> dict with q_hat, k_hat, rstd_q, rstd_k,
    o [N, H, d] and lse [N, H] (all float64)."""
    if lay is None:
        lay = layout(text_len, grid_h, grid_w)
    qh, kh, rq, rk = prologue(q, k, gains, lay, eps, theta)
    o, lse = attention_forward(qh, kh, v, lay.cu_seqlens)
    return dict(layout=lay, q_hat=qh, k_hat=kh, rstd_q=rq, rstd_k=rk, o=o, lse=lse)


def backward(text_len, grid_h, grid_w, q, k, v, gains, dout, eps=1e-6,
             theta=10000.0, lay: Optional[Layout] = None):
    """Gradients of sum(dout * O) with respect to the pre-norm q, k, v and the
    four gain rows. Returns dict with dq, dk, dv [N, H, d], dgains [4, d], and
    the intermediate dq_hat, dk_hat."""
    if lay is None:
        lay = layout(text_len, grid_h, grid_w)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[-1]
    ang = rope_angles(lay, d, theta)
    gq, gk = token_gains(gains, lay, "q"), token_gains(gains, lay, "k")
    yq, rq = rms_norm(q, gq, eps)
    yk, rk = rms_norm(k, gk, eps)
    qh, kh = rope_apply(yq, ang), rope_apply(yk, ang)
    dqh, dkh, dv = attention_backward(qh, kh, v, dout, lay.cu_seqlens)
    dq, dgq = rms_norm_backward(q, gq, rq, rope_backward(dqh, ang))
    dk, dgk = rms_norm_backward(k, gk, rk, rope_backward(dkh, ang))
    img = lay.is_image
    dgains = np.stack([
        dgq[~img].sum(axis=(0, 1)), dgq[img].sum(axis=(0, 1)),
        dgk[~img].sum(axis=(0, 1)), dgk[img].sum(axis=(0, 1)),
    ])
    return dict(dq=dq, dk=dk, dv=dv, dgains=dgains, dq_hat=dqh, dk_hat=dkh)


# --------------------------------------------------------------------------
# Adaptive LayerNorm modulation and gated residual (the memory-bound chains
# on either side of the attention core)
# --------------------------------------------------------------------------
# picx.dev, section "Training Infrastructure": adaptive normalisation and
# gating of the NR-MMDiT are fused into custom kernels; transcript [00:04:20]:
# normalisation and residual chains fused so that intermediates stay on chip.
# The pages give no formula. Readings:
# * the DiT/MMDiT adaLN: LayerNorm over the model width D without affine
#   parameters, eps inside the root, then h = x_hat * (1 + scale) + shift;
# * one (shift, scale, gate) per sample and per stream (text or image): the
#   modulation comes from each sample's own conditioning, and MMDiT keeps
#   separate parameters per modality; all image tokens of a sample (an editing
#   sample's target and source alike) use the image stream's;
# * gated residual: z = x + gate * y, y being the output projection of the
#   attention; the LayerNorm that follows is fused, so the op's outputs are
#   z and h = adaLN(z). Without y the op is the plain adaLN of x (z = x).
def modulation_index(lay: Layout) -> np.ndarray:
    """Row of the [S, 2] modulation table of each token: (sample, stream),
    stream 0 text and 1 image, flattened to 2 * sample + stream."""
    return 2 * lay.segment + lay.is_image.astype(np.int64)


def _per_token(table: np.ndarray, lay: Layout) -> np.ndarray:
    t = np.asarray(table, dtype=np.float64)
    return t.reshape(-1, t.shape[-1])[modulation_index(lay)]


def _segment_sum(vals: np.ndarray, lay: Layout, S: int) -> np.ndarray:
    """Sum of the rows of vals [N, D] over each (sample, stream): [S, 2, D]."""
    out = np.zeros((2 * S, vals.shape[-1]))
    np.add.at(out, modulation_index(lay), vals)
    return out.reshape(S, 2, -1)


def adaln_forward(lay: Layout, x, shift, scale, eps: float = 1e-6, y=None, gate=None):
    """z = x (+ gate * y); mu, var = mean and biased variance of z over its D
    elements; rstd = (var + eps)^(-1/2); h = (z - mu) * rstd * (1 + scale) +
    shift. x, y: [N, D]; shift, scale, gate: [S, 2, D]. Returns dict with z,
    h, mean and rstd (float64)."""
    z = np.asarray(x, dtype=np.float64)
    if y is not None:
        z = z + _per_token(gate, lay) * np.asarray(y, dtype=np.float64)
    mu = np.mean(z, axis=-1)
    var = np.mean((z - mu[:, None]) ** 2, axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    zh = (z - mu[:, None]) * rstd[:, None]
    h = zh * (1.0 + _per_token(scale, lay)) + _per_token(shift, lay)
    return dict(z=z, h=h, mean=mu, rstd=rstd)


def adaln_backward(lay: Layout, x, shift, scale, dh, eps: float = 1e-6, y=None, gate=None,
                   dz=None):
    """Gradients of sum(dh * h) + sum(dz * z) for ``adaln_forward``.

    g = dh * (1 + scale); dz_total = dz + rstd * (g - mean(g) - z_hat * mean(g * z_hat)),
    the means over the D elements of a row; dx = dz_total; dy = gate * dz_total;
    dshift, dscale, dgate [S, 2, D] = sums over each (sample, stream) of dh,
    dh * z_hat and dz_total * y."""
    S = len(lay.cu_seqlens) - 1
    f = adaln_forward(lay, x, shift, scale, eps, y, gate)
    dh = np.asarray(dh, dtype=np.float64)
    zh = (f["z"] - f["mean"][:, None]) * f["rstd"][:, None]
    g = dh * (1.0 + _per_token(scale, lay))
    dzt = f["rstd"][:, None] * (g - np.mean(g, -1, keepdims=True)
                                - zh * np.mean(g * zh, -1, keepdims=True))
    if dz is not None:
        dzt = dzt + np.asarray(dz, dtype=np.float64)
    out = dict(dx=dzt, dshift=_segment_sum(dh, lay, S), dscale=_segment_sum(dh * zh, lay, S))
    if y is not None:
        out["dy"] = _per_token(gate, lay) * dzt
        out["dgate"] = _segment_sum(dzt * np.asarray(y, dtype=np.float64), lay, S)
    return out
