"""Pins of the fp64 oracle against things other than itself (CPU only).

Every ``pin_*`` function below checks one part of ``oracle`` against a hand
fixture under tests/golden/, a closed form, an invariant the pages state, a
pure-Python brute force on tiny inputs, a torch fp64 library routine, or
central finite differences. ``test_mutants_are_caught`` plants plausible
mistakes in the oracle (monkeypatched, on the CPU) and checks that at least one
pin fails for each.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.oracle as om
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers that do not use the oracle's arithmetic
# --------------------------------------------------------------------------
def _enumerate_tokens(text, hs, ws):
    """Pure-Python token list: (segment, is_image, row, col)."""
    toks = []
    for s, (t, h, w) in enumerate(zip(text, hs, ws)):
        for _ in range(t):
            toks.append((s, False, 0, 0))
        for r in range(h):
            for c in range(w):
                toks.append((s, True, r, c))
    return toks


def _enumerate_tokens_edit(text, hs, ws, sh, sw):
    """Pure-Python token list of an editing pack: (segment, is_image, row,
    col, frame); per sample its text, the target grid on frame 0, then the
    source grid on frame 1."""
    toks = []
    for s in range(len(text)):
        toks += [(s, False, 0, 0, 0)] * int(text[s])
        for f, (h, w) in enumerate(((hs[s], ws[s]), (sh[s], sw[s]))):
            for r in range(h):
                for c in range(w):
                    toks.append((s, True, r, c, f))
    return toks


def _brute_attention(qh, kh, v, seg):
    """Pure-Python loops: O[t] = sum_j softmax_j(q_t.k_j/sqrt d) v_j over the
    tokens j of t's own sample."""
    N, H, d = qh.shape
    O = np.zeros((N, H, d))
    lse = np.zeros((N, H))
    for h in range(H):
        for t in range(N):
            js = [j for j in range(N) if seg[j] == seg[t]]
            s = [sum(qh[t, h, x] * kh[j, h, x] for x in range(d)) / math.sqrt(d) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for x in range(d):
                O[t, h, x] = sum(e[i] * v[js[i], h, x] for i in range(len(js))) / z
            lse[t, h] = m + math.log(z)
    return O, lse


def _torch_reference(inp, lay_seg, is_img, row, col, theta=10000.0):
    """Torch fp64 forward (RMSNorm per modality, RoPE from cos/sin of the fixture
    angles, library attention with a block-diagonal mask) for autograd and
    library cross-checks. Returns a function of (q, k, v, gains) -> O."""
    d = inp.head_dim
    seg = torch.as_tensor(lay_seg)
    mask = seg[:, None] == seg[None, :]
    img = torch.as_tensor(is_img)
    j = torch.arange(d // 4, dtype=torch.float64)
    om_ = theta ** (-(4.0 * j) / d)
    r = torch.as_tensor(np.where(is_img, row, 0), dtype=torch.float64)
    c = torch.as_tensor(np.where(is_img, col, 0), dtype=torch.float64)
    ang = torch.cat([r[:, None] * om_, c[:, None] * om_], dim=1)   # [N, d/2]
    cs, sn = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rot(x):
        a, b = x[..., 0::2], x[..., 1::2]
        return torch.stack([a * cs - b * sn, a * sn + b * cs], dim=-1).flatten(-2)

    def norm(x, g_text, g_img, eps):
        rho = torch.rsqrt((x * x).mean(-1, keepdim=True) + eps)
        g = torch.where(img[:, None], g_img[None, :], g_text[None, :])
        return x * rho * g[:, None, :]

    def fwd(q, k, v, gains):
        qh = rot(norm(q, gains[0], gains[1], inp.rms_eps))
        kh = rot(norm(k, gains[2], gains[3], inp.rms_eps))
        o = torch.nn.functional.scaled_dot_product_attention(
            qh.transpose(0, 1), kh.transpose(0, 1), v.transpose(0, 1),
            attn_mask=mask)
        return o.transpose(0, 1), qh, kh
    return fwd


def _run(inp):
    return oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k,
                          inp.v, inp.gains, inp.rms_eps, inp.rope_theta)


def _run_bwd(inp, dout=None):
    return oracle.backward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k,
                           inp.v, inp.gains, inp.dout if dout is None else dout,
                           inp.rms_eps, inp.rope_theta)


def _close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= tol * scale + 1e-300, f"max err {err:.3e} vs scale {scale:.3e}"


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_layout_golden():
    samples, cu, toks = [], None, []
    with open(os.path.join(GOLDEN, "layout_small.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] == "sample":
                samples.append(tuple(int(x) for x in p[1:]))
            elif p[0] == "cu":
                cu = [int(x) for x in p[1:]]
            elif p[0] == "tok":
                toks.append((int(p[2]), p[3] == "i", int(p[4]), int(p[5])))
    T = [s[0] for s in samples]; hs = [s[1] for s in samples]; ws = [s[2] for s in samples]
    lay = oracle.layout(T, hs, ws)
    assert list(lay.cu_seqlens) == cu
    got = list(zip(lay.segment.tolist(), lay.is_image.tolist(), lay.row.tolist(), lay.col.tolist()))
    assert got == toks


def pin_layout_enumeration():
    rng = np.random.default_rng(1)
    for _ in range(20):
        S = int(rng.integers(1, 7))
        T = rng.integers(0, 20, S); hs = rng.integers(0, 6, S); ws = rng.integers(1, 6, S)
        hs = np.where(T + hs * ws == 0, 1, hs)
        lay = oracle.layout(T, hs, ws)
        toks = _enumerate_tokens(T, hs, ws)
        got = list(zip(lay.segment.tolist(), lay.is_image.tolist(), lay.row.tolist(), lay.col.tolist()))
        assert got == toks
    # the tiny two-sample workload: (32 + 16*16) + (24 + 16*8) = 440 tokens
    w = workloads.get("tiny_fp32")
    lay = oracle.layout(w.text, [g[0] for g in w.grids], [g[1] for g in w.grids])
    assert list(lay.cu_seqlens) == [0, 288, 440]


def pin_layout_edit_enumeration():
    rng = np.random.default_rng(11)
    for _ in range(20):
        S = int(rng.integers(1, 6))
        T = rng.integers(0, 9, S); hs = rng.integers(1, 5, S); ws = rng.integers(1, 5, S)
        sh = rng.integers(0, 5, S); sw = rng.integers(1, 5, S)
        sh = np.where(rng.random(S) < 0.3, 0, sh); sw = np.where(sh == 0, 0, sw)
        lay = oracle.layout(T, hs, ws, sh, sw)
        assert lay.three_axes
        got = list(zip(lay.segment.tolist(), lay.is_image.tolist(), lay.row.tolist(),
                       lay.col.tolist(), lay.frame.tolist()))
        assert got == _enumerate_tokens_edit(T, hs, ws, sh, sw)
    # one 1024^2 edit: 512 text tokens, 64x64 target and 64x64 source latents
    lay = oracle.layout([512], [64], [64], [64], [64])
    assert list(lay.cu_seqlens) == [0, 512 + 2 * 4096]
    assert lay.frame[512:512 + 4096].max() == 0 and lay.frame[512 + 4096:].min() == 1
    # a generation pack has no frame axis and frame 0 everywhere
    g = oracle.layout([3], [2], [2])
    assert not g.three_axes and not np.any(g.frame)


def pin_rmsnorm_closed_forms():
    rng = np.random.default_rng(2)
    eps = 1e-6
    # x = (3, 4, 0, 0): mean square 25/4, rho = 2/5 (eps = 0) -> y = (1.2, 1.6, 0, 0) * g
    x = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    g = np.array([[0.5, 2.0, 1.0, 1.0]])
    y, rho = oracle.rms_norm(x, g, 0.0)
    _close(y[0, 0], [0.6, 3.2, 0.0, 0.0], 1e-15)
    _close(rho, [[0.4]], 1e-15)
    # unit gain: mean(y^2) = m / (m + eps)
    x = rng.standard_normal((5, 3, 16)) * rng.uniform(0.01, 3.0, (5, 3, 1))
    y, _ = oracle.rms_norm(x, np.ones((5, 16)), eps)
    m = np.mean(x * x, -1)
    _close(np.mean(y * y, -1), m / (m + eps), 1e-13)
    # scale invariance when eps = 0
    y1, _ = oracle.rms_norm(x, np.ones((5, 16)), 0.0)
    y2, _ = oracle.rms_norm(7.5 * x, np.ones((5, 16)), 0.0)
    _close(y1, y2, 1e-14)
    # constant vector c*1 with eps: y = c / sqrt(c^2 + eps) * g
    c = 0.003
    y, _ = oracle.rms_norm(np.full((1, 1, 8), c), np.ones((1, 8)) * 2.0, eps)
    _close(y, np.full((1, 1, 8), 2.0 * c / math.sqrt(c * c + eps)), 1e-14)


def pin_modality_separation():
    inp = workloads.random_pack(3, heads=2, head_dim=8, backward=False,
                                text=[5, 3], grids=[(2, 3), (3, 2)])
    lay = oracle.layout(inp.text_len, inp.grid_h, inp.grid_w)
    a = oracle.prologue(inp.q, inp.k, inp.gains, lay)
    g2 = inp.gains.copy()
    g2[0] += 1.0; g2[2] -= 0.5     # text gains only
    b = oracle.prologue(inp.q, inp.k, g2, lay)
    img = lay.is_image
    for i in (0, 1):
        _close(a[i][img], b[i][img], 0.0)
        assert np.max(np.abs(a[i][~img] - b[i][~img])) > 1e-3
    g3 = inp.gains.copy()
    g3[1] *= 3.0; g3[3] *= -1.0    # image gains only
    c = oracle.prologue(inp.q, inp.k, g3, lay)
    for i in (0, 1):
        _close(a[i][~img], c[i][~img], 0.0)
        assert np.max(np.abs(a[i][img] - c[i][img])) > 1e-3


def pin_rope_golden():
    with open(os.path.join(GOLDEN, "rope_angles.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    rng = np.random.default_rng(4)
    for p in rows:
        d, mod, r, c = int(p[0]), p[1], int(p[2]), int(p[3])
        ang = [float(x) for x in p[4:]]
        assert len(ang) == d // 2
        if mod == "i":
            lay = oracle.layout([0], [r + 1], [c + 1])
            t = r * (c + 1) + c
        else:
            lay = oracle.layout([1], [0], [0])
            t = 0
        x = rng.standard_normal((lay.num_tokens, 1, d))
        y = oracle.rope_apply(x, oracle.rope_angles(lay, d))[t, 0]
        for j, phi in enumerate(ang):
            a_, b_ = x[t, 0, 2 * j], x[t, 0, 2 * j + 1]
            exp = (a_ * math.cos(phi) - b_ * math.sin(phi), a_ * math.sin(phi) + b_ * math.cos(phi))
            assert abs(y[2 * j] - exp[0]) < 1e-12 and abs(y[2 * j + 1] - exp[1]) < 1e-12, (p, j)


def pin_rope_properties():
    rng = np.random.default_rng(5)
    d = 64
    lay = oracle.layout([3, 2], [6, 5], [7, 9])
    ang = oracle.rope_angles(lay, d)
    x = rng.standard_normal((lay.num_tokens, 2, d))
    y = oracle.rope_apply(x, ang)
    # per-pair norm preservation
    _close(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2, 1e-13)
    # text tokens are not rotated
    _close(y[~lay.is_image], x[~lay.is_image], 0.0)
    # inverse and composition
    _close(oracle.rope_backward(y, ang), x, 1e-13)
    _close(oracle.rope_apply(oracle.rope_apply(x, ang), 0.5 * ang), oracle.rope_apply(x, 1.5 * ang), 1e-12)
    # q.k after rotation depends only on (row1 - row2, col1 - col2)
    q = rng.standard_normal(d); k = rng.standard_normal(d)
    big = oracle.layout([0], [40], [40])
    angb = oracle.rope_angles(big, d)
    def score(p1, p2):
        i1 = p1[0] * 40 + p1[1]; i2 = p2[0] * 40 + p2[1]
        qq = oracle.rope_apply(np.broadcast_to(q, (big.num_tokens, 1, d)).copy(), angb)[i1, 0]
        kk = oracle.rope_apply(np.broadcast_to(k, (big.num_tokens, 1, d)).copy(), angb)[i2, 0]
        return float(qq @ kk)
    base = score((3, 5), (10, 2))
    for sh in [(1, 0), (0, 7), (20, 20), (-3, 4)]:
        s2 = score((3 + sh[0], 5 + sh[1]), (10 + sh[0], 2 + sh[1]))
        assert abs(s2 - base) < 1e-10 * max(1.0, abs(base))
    # and it does depend on the offset
    assert abs(score((3, 5), (10, 3)) - base) > 1e-6
    # frequencies: omega_0 = 1, and the last one is theta^(-(d-4)/d)
    om_ = oracle.rope_frequencies(128)
    assert om_[0] == 1.0 and abs(om_[-1] / 10000.0 ** (-124.0 / 128.0) - 1) < 1e-14


def _edit_token(d, f, r, c, image=True):
    """Layout of an editing pack holding the given token, and its index."""
    if not image:
        return oracle.layout([1], [0], [0], [0], [0]), 0
    if f == 0:
        return oracle.layout([0], [r + 1], [c + 1], [0], [0]), r * (c + 1) + c
    return oracle.layout([0], [1], [1], [r + 1], [c + 1]), 1 + r * (c + 1) + c


def pin_rope3d_golden():
    with open(os.path.join(GOLDEN, "rope3d_angles.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 6
    for p in rows:
        d, theta, mod = int(p[0]), float(p[1]), p[2]
        f_, r, c = int(p[3]), int(p[4]), int(p[5])
        want = np.array([float(x) for x in p[6:]])
        assert len(want) == d // 2
        lay, t = _edit_token(d, f_, r, c, mod == "i")
        assert lay.frame[t] == f_ and lay.row[t] == (r if mod == "i" else 0)
        got = oracle.rope_angles(lay, d, theta)[t]
        assert np.max(np.abs(got - want)) <= 1e-14 * max(1.0, np.max(np.abs(want))), (p, got)


def pin_rope3d_properties():
    rng = np.random.default_rng(12)
    for d in (64, 128):
        fp = d // 8
        lay = oracle.layout([4, 3], [5, 3], [6, 7], [4, 0], [3, 0])
        ang = oracle.rope_angles(lay, d)
        x = rng.standard_normal((lay.num_tokens, 2, d))
        y = oracle.rope_apply(x, ang)
        _close(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2, 1e-13)
        _close(y[~lay.is_image], x[~lay.is_image], 0.0)
        # frame-0 (target) tokens leave the frame pairs unrotated; frame-1
        # (source) tokens do not
        tgt = lay.is_image & (lay.frame == 0)
        src = lay.is_image & (lay.frame == 1)
        _close(y[tgt][..., :2 * fp], x[tgt][..., :2 * fp], 0.0)
        assert np.all(np.abs(y[src][..., 0:2] - x[src][..., 0:2]) > 0)
        # the same (row, col) on both frames differs only in the frame pairs
        i0 = np.flatnonzero(tgt & (lay.row == 2) & (lay.col == 1))[0]
        i1 = np.flatnonzero(src & (lay.row == 2) & (lay.col == 1))[0]
        _close(ang[i0, fp:], ang[i1, fp:], 0.0)
        assert np.all(ang[i1, :fp] != ang[i0, :fp])
        # q.k after rotation depends only on (dframe, drow, dcol)
        q = rng.standard_normal(d); k = rng.standard_normal(d)

        def score(p1, p2):
            pts = np.array([p1, p2], np.int64)
            L = oracle.Layout(np.array([0, 2]), np.zeros(2, np.int64), np.ones(2, bool),
                              pts[:, 1], pts[:, 2], pts[:, 0], True)
            a_ = oracle.rope_angles(L, d)
            qq = oracle.rope_apply(q[None, None, :].copy(), a_[:1])[0, 0]
            kk = oracle.rope_apply(k[None, None, :].copy(), a_[1:])[0, 0]
            return float(qq @ kk)
        base = score((1, 3, 5), (0, 10, 2))
        for sh in [(1, 0, 0), (0, 1, 0), (0, 0, 7), (5, 20, 20), (-1, -3, 4)]:
            s2 = score((1 + sh[0], 3 + sh[1], 5 + sh[2]), (sh[0], 10 + sh[1], 2 + sh[2]))
            assert abs(s2 - base) < 1e-10 * max(1.0, abs(base))
        # and each axis matters
        for other in [(0, 3, 5), (1, 4, 5), (1, 3, 6)]:
            assert abs(score(other, (0, 10, 2)) - base) > 1e-6
        # section sizes: 1/8, 3/16, 3/16 of d in pairs, covering d/2
        secs = oracle.rope_sections(d, True)
        assert [n for _, n in secs] == [d // 8, 3 * d // 16, 3 * d // 16]
        assert sum(n for _, n in secs) == d // 2


def pin_attention_bruteforce():
    for seed in range(3):
        inp = workloads.random_pack(10 + seed, max_samples=3, max_text=6, max_side=4,
                                    heads=2, head_dim=8, backward=False)
        out = _run(inp)
        lay = out["layout"]
        O, lse = _brute_attention(out["q_hat"], out["k_hat"], inp.v.astype(np.float64), lay.segment)
        _close(out["o"], O, 1e-12)
        _close(out["lse"], lse, 1e-12)


def pin_attention_library():
    for seed in range(3):
        inp = workloads.random_pack(20 + seed, max_samples=4, max_text=30, max_side=7,
                                    heads=3, head_dim=16, backward=False)
        out = _run(inp)
        lay = out["layout"]
        f = _torch_reference(inp, lay.segment, lay.is_image, lay.row, lay.col)
        T = lambda a: torch.as_tensor(np.asarray(a, np.float64))
        o, qh, kh = f(T(inp.q), T(inp.k), T(inp.v), T(inp.gains))
        _close(out["q_hat"], qh.numpy(), 1e-13)
        _close(out["k_hat"], kh.numpy(), 1e-13)
        _close(out["o"], o.numpy(), 1e-12)


def pin_attention_closed_forms():
    inp = workloads.random_pack(30, heads=2, head_dim=8, backward=False,
                                text=[4, 1, 0, 3], grids=[(2, 3), (0, 0), (1, 1), (3, 3)])
    lay = oracle.layout(inp.text_len, inp.grid_h, inp.grid_w)
    cu = lay.cu_seqlens
    # zero gains: Q-hat = K-hat = 0, uniform weights, O = segment mean of V, lse = ln L
    out = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k, inp.v,
                         np.zeros_like(inp.gains))
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        _close(out["o"][a:b], np.broadcast_to(inp.v[a:b].astype(np.float64).mean(0), (b - a,) + inp.v.shape[1:]), 1e-14)
        _close(out["lse"][a:b], np.full((b - a, inp.heads), math.log(b - a)), 1e-14)
    # a one-token sample: O = V, lse = q.k / sqrt(d)
    out = _run(inp)
    t = cu[1]
    _close(out["o"][t], inp.v[t], 1e-15)
    _close(out["lse"][t], np.sum(out["q_hat"][t] * out["k_hat"][t], -1) / math.sqrt(8), 1e-14)
    # constant V: O is that constant
    v = np.broadcast_to(np.arange(8, dtype=np.float64) - 3.5, inp.v.shape).copy()
    out = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k, v, inp.gains)
    _close(out["o"], v, 1e-14)


def pin_packing_invariants():
    inp = workloads.random_pack(40, heads=2, head_dim=16, backward=False,
                                text=[7, 0, 12, 3], grids=[(3, 4), (5, 2), (0, 0), (4, 4)])
    out = _run(inp)
    cu = out["layout"].cu_seqlens
    S = len(cu) - 1
    # packed == each sample run alone
    for i in range(S):
        a, b = cu[i], cu[i + 1]
        one = oracle.forward(inp.text_len[i:i + 1], inp.grid_h[i:i + 1], inp.grid_w[i:i + 1],
                             inp.q[a:b], inp.k[a:b], inp.v[a:b], inp.gains)
        _close(out["o"][a:b], one["o"], 1e-13)
        _close(out["lse"][a:b], one["lse"], 1e-13)
    # permuting samples permutes outputs
    perm = [2, 0, 3, 1]
    sl = lambda x: np.concatenate([x[cu[i]:cu[i + 1]] for i in perm])
    pout = oracle.forward(inp.text_len[perm], inp.grid_h[perm], inp.grid_w[perm],
                          sl(inp.q), sl(inp.k), sl(inp.v), inp.gains)
    _close(pout["o"], sl(out["o"]), 1e-13)
    # joint coupling: moving one image token's V changes that sample's text
    # outputs and no other sample's outputs
    v2 = inp.v.copy()
    t_img = cu[0] + 7 + 5
    v2[t_img] += 1.0
    out2 = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k, v2, inp.gains)
    assert np.max(np.abs(out2["o"][cu[0]:cu[0] + 7] - out["o"][cu[0]:cu[0] + 7])) > 1e-4
    _close(out2["o"][cu[1]:], out["o"][cu[1]:], 0.0)


def _loss(inp, q, k, v, gains, dout):
    out = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, q, k, v, gains,
                         inp.rms_eps, inp.rope_theta)
    return float(np.sum(out["o"] * dout))


def pin_backward_finite_differences():
    rng = np.random.default_rng(50)
    for seed in range(2):
        inp = workloads.random_pack(50 + seed, max_samples=3, max_text=8, max_side=4,
                                    heads=2, head_dim=8, backward=True)
        q, k, v = (inp.q.astype(np.float64), inp.k.astype(np.float64), inp.v.astype(np.float64))
        g = inp.gains.astype(np.float64)
        dout = inp.dout.astype(np.float64)
        got = _run_bwd(inp)
        h = 1e-6
        for name, arr, grad in (("q", q, got["dq"]), ("k", k, got["dk"]),
                                ("v", v, got["dv"]), ("g", g, got["dgains"])):
            for _ in range(6):
                idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
                ap, am = arr.copy(), arr.copy()
                ap[idx] += h; am[idx] -= h
                args = {"q": q, "k": k, "v": v, "g": g}
                args[name] = ap; lp = _loss(inp, args["q"], args["k"], args["v"], args["g"], dout)
                args[name] = am; lm = _loss(inp, args["q"], args["k"], args["v"], args["g"], dout)
                fd = (lp - lm) / (2 * h)
                assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def pin_backward_autograd():
    for seed in range(2):
        inp = workloads.random_pack(60 + seed, max_samples=4, max_text=20, max_side=6,
                                    heads=2, head_dim=16, backward=True)
        got = _run_bwd(inp)
        lay = oracle.layout(inp.text_len, inp.grid_h, inp.grid_w)
        f = _torch_reference(inp, lay.segment, lay.is_image, lay.row, lay.col)
        ts = [torch.tensor(np.asarray(a, np.float64), requires_grad=True)
              for a in (inp.q, inp.k, inp.v, inp.gains)]
        o, _, _ = f(*ts)
        (o * torch.as_tensor(inp.dout.astype(np.float64))).sum().backward()
        for t, key in zip(ts, ("dq", "dk", "dv", "dgains")):
            _close(got[key], t.grad.numpy(), 1e-11)


def pin_backward_closed_forms():
    inp = workloads.random_pack(70, heads=2, head_dim=8, backward=True,
                                text=[3, 5], grids=[(2, 2), (3, 1)])
    # constant V: O does not depend on Q, K or the gains
    v = np.broadcast_to(np.linspace(-1, 1, 8), inp.v.shape).copy()
    got = oracle.backward(inp.text_len, inp.grid_h, inp.grid_w, inp.q, inp.k, v, inp.gains, inp.dout)
    for key in ("dq", "dk", "dgains", "dq_hat", "dk_hat"):
        assert np.max(np.abs(got[key])) < 1e-14, key
    # dO = 0: every gradient is zero
    got = _run_bwd(inp, dout=np.zeros_like(inp.dout))
    for key in ("dq", "dk", "dv", "dgains"):
        assert np.max(np.abs(got[key])) == 0.0
    # linear in dO
    a = _run_bwd(inp)
    b = _run_bwd(inp, dout=-2.5 * inp.dout.astype(np.float64))
    for key in ("dq", "dk", "dv", "dgains"):
        _close(b[key], -2.5 * a[key], 1e-13)


# --------------------------------------------------------------------------
# adaLN modulation and gated residual
# --------------------------------------------------------------------------
def _adaln_pack(seed, D, edit=False):
    rng = np.random.default_rng(seed)
    if edit:
        lay = oracle.layout([3, 0, 2], [2, 1, 0], [2, 3, 0], [1, 2, 0], [3, 2, 0])
    else:
        lay = oracle.layout([3, 0, 2], [2, 1, 0], [2, 3, 0])
    S, N = 3, lay.num_tokens
    t = lambda *sh: rng.standard_normal(sh)
    return lay, dict(x=t(N, D) * 2 + 0.5, y=t(N, D), shift=0.3 * t(S, 2, D), scale=0.3 * t(S, 2, D),
                     gate=t(S, 2, D), dh=t(N, D), dz=t(N, D))


def pin_adaln_closed_forms():
    lay = oracle.layout([1], [0], [0])
    z0 = np.zeros((1, 2, 4))
    # (1, 2, 3, 4): mean 2.5, biased variance 1.25, eps = 0
    f = oracle.adaln_forward(lay, np.array([[1.0, 2.0, 3.0, 4.0]]), z0, z0, eps=0.0)
    _close(f["h"][0], [-1.3416407864998738, -0.4472135954999579, 0.4472135954999579,
                       1.3416407864998738], 1e-15)
    _close(f["mean"], [2.5], 0.0)
    _close(f["rstd"], [1 / math.sqrt(1.25)], 1e-15)
    # (1 + scale) = 2, shift = 0.5; text stream of sample 0
    sc = np.zeros((1, 2, 4)); sc[0, 0] = 1.0
    sh = np.zeros((1, 2, 4)); sh[0, 0] = 0.5
    f2 = oracle.adaln_forward(lay, np.array([[1.0, 2.0, 3.0, 4.0]]), sh, sc, eps=0.0)
    _close(f2["h"], 2 * f["h"] + 0.5, 1e-15)
    # a constant row normalises to zero: h = shift
    f3 = oracle.adaln_forward(lay, np.full((1, 4), 7.0), sh, sc, eps=1e-6)
    _close(f3["h"][0], [0.5] * 4, 0.0)
    # residual: gate 0 gives z = x, gate 1 gives z = x + y
    rng = np.random.default_rng(30)
    x, y = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    _close(oracle.adaln_forward(lay, x, z0, z0, 1e-6, y, np.zeros((1, 2, 4)))["z"], x, 0.0)
    _close(oracle.adaln_forward(lay, x, z0, z0, 1e-6, y, np.ones((1, 2, 4)))["z"], x + y, 0.0)
    # unit modulation: mean 0 and mean square var / (var + eps) per row
    x = rng.standard_normal((1, 64)) * 3 + 1
    f4 = oracle.adaln_forward(lay, x, np.zeros((1, 2, 64)), np.zeros((1, 2, 64)), 1e-3)
    var = np.var(x)
    assert abs(np.mean(f4["h"])) < 1e-14
    assert abs(np.mean(f4["h"] ** 2) - var / (var + 1e-3)) < 1e-13


def pin_adaln_library():
    """Per (sample, stream), the op is torch's layer_norm with weight 1 + scale
    and bias shift, applied to x + gate * y."""
    for edit in (False, True):
        lay, a = _adaln_pack(31, 16, edit)
        f = oracle.adaln_forward(lay, a["x"], a["shift"], a["scale"], 1e-5, a["y"], a["gate"])
        for i in range(len(lay.cu_seqlens) - 1):
            for m in (0, 1):
                rows = (lay.segment == i) & (lay.is_image == bool(m))
                if not rows.any():
                    continue
                z = torch.as_tensor(a["x"][rows] + a["gate"][i, m] * a["y"][rows])
                ref = torch.nn.functional.layer_norm(
                    z, (16,), torch.as_tensor(1 + a["scale"][i, m]), torch.as_tensor(a["shift"][i, m]),
                    eps=1e-5)
                _close(f["h"][rows], ref.numpy(), 1e-13)
                _close(f["z"][rows], z.numpy(), 0.0)


def pin_adaln_selection():
    """Changing one (sample, stream) modulation row changes exactly that
    sample's tokens of that stream; an editing sample's target and source
    share the image stream's row."""
    for edit in (False, True):
        lay, a = _adaln_pack(32, 8, edit)
        base = oracle.adaln_forward(lay, a["x"], a["shift"], a["scale"], 1e-6, a["y"], a["gate"])
        for key in ("shift", "scale", "gate"):
            for i in range(3):
                for m in (0, 1):
                    b = {k: v.copy() for k, v in a.items()}
                    b[key][i, m] += 0.7
                    f = oracle.adaln_forward(lay, b["x"], b["shift"], b["scale"], 1e-6, b["y"], b["gate"])
                    changed = np.any(f["h"] != base["h"], axis=1)
                    rows = (lay.segment == i) & (lay.is_image == bool(m))
                    assert np.array_equal(changed, rows), (edit, key, i, m)
        if edit:
            img1 = (lay.segment == 1) & lay.is_image
            assert set(lay.frame[img1].tolist()) == {0, 1}


def _adaln_loss(lay, a, eps=1e-6):
    f = oracle.adaln_forward(lay, a["x"], a["shift"], a["scale"], eps, a["y"], a["gate"])
    return float(np.sum(a["dh"] * f["h"]) + np.sum(a["dz"] * f["z"]))


def pin_adaln_backward_finite_differences():
    lay, a = _adaln_pack(33, 6, edit=True)
    g = oracle.adaln_backward(lay, a["x"], a["shift"], a["scale"], a["dh"], 1e-6, a["y"], a["gate"],
                              a["dz"])
    names = {"x": "dx", "y": "dy", "shift": "dshift", "scale": "dscale", "gate": "dgate"}
    rng = np.random.default_rng(34)
    for key, gk in names.items():
        flat = a[key].reshape(-1)
        for idx in rng.choice(flat.size, size=min(flat.size, 12), replace=False):
            h = 1e-6
            old = flat[idx]
            flat[idx] = old + h; lp = _adaln_loss(lay, a)
            flat[idx] = old - h; lm = _adaln_loss(lay, a)
            flat[idx] = old
            num = (lp - lm) / (2 * h)
            got = g[gk].reshape(-1)[idx]
            assert abs(num - got) < 1e-6 * max(1.0, abs(num)), (key, idx, num, got)


def pin_adaln_backward_autograd():
    lay, a = _adaln_pack(35, 12, edit=False)
    g = oracle.adaln_backward(lay, a["x"], a["shift"], a["scale"], a["dh"], 1e-6, a["y"], a["gate"],
                              a["dz"])
    T = {k: torch.tensor(v, requires_grad=k in ("x", "y", "shift", "scale", "gate"))
         for k, v in a.items()}
    seg = torch.as_tensor(lay.segment)
    st = torch.as_tensor(lay.is_image.astype(np.int64))
    z = T["x"] + T["gate"][seg, st] * T["y"]
    h = torch.nn.functional.layer_norm(z, (12,), eps=1e-6) * (1 + T["scale"][seg, st]) + T["shift"][seg, st]
    (torch.sum(T["dh"] * h) + torch.sum(T["dz"] * z)).backward()
    for key, gk in (("x", "dx"), ("y", "dy"), ("shift", "dshift"), ("scale", "dscale"), ("gate", "dgate")):
        _close(g[gk], T[key].grad.numpy(), 1e-12)


def pin_adaln_backward_closed_forms():
    lay, a = _adaln_pack(36, 8)
    zero = np.zeros_like(a["dh"])
    g = oracle.adaln_backward(lay, a["x"], a["shift"], a["scale"], zero, 1e-6, a["y"], a["gate"])
    for k in ("dx", "dy", "dshift", "dscale", "dgate"):
        _close(g[k], np.zeros_like(g[k]), 0.0)
    # dh = c on every row and scale = 0: sum(h) does not depend on z (the
    # normalised row sums to zero), so dx = 0; dshift = c * (tokens per stream)
    sc0 = np.zeros_like(a["scale"])
    g = oracle.adaln_backward(lay, a["x"], a["shift"], sc0, np.full_like(a["dh"], 0.25), 1e-6)
    assert np.max(np.abs(g["dx"])) < 1e-14
    counts = np.zeros((3, 2))
    for i, m in zip(lay.segment, lay.is_image):
        counts[i, int(m)] += 1
    _close(g["dshift"], 0.25 * counts[:, :, None] * np.ones((1, 1, 8)), 1e-15)
    # without y the op has no dy / dgate, and dz passes straight through
    g1 = oracle.adaln_backward(lay, a["x"], a["shift"], a["scale"], zero, 1e-6, dz=a["dz"])
    assert "dy" not in g1
    _close(g1["dx"], a["dz"], 0.0)


PINS = [pin_layout_golden, pin_layout_enumeration, pin_layout_edit_enumeration,
        pin_rmsnorm_closed_forms, pin_modality_separation, pin_rope_golden,
        pin_rope_properties, pin_rope3d_golden, pin_rope3d_properties,
        pin_attention_bruteforce, pin_attention_library, pin_attention_closed_forms,
        pin_packing_invariants, pin_backward_finite_differences,
        pin_backward_autograd, pin_backward_closed_forms, pin_adaln_closed_forms,
        pin_adaln_library, pin_adaln_selection, pin_adaln_backward_finite_differences,
        pin_adaln_backward_autograd, pin_adaln_backward_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# --------------------------------------------------------------------------
def _mut_rope_sign(x, angles):
    cos, sin = np.cos(angles)[:, None, :], np.sin(angles)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * cos + x[..., 1::2] * sin
    out[..., 1::2] = -x[..., 0::2] * sin + x[..., 1::2] * cos
    return out


def _mut_rope_half(x, angles):
    # rotate-half pairing (p, p + d/4 inside each half) instead of adjacent pairs
    d = x.shape[-1]
    out = x.copy()
    q = d // 4
    for half in (0, 1):
        a = x[..., half * 2 * q: half * 2 * q + q]
        b = x[..., half * 2 * q + q: (half + 1) * 2 * q]
        ang = angles[:, half * q:(half + 1) * q][:, None, :]
        out[..., half * 2 * q: half * 2 * q + q] = a * np.cos(ang) - b * np.sin(ang)
        out[..., half * 2 * q + q:(half + 1) * 2 * q] = a * np.sin(ang) + b * np.cos(ang)
    return out


def _mut_angles_swap(lay, d, theta=10000.0):
    a = om.__dict__["_orig_rope_angles"](lay, d, theta)
    return np.concatenate([a[:, d // 4:], a[:, :d // 4]], axis=1)


def _mut_freq(d, theta=10000.0):
    return np.power(float(theta), -2.0 * np.arange(d // 4) / d)


def _mut_section_freq(n, theta=10000.0):
    return np.power(float(theta), -2.0 * np.arange(n) / n)


def _mut_3d_frame_dropped(d, three_axes=False):
    return [("row", d // 4), ("col", d // 4)]


def _mut_3d_sections_reordered(d, three_axes=False):
    if not three_axes:
        return [("row", d // 4), ("col", d // 4)]
    return [("row", 3 * d // 16), ("col", 3 * d // 16), ("frame", d // 8)]


def _mut_3d_even_split(d, three_axes=False):
    if not three_axes:
        return [("row", d // 4), ("col", d // 4)]
    n = d // 6
    return [("frame", n), ("row", n), ("col", d // 2 - 2 * n)]


def _mut_layout_frames_swapped(text_len, grid_h, grid_w, src_h=None, src_w=None):
    lay = om.__dict__["_orig_layout"](text_len, grid_h, grid_w, src_h, src_w)
    if lay.three_axes:
        lay.frame = np.where(lay.is_image, 1 - lay.frame, 0)
    return lay


def _mut_layout_source_first(text_len, grid_h, grid_w, src_h=None, src_w=None):
    orig = om.__dict__["_orig_layout"]
    if src_h is None:
        return orig(text_len, grid_h, grid_w)
    hs, ws = np.asarray(grid_h), np.asarray(grid_w)
    sh, sw = np.asarray(src_h), np.asarray(src_w)
    has = sh * sw > 0
    # a sample with a source grid lists it first (frame 1), then the target
    lay = orig(text_len, np.where(has, sh, hs), np.where(has, sw, ws),
               np.where(has, hs, 0), np.where(has, ws, 0))
    for i in np.flatnonzero(has):
        seg = (lay.segment == i) & lay.is_image
        lay.frame[seg] = 1 - lay.frame[seg]
    return lay


def _mut_adaln_variant(kind):
    def fwd(lay, x, shift, scale, eps=1e-6, y=None, gate=None):
        z = np.asarray(x, dtype=np.float64)
        if y is not None:
            gt = om._per_token(gate, lay)
            z = gt * z + y if kind == "gate_on_x" else z + gt * y
        mu = z.mean(-1)
        var = z.var(-1, ddof=1 if kind == "unbiased" else 0)
        rstd = 1 / (np.sqrt(var) + eps) if kind == "eps_out" else 1 / np.sqrt(var + eps)
        zh = (z - mu[:, None]) * rstd[:, None]
        mult = om._per_token(scale, lay) + (0.0 if kind == "no_one" else 1.0)
        return dict(z=z, h=zh * mult + om._per_token(shift, lay), mean=mu, rstd=rstd)
    return fwd


def _mut_modulation_stream_swap(lay):
    return 2 * lay.segment + 1 - lay.is_image.astype(np.int64)


def _mut_modulation_sample_shift(lay):
    S = len(lay.cu_seqlens) - 1
    return 2 * ((lay.segment + 1) % S) + lay.is_image.astype(np.int64)


def _mut_adaln_bwd(kind):
    def bwd(lay, x, shift, scale, dh, eps=1e-6, y=None, gate=None, dz=None):
        out = om.__dict__["_orig_adaln_backward"](lay, x, shift, scale, dh, eps, y, gate, dz)
        f = om.adaln_forward(lay, x, shift, scale, eps, y, gate)
        zh = (f["z"] - f["mean"][:, None]) * f["rstd"][:, None]
        g = np.asarray(dh) * (1 + om._per_token(scale, lay))
        S = len(lay.cu_seqlens) - 1
        if kind == "no_proj_term":
            dzt = f["rstd"][:, None] * (g - g.mean(-1, keepdims=True))
            out["dx"] = dzt + (0 if dz is None else dz)
        elif kind == "dscale_no_zhat":
            out["dscale"] = om._segment_sum(np.asarray(dh, np.float64), lay, S)
        elif kind == "dy_no_gate" and y is not None:
            out["dy"] = out["dx"].copy()
        return out
    return bwd


def _mut_rms_eps_out(x, g_tok, eps):
    rho = 1.0 / (np.sqrt(np.mean(x * x, -1)) + eps)
    return x * rho[..., None] * g_tok[:, None, :], rho


def _mut_rms_sum(x, g_tok, eps):
    rho = 1.0 / np.sqrt(np.sum(x * x, -1) + eps)
    return x * rho[..., None] * g_tok[:, None, :], rho


def _mut_gain_swap(gains, lay, which):
    g = np.asarray(gains, np.float64)
    base = 0 if which == "q" else 2
    return np.where(lay.is_image[:, None], g[base][None, :], g[base + 1][None, :])


def _mut_attn_noscale(qh, kh, v, cu, q_block=2048):
    d = qh.shape[-1]
    return om.__dict__["_orig_attention_forward"](qh * math.sqrt(d) ** 0.5, kh * math.sqrt(d) ** 0.5, v, cu, q_block)


def _mut_attn_leak(qh, kh, v, cu, q_block=2048):
    cu = np.asarray(cu).copy()
    if len(cu) > 2:
        cu[1] += 1
    return om.__dict__["_orig_attention_forward"](qh, kh, v, cu, q_block)


def _mut_bwd_no_rowsum(qh, kh, v, dout, cu, q_block=2048):
    Q, K, V, dO = (om._heads_first(t) for t in (qh, kh, v, dout))
    H, N, d = Q.shape
    sc = 1 / math.sqrt(d)
    dQ, dK, dV = np.zeros((H, N, d)), np.zeros((H, N, d)), np.zeros((H, N, d))
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for h in range(H):
            s = Q[h, a:b] @ K[h, a:b].T * sc
            p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
            dV[h, a:b] = p.T @ dO[h, a:b]
            ds = p * (dO[h, a:b] @ V[h, a:b].T)
            dQ[h, a:b] = ds @ K[h, a:b] * sc
            dK[h, a:b] = ds.T @ Q[h, a:b] * sc
    back = lambda t: t.transpose(1, 0, 2).copy()
    return back(dQ), back(dK), back(dV)


def _mut_bwd_dk_transposed(qh, kh, v, dout, cu, q_block=2048):
    dq, dk, dv = om.__dict__["_orig_attention_backward"](qh, kh, v, dout, cu, q_block)
    return dq, dq.copy(), dv


def _mut_rmsbwd_first_term_only(x, g_tok, rho, dy):
    dx = rho[..., None] * g_tok[:, None, :] * dy
    return dx, dy * x * rho[..., None]


def _mut_ropebwd_forward_dir(dy, angles):
    return om.rope_apply(dy, angles)


MUTANTS = {
    "rope_sign": ("rope_apply", _mut_rope_sign),
    "rope_rotate_half": ("rope_apply", _mut_rope_half),
    "rope_row_col_swapped": ("rope_angles", _mut_angles_swap),
    "rope_freq_schedule": ("rope_frequencies", _mut_freq),
    "rope_section_freq_schedule": ("rope_section_frequencies", _mut_section_freq),
    "rope3d_frame_axis_dropped": ("rope_sections", _mut_3d_frame_dropped),
    "rope3d_sections_reordered": ("rope_sections", _mut_3d_sections_reordered),
    "rope3d_even_split": ("rope_sections", _mut_3d_even_split),
    "layout_edit_frames_swapped": ("layout", _mut_layout_frames_swapped),
    "layout_edit_source_first": ("layout", _mut_layout_source_first),
    "adaln_eps_outside_sqrt": ("adaln_forward", _mut_adaln_variant("eps_out")),
    "adaln_unbiased_variance": ("adaln_forward", _mut_adaln_variant("unbiased")),
    "adaln_scale_without_one": ("adaln_forward", _mut_adaln_variant("no_one")),
    "adaln_gate_on_residual_input": ("adaln_forward", _mut_adaln_variant("gate_on_x")),
    "adaln_streams_swapped": ("modulation_index", _mut_modulation_stream_swap),
    "adaln_wrong_sample": ("modulation_index", _mut_modulation_sample_shift),
    "adaln_bwd_projection_term_dropped": ("adaln_backward", _mut_adaln_bwd("no_proj_term")),
    "adaln_bwd_dscale_without_zhat": ("adaln_backward", _mut_adaln_bwd("dscale_no_zhat")),
    "adaln_bwd_dy_without_gate": ("adaln_backward", _mut_adaln_bwd("dy_no_gate")),
    "rms_eps_outside_sqrt": ("rms_norm", _mut_rms_eps_out),
    "rms_sum_not_mean": ("rms_norm", _mut_rms_sum),
    "gains_modality_swapped": ("token_gains", _mut_gain_swap),
    "attn_scale_dropped": ("attention_forward", _mut_attn_noscale),
    "attn_segment_leak": ("attention_forward", _mut_attn_leak),
    "bwd_rowsum_dropped": ("attention_backward", _mut_bwd_no_rowsum),
    "bwd_dk_wrong": ("attention_backward", _mut_bwd_dk_transposed),
    "rmsbwd_term_dropped": ("rms_norm_backward", _mut_rmsbwd_first_term_only),
    "ropebwd_wrong_direction": ("rope_backward", _mut_ropebwd_forward_dir),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(om, "_orig_" + attr, getattr(om, attr), raising=False)
    monkeypatch.setattr(om, attr, fn)
    # the package-level re-exports must see the mutant too
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
