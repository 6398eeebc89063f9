"""Helpers for GPU-vs-oracle parity tests: tolerance gates, device upload,
running the HIP path through the binding, and the oracle on a head subset."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle

# Tolerances: fp32 packs, normwise max relative error <= 1e-5
# (max |g - r| / max |r| per tensor); bf16 packs, per tensor max abs <= 2e-2
# and relative L2 <= 5e-3 (gain gradients: relative L2 only, being sums over
# N*H terms).
F32_TOL = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def errors(got, ref):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    diff = g - r
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    max_ref = float(np.max(np.abs(r))) if r.size else 0.0
    rel_l2 = float(np.linalg.norm(diff) / max(np.linalg.norm(r), 1e-300)) if diff.size else 0.0
    return dict(max_abs=max_abs, normwise=max_abs / max(max_ref, 1e-300), rel_l2=rel_l2)


def check(name, got, ref, dtype, *, l2_only=False, failures=None):
    e = errors(got, ref)
    if not np.any(np.asarray(ref)):
        # An exactly-zero reference (e.g. dQ = dK = 0 for one-token samples):
        # relative errors are undefined; gate the absolute error instead, at the
        # scale of unit-variance inputs.
        ok = e["max_abs"] <= (F32_TOL if dtype == "f32" else BF16_MAX_ABS)
    elif dtype == "f32":
        ok = e["normwise"] <= F32_TOL
    elif l2_only:
        ok = e["rel_l2"] <= BF16_REL_L2
    else:
        ok = e["max_abs"] <= BF16_MAX_ABS and e["rel_l2"] <= BF16_REL_L2
    msg = f"{name}: max_abs={e['max_abs']:.3e} normwise={e['normwise']:.3e} rel_l2={e['rel_l2']:.3e}"
    if failures is not None and not ok:
        failures.append(msg)
    return ok, msg


def to_device(inp, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    up = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    return dict(q=up(inp.q), k=up(inp.k), v=up(inp.v), dout=up(inp.dout),
                gains=torch.from_numpy(inp.gains).to(device))


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def run_gpu(inp, backward=True, device="cuda", bwd_mode="recompute"):
    """Forward (and backward) through the binding. Returns numpy fp64 arrays.
    bwd_mode: "recompute" (dQ with S and dP formed again, the default) or
    "stored_ds" (dQ from the dS the dK/dV kernel stores)."""
    import packed_attention_nr_amd as pam
    import torch
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim,
                    inp.dtype, inp.rope_theta, inp.rms_eps, device=device,
                    src_h=inp.src_h, src_w=inp.src_w)
    t = to_device(inp, device)
    saved = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    out = {k: host(v) for k, v in saved.items()}
    if backward and inp.dout is not None:
        g = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], saved, t["dout"], mode=bwd_mode)
        out.update({k: host(v) for k, v in g.items() if k != "workspace"})
    torch.cuda.synchronize()
    out["lse"] = out["lse"].T            # [N, H] like the oracle
    out["rstd_q"] = out["rstd"][0]
    out["rstd_k"] = out["rstd"][1]
    return out


def run_oracle(inp, heads=None, backward=True):
    """Oracle on a subset of heads (heads are independent except for the gain
    gradients, which are then summed over that subset only)."""
    hs = slice(None) if heads is None else list(heads)
    q, k, v = inp.q[:, hs], inp.k[:, hs], inp.v[:, hs]
    lay = oracle.layout(inp.text_len, inp.grid_h, inp.grid_w, inp.src_h, inp.src_w)
    f = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, q, k, v, inp.gains,
                       inp.rms_eps, inp.rope_theta, lay=lay)
    out = dict(q_hat=f["q_hat"], k_hat=f["k_hat"], o=f["o"], lse=f["lse"],
               rstd_q=f["rstd_q"], rstd_k=f["rstd_k"])
    if backward and inp.dout is not None:
        b = oracle.backward(inp.text_len, inp.grid_h, inp.grid_w, q, k, v, inp.gains,
                            inp.dout[:, hs], inp.rms_eps, inp.rope_theta, lay=f["layout"])
        out.update(b)
    return out


def subset_heads(inp, heads):
    """The same pack restricted to the given heads (inputs sliced, nothing
    redrawn): heads are independent, so each kept head's outputs are those of
    the full pack; the gain gradients become sums over the kept heads only."""
    hs = list(heads)
    cut = lambda a: None if a is None else np.ascontiguousarray(a[:, hs])
    return dataclasses.replace(inp, q=cut(inp.q), k=cut(inp.k), v=cut(inp.v), dout=cut(inp.dout),
                               heads=len(hs))


def sample_offsets(inp):
    L = inp.seqlens().astype(np.int64)
    return np.concatenate([[0], np.cumsum(L)])


def subset_samples(inp, order):
    """The pack made of the given samples, in the given order (token rows
    moved with their samples, nothing redrawn)."""
    off = sample_offsets(inp)
    rows = np.concatenate([np.arange(off[i], off[i + 1]) for i in order])
    pick = lambda a: None if a is None else np.ascontiguousarray(a[rows])
    sel = lambda a: None if a is None else np.asarray(a)[list(order)]
    return dataclasses.replace(inp, text_len=sel(inp.text_len), grid_h=sel(inp.grid_h),
                               grid_w=sel(inp.grid_w), src_h=sel(inp.src_h), src_w=sel(inp.src_w),
                               q=pick(inp.q), k=pick(inp.k), v=pick(inp.v),
                               dout=pick(inp.dout)), rows

