"""Benchmark of the packed joint-attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixed6]

One step = one pass of the whole path over one synthetic pack: the host pack
plan and its upload, the forward (QK-norm + 2D RoPE prologue, var-len
attention) and the backward (D = rowsum(dO*O), var-len attention backward
with the prologue backward fused into its epilogues, gain-gradient reduction;
--bwd-mode stored_ds forms dQ from the dS that the dK/dV kernel stores).
HIP events recorded on the launch stream between the stages give each
kernel's duration inside the timed region.
Prints one JSON line.

metric: bf16 forward+backward attention throughput in TFLOP/s, counting
4*H*d*sum(L_i^2) for the forward and 10*H*d*sum(L_i^2) for the backward,
divided by the whole step time (plan, prologues and preprocess included).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "packed varlen attn TFLOP/s (bf16 fwd+bwd) & % MFMA peak; ms/layer at 1024²"


def sum_l2(inp):
    L = inp.seqlens().astype(np.int64)
    return int((L * L).sum())


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernels_mixed6_hbm_traffic.md")


def source_fingerprint() -> str:
    """sha256 (first 16 hex) over the kernel sources' names and bytes."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "packed_attention_nr_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE/WRITE_SIZE
    summary, or None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            line = next(l for l in fh if l.startswith("traffic_json:"))
        rec = json.loads(line.split(":", 1)[1])
    except (OSError, StopIteration, ValueError):
        return None
    if rec.get("source_fingerprint") != source_fingerprint():
        return None
    k = rec["kernels"].get("mmdit::" + kernel)
    return None if k is None else k["hbm_bytes"]


def cpu_baseline(inp, heads):
    """Time the fp64 oracle (fwd+bwd) on a subset of heads; report TFLOP/s of
    the same algorithmic count, scaled to the metric's unit."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    hs = list(range(heads))
    q, k, v, do = (x[:, hs] for x in (inp.q, inp.k, inp.v, inp.dout))
    t0 = time.perf_counter()
    f = oracle.forward(inp.text_len, inp.grid_h, inp.grid_w, q, k, v, inp.gains)
    oracle.backward(inp.text_len, inp.grid_h, inp.grid_w, q, k, v, inp.gains, do, lay=f["layout"])
    dt = time.perf_counter() - t0
    flops = 14.0 * heads * inp.head_dim * sum_l2(inp)
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=int(threads),
                kind="oracle",
                sample=f"fp64 numpy oracle forward+backward of {heads} of {inp.heads} heads "
                       f"of the same pack ({dt:.1f} s); throughput of that sample")


def pass_runner(pam, torch, dev, text, hs, ws, H, d, backward, seed, src=None):
    """A callable that runs one whole pass (forward, and backward if asked)
    of the library on a pack of the given geometry (src = (src_h, src_w):
    an editing pack). Inputs are drawn on the device: only the timing of such
    passes is used."""
    sh, sw = (None, None) if src is None else src
    pack = pam.Pack(text, hs, ws, H, d, "bf16", device=dev, src_h=sh, src_w=sw)
    N = pack.N
    g = torch.Generator(device=dev).manual_seed(seed)
    rnd = lambda: torch.randn((N, H, d), generator=g, device=dev).to(torch.bfloat16)
    q, k, v = rnd(), rnd(), rnd()
    gains = 1.0 + 0.1 * torch.randn((4, d), generator=g, device=dev)
    bf = torch.bfloat16
    o = torch.empty((N, H, d), dtype=bf, device=dev)
    q_hat, k_hat = torch.empty_like(o), torch.empty_like(o)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    rstd = torch.empty((2, N, H), dtype=torch.float32, device=dev)
    fa = dict(q=q, k=k, v=v, q_stride=H * d, k_stride=H * d, v_stride=H * d, gains=gains,
              o=o, lse=lse, q_hat=q_hat, k_hat=k_hat, rstd=rstd)
    if backward:
        do = rnd()
        dq, dk, dv = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)
        dgains = torch.empty((4, d), dtype=torch.float32, device=dev)
        wsb = pack.workspace("bwd")
        ba = dict(q=q, k=k, v=v, q_hat=q_hat, k_hat=k_hat, o=o, dout=do, q_stride=H * d,
                  k_stride=H * d, v_stride=H * d, dout_stride=H * d, gains=gains, lse=lse,
                  rstd=rstd, dq=dq, dk=dk, dv=dv, dgains=dgains, workspace=wsb)

    def run():
        pam.mmdit_attn_fwd(pack.plan, pack.blob_dev, **fa)
        if backward:
            pam.mmdit_attn_bwd(pack.plan, pack.blob_dev, **ba)
    return run


def time_passes(torch, runs, reps=20):
    """Milliseconds per round of the given callables run back to back."""
    for _ in range(3):
        for r in runs:
            r()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for r in runs:
            r()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def packed_cfg_1024(pam, torch, dev, H, d):
    """Packed classifier-free guidance at 1024^2: the conditional sample
    (512 text tokens + 64x64 latents) and its unconditional twin (same grid,
    a null prompt) as one forward pass, against the two branches as two
    passes. Null prompt of 0 tokens (empty) and of 512 (padded prompt)."""
    out = {}
    for null in (0, 512):
        t, h, w = pam.mmdit_cfg_pack_desc([512], [64], [64], null)
        packed = pass_runner(pam, torch, dev, t, h, w, H, d, False, 1)
        cond = pass_runner(pam, torch, dev, t[:1], h[:1], w[:1], H, d, False, 2)
        unc = pass_runner(pam, torch, dev, t[1:], h[1:], w[1:], H, d, False, 3)
        t_packed = time_passes(torch, [packed], 50)
        t_two = time_passes(torch, [cond, unc], 50)
        out[f"null_text_{null}"] = {"packed_ms": round(t_packed, 4), "two_passes_ms": round(t_two, 4),
                                    "speedup": round(t_two / t_packed, 3)}
    return out


def edit_1024(pam, torch, dev):
    """One 1024^2 editing step's attention core: 512 text tokens, the 64x64
    target latents and the 64x64 source latents on a second RoPE frame
    (8,704 tokens, H=24, d=128): whole forward call, and forward + backward."""
    w = workloads.get("edit1024")
    t, hs, ws = list(w.text), [g[0] for g in w.grids], [g[1] for g in w.grids]
    src = ([g[0] for g in w.src], [g[1] for g in w.src])
    fwd = pass_runner(pam, torch, dev, t, hs, ws, w.heads, w.head_dim, False, 4, src)
    both = pass_runner(pam, torch, dev, t, hs, ws, w.heads, w.head_dim, True, 5, src)
    L = t[0] + hs[0] * ws[0] + src[0][0] * src[1][0]
    flop1 = w.heads * w.head_dim * float(L) ** 2
    t_f = time_passes(torch, [fwd], 50)
    t_fb = time_passes(torch, [both], 20)
    return {"tokens": L, "fwd_ms": round(t_f, 4), "fwd_tflops": round(4 * flop1 / t_f / 1e9, 1),
            "fwd_bwd_ms": round(t_fb, 4), "fwd_bwd_tflops": round(14 * flop1 / t_fb / 1e9, 1)}


def adaln_block(pam, torch, dev, inp, D):
    """adaLN modulation with the fused gated residual on the timed pack at
    model width D (= H * d): forward (x, y -> z, h, statistics) and backward
    (x, y, dh, dz -> dx, dy and the modulation gradients), bf16, inputs drawn
    on the device. HBM roofline: algorithmic bytes = every token tensor once
    (forward 8*N*D + 8*N, backward 12*N*D + 8*N) over the event-timed call."""
    N, S = inp.num_tokens, len(inp.text_len)
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, 24, 128, "bf16", device=dev)
    g = torch.Generator(device=dev).manual_seed(7)
    x, y, dh, dz = (torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(4))
    shift, scale, gate = (0.3 * torch.randn((S, 2, D), generator=g, device=dev) for _ in range(3))
    h, z = torch.empty_like(x), torch.empty_like(x)
    stats = torch.empty((N, 2), dtype=torch.float32, device=dev)
    dx, dy = torch.empty_like(x), torch.empty_like(x)
    dsh, dsc, dg = (torch.empty((S, 2, D), device=dev) for _ in range(3))
    ws = pack.workspace("adaln", D)

    def fwd():
        pam.mmdit_adaln_fwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=D, y_stride=D, shift=shift,
                            scale=scale, gate=gate, model_dim=D, z=z, h=h, stats=stats)

    def bwd():
        pam.mmdit_adaln_bwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=D, y_stride=D, scale=scale,
                            gate=gate, model_dim=D, stats=stats, dh=dh, dz=dz, dh_stride=D,
                            dz_stride=D, dx=dx, dy=dy, dshift=dsh, dscale=dsc, dgate=dg, workspace=ws)
    out = {"model_dim": D, "tokens": N}
    for name, fn, nbytes in (("fwd", fwd, 8 * N * D + 8 * N), ("bwd", bwd, 12 * N * D + 8 * N)):
        ms = time_passes(torch, [fn], 50)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 1), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def bucket_padding(pam, torch, dev, inp, H, d):
    """The same samples as dense per-bucket batches: one batch per distinct
    latent grid, every text padded to the longest prompt of the workload's
    range (512, or the longest drawn), padded tokens computed. Forward +
    backward of all bucket batches, against the packed pass."""
    text_pad = max(512, int(np.max(inp.text_len)))
    buckets = {}
    for hh, ww in zip(inp.grid_h.tolist(), inp.grid_w.tolist()):
        buckets[(hh, ww)] = buckets.get((hh, ww), 0) + 1
    runs = []
    padded_l2 = 0.0
    for j, ((hh, ww), n) in enumerate(sorted(buckets.items())):
        runs.append(pass_runner(pam, torch, dev, [text_pad] * n, [hh] * n, [ww] * n, H, d, True, 10 + j))
        padded_l2 += n * float(text_pad + hh * ww) ** 2
    t_buckets = time_passes(torch, runs, 10)
    packed = pass_runner(pam, torch, dev, inp.text_len, inp.grid_h, inp.grid_w, H, d, True, 9)
    packed_ms = time_passes(torch, [packed], 10)
    return {"buckets": len(buckets), "text_padded_to": text_pad,
            "padded_flop_ratio": round(padded_l2 / sum_l2(inp), 3),
            "bucketed_ms": round(t_buckets, 4), "packed_ms": round(packed_ms, 4),
            "time_ratio": round(t_buckets / packed_ms, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed6", choices=["mixed6", "gen2048", "small64"])
    ap.add_argument("--cpu-heads", type=int, default=12)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-mode", default="recompute", choices=["recompute", "stored_ds"],
                    help="backward mode of the timed step (stored_ds: dQ from the dS the "
                         "dK/dV kernel writes; needs ~2*H*sum(L^2) bytes of workspace)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(samples and heads are independent, so each GPU would run its own pack).", file=sys.stderr)
        sys.exit(2)

    import torch
    import packed_attention_nr_amd as pam

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = workloads.get(args.workload)
    inp = workloads.draw(args.workload)
    N, H, d = inp.num_tokens, inp.heads, inp.head_dim
    sl2 = sum_l2(inp)
    fwd_flop = 4.0 * H * d * sl2
    bwd_flop = 10.0 * H * d * sl2

    bf = torch.bfloat16
    up = lambda a: torch.from_numpy(a).to(device=dev, dtype=bf)
    q, k, v, do = up(inp.q), up(inp.k), up(inp.v), up(inp.dout)
    gains = torch.from_numpy(inp.gains).to(dev)
    o = torch.empty((N, H, d), dtype=bf, device=dev)
    q_hat, k_hat = torch.empty_like(o), torch.empty_like(o)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    rstd = torch.empty((2, N, H), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(o), torch.empty_like(o), torch.empty_like(o)
    dgains = torch.empty((4, d), dtype=torch.float32, device=dev)

    plan0, blob0 = pam.mmdit_pack_plan(inp.text_len, inp.grid_h, inp.grid_w, H, d, pam.MMDIT_BF16)
    # The backward in its recompute mode (dQ with D, then dK/dV) or, with
    # --bwd-mode stored_ds, in its stored-dS mode (D, then dK/dV writing dS,
    # then dQ from dS); each stage is its own call so that events separate them.
    B = pam.BWD_STAGES
    ds_mode = args.bwd_mode == "stored_ds"
    if ds_mode and not plan0.bwd_ds_workspace_bytes > plan0.bwd_workspace_bytes:
        raise SystemExit("this pack has no stored-dS backward")
    if ds_mode:
        bcalls = [("bwd_d", B["d"] | B["store_ds"]), ("attn_bwd_dkdv", B["dkdv"] | B["store_ds"]),
                  ("attn_bwd_dq", B["dq"] | B["store_ds"]), ("gain_reduce", B["gains"])]
    else:
        bcalls = [("attn_bwd_dq", B["dq"]), ("attn_bwd_dkdv", B["dkdv"]), ("gain_reduce", B["gains"])]
    names = ["prologue_fwd", "attn_fwd"] + [n for n, _ in bcalls]
    ws_bytes = plan0.bwd_ds_workspace_bytes if ds_mode else plan0.bwd_workspace_bytes
    ws = torch.empty(int(ws_bytes), dtype=torch.uint8, device=dev)
    blob_dev = [torch.empty(int(plan0.blob_bytes), dtype=torch.uint8, device=dev) for _ in range(2)]
    pinned = [torch.empty(int(plan0.blob_bytes), dtype=torch.uint8).pin_memory() for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    for e in copied:
        e.record()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    S = pam.FWD_STAGES

    def step(i, evs=None):
        # a1: host plan + upload of its blob (pinned ring of two buffers)
        plan, blob = pam.mmdit_pack_plan(inp.text_len, inp.grid_h, inp.grid_w, H, d, pam.MMDIT_BF16)
        slot = i & 1
        copied[slot].synchronize()
        pinned[slot].numpy()[:] = blob
        blob_dev[slot].copy_(pinned[slot], non_blocking=True)
        copied[slot].record()
        bd = blob_dev[slot]
        rec = (lambda j: evs[j].record(stream)) if evs else (lambda j: None)
        fa = dict(q=q, k=k, v=v, q_stride=H * d, k_stride=H * d, v_stride=H * d, gains=gains,
                  o=o, lse=lse, q_hat=q_hat, k_hat=k_hat, rstd=rstd)
        rec(0)
        pam.mmdit_attn_fwd(plan, bd, stages=S["prologue"], **fa)
        rec(1)
        pam.mmdit_attn_fwd(plan, bd, stages=S["attention"], **fa)
        rec(2)
        ba = dict(q=q, k=k, v=v, q_hat=q_hat, k_hat=k_hat, o=o, dout=do, q_stride=H * d,
                  k_stride=H * d, v_stride=H * d, dout_stride=H * d, gains=gains, lse=lse,
                  rstd=rstd, dq=dq, dk=dk, dv=dv, dgains=dgains, workspace=ws)
        for j, (_, st) in enumerate(bcalls):
            pam.mmdit_attn_bwd(plan, bd, stages=st, **ba)
            rec(3 + j)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    kt = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
          for j, n in enumerate(names)}
    value = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12
    t_bwd = kt["attn_bwd_dq"] + kt["attn_bwd_dkdv"] + kt.get("bwd_d", 0.0)
    bwd_tflops = bwd_flop / (t_bwd * 1e-3) / 1e12
    fwd_tflops = fwd_flop / (kt["attn_fwd"] * 1e-3) / 1e12
    # Dominant kernel's roofline. Algorithmic FLOPs per launch: the dK/dV kernel
    # performs 4 of the backward's 5 products (S, dP, dV, dK: 8*H*d*sum L^2);
    # the dQ kernel adds only dQ (2*H*d*sum L^2), from the stored dS or with
    # S and dP recomputed.
    dkdv_name = "attn_bwd_dkdv_kernel<128, true>" if ds_mode else "attn_bwd_dkdv_kernel<128, false>"
    dq_name = "attn_bwd_dq_ds_kernel<128>" if ds_mode else "attn_bwd_dq_kernel<128>"
    cand = {"attn_bwd_dkdv": (8.0 * H * d * sl2, dkdv_name),
            "attn_bwd_dq": (2.0 * H * d * sl2, dq_name),
            "attn_fwd": (fwd_flop, "attn_fwd_bf16_kernel<128>")}
    dom = max(cand, key=lambda n: kt[n])
    ach = cand[dom][0] / (kt[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": cand[dom][1], "achieved": round(ach, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(cand[dom][1]) if args.workload == "mixed6" else None,
            "algorithmic_flop_per_launch": cand[dom][0]}
    pro_bytes = 8.0 * N * H * d
    pro_gbs = pro_bytes / (kt["prologue_fwd"] * 1e-3) / 1e9

    # ms/layer at 1024^2: the whole forward call (prologue + attention) on the
    # 1024^2 generation pack (512 text + 64x64 latents, H=24, d=128).
    g = workloads.draw("gen1024")
    gpack = pam.Pack(g.text_len, g.grid_h, g.grid_w, g.heads, g.head_dim, "bf16", device=dev)
    gq, gk, gv = up(g.q), up(g.k), up(g.v)
    ggains = torch.from_numpy(g.gains).to(dev)
    for _ in range(5):
        pam.forward(gpack, gq, gk, gv, ggains, save_for_backward=False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 50
    gout = dict(o=torch.empty((g.num_tokens, g.heads, g.head_dim), dtype=bf, device=dev),
                lse=torch.empty((g.heads, g.num_tokens), dtype=torch.float32, device=dev))
    gws = gpack.workspace("fwd")
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        pam.mmdit_attn_fwd(gpack.plan, gpack.blob_dev, q=gq, k=gk, v=gv, q_stride=g.heads * g.head_dim,
                           k_stride=g.heads * g.head_dim, v_stride=g.heads * g.head_dim,
                           gains=ggains, workspace=gws, **gout)
    e1.record()
    torch.cuda.synchronize()
    ms_layer_1024 = e0.elapsed_time(e1) / reps
    gen_fwd_tflops = 4.0 * g.heads * g.head_dim * sum_l2(g) / (ms_layer_1024 * 1e-3) / 1e12

    cfg = packed_cfg_1024(pam, torch, dev, H, d)
    edit = edit_1024(pam, torch, dev)
    adaln = adaln_block(pam, torch, dev, inp, H * d)
    bucket = bucket_padding(pam, torch, dev, inp, H, d)

    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, gains 1+0.1*N(0,1))",
        "config": {"workload": w.title, "tokens": N, "samples": len(inp.text_len),
                   "seqlens": inp.seqlens().tolist(), "heads": H, "head_dim": d,
                   "parallelism": "none (1 GPU)"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {n: round(t, 4) for n, t in kt.items()},
        "bwd_mode": "stored_ds" if ds_mode else "recompute",
        "attn_fwd_tflops": round(fwd_tflops, 2),
        "attn_fwd_frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "attn_bwd_tflops": round(bwd_tflops, 2),
        "attn_bwd_frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
        "prologue_fwd_gbs": round(pro_gbs, 1),
        "prologue_fwd_frac_hbm": round(pro_gbs / PEAK_HBM_GBS, 4),
        "ms_per_layer_1024": round(ms_layer_1024, 4),
        "gen1024_fwd_tflops": round(gen_fwd_tflops, 2),
        "roofline": roof,
        "packed_cfg_1024": cfg,
        "edit_1024": edit,
        "adaln_gated_residual": adaln,
        "bucket_padding": bucket,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
