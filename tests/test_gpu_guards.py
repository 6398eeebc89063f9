"""GPU checks of the boundary: guard bands around every output and past every
workspace, closed forms the method reaches exactly or nearly (constant V,
zero gains), a device blob of another pack, and an explicit side stream.
Marked ``gpu``: needs an MI355X and the built library.

The closed forms follow from the definition of the attention the pages pack
(picx.dev "Mage-Flow: An Efficient Native-Resolution Foundation Model for
Image Generation and Editing", section "Native-Resolution MMDiT (NR-MMDiT)"):
with zero gains every normalised query and key is zero, so every score is
zero and each token attends uniformly to its own sample; with V constant over
a sample, every output row equals that constant."""
import sys

import numpy as np
import pytest

import workloads
from parity import check, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_attention_nr_amd as pam
    pam.lib()  # must load: no fallback
    assert pam.mmdit_device_faults() == 0


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


GUARD = 4096          # guard bytes on each side of every output
PATTERN = 0xA5        # guard byte value (not a value any kernel writes by chance)


class Guarded:
    """Device buffers carved out of larger ones with GUARD pattern bytes on
    both sides; check() says which guards changed."""

    def __init__(self, dev="cuda"):
        self.dev = dev
        self.bufs = {}

    def empty(self, name, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device=self.dev)
        self.bufs[name] = (raw, n)
        return raw[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        bad = []
        for name, (raw, n) in self.bufs.items():
            lo, hi = raw[:GUARD], raw[GUARD + n:]
            if not (bool((lo == PATTERN).all()) and bool((hi == PATTERN).all())):
                bad.append(name)
        return bad


def _pack_and_inputs(inp):
    import packed_attention_nr_amd as pam
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, inp.dtype,
                    src_h=inp.src_h, src_w=inp.src_w)
    return pack, to_device(inp)


GUARD_PACKS = [
    ("bf16_d128_ragged", 61, "bf16", 128, dict(text=[45, 3, 130], grids=[(13, 11), (2, 5), (7, 19)])),
    ("bf16_d64_one_token", 62, "bf16", 64, dict(text=[1, 0, 77], grids=[(0, 0), (1, 1), (5, 9)])),
    ("f32_d64_ragged", 63, "f32", 64, dict(text=[20, 9], grids=[(6, 7), (3, 3)])),
]


@pytest.mark.parametrize("name,seed,dtype,d,spec", GUARD_PACKS, ids=[c[0] for c in GUARD_PACKS])
def test_guard_bands(name, seed, dtype, d, spec):
    """Every output of the forward, both backward modes and the inference
    forward sits between guard bands, and every workspace is handed over
    larger than needed: after the calls the guards and the bytes past the
    needed workspace are unchanged, and the results still match the oracle."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(seed, heads=3, head_dim=d, dtype=dtype, **spec)
    _say(f"guard bands {name} N={inp.num_tokens}")
    pack, t = _pack_and_inputs(inp)
    N, H = pack.N, pack.H
    dt = pack.torch_dtype
    G = Guarded()
    o = G.empty("o", (N, H, d), dt)
    lse = G.empty("lse", (H, N), torch.float32)
    q_hat, k_hat = G.empty("q_hat", (N, H, d), dt), G.empty("k_hat", (N, H, d), dt)
    rstd = G.empty("rstd", (2, N, H), torch.float32)
    HD = H * d
    pam.mmdit_attn_fwd(pack.plan, pack.blob_dev, q=t["q"], k=t["k"], v=t["v"], q_stride=HD,
                       k_stride=HD, v_stride=HD, gains=t["gains"], o=o, lse=lse, q_hat=q_hat,
                       k_hat=k_hat, rstd=rstd)
    # inference forward: Q-hat / K-hat in a workspace handed over 64 KiB too large
    fws_need = int(pack.plan.fwd_workspace_bytes)
    fws = torch.full((fws_need + 65536,), PATTERN, dtype=torch.uint8, device="cuda")
    o2 = G.empty("o (inference)", (N, H, d), dt)
    lse2 = G.empty("lse (inference)", (H, N), torch.float32)
    pam.mmdit_attn_fwd(pack.plan, pack.blob_dev, q=t["q"], k=t["k"], v=t["v"], q_stride=HD,
                       k_stride=HD, v_stride=HD, gains=t["gains"], o=o2, lse=lse2, workspace=fws)
    modes = [("recompute", 0, int(pack.plan.bwd_workspace_bytes))]
    if pack.plan.bwd_ds_workspace_bytes > pack.plan.bwd_workspace_bytes:
        modes.append(("stored_ds", pam.STAGE_BWD_STORE_DS, int(pack.plan.bwd_ds_workspace_bytes)))
    grads, tails = {}, []
    for mode, stages, need in modes:
        ws = torch.full((need + 65536,), PATTERN, dtype=torch.uint8, device="cuda")
        g = {n: G.empty(f"{n} ({mode})", (N, H, d), dt) for n in ("dq", "dk", "dv")}
        g["dgains"] = G.empty(f"dgains ({mode})", (4, d), torch.float32)
        pam.mmdit_attn_bwd(pack.plan, pack.blob_dev, q=t["q"], k=t["k"], v=t["v"], q_hat=q_hat,
                           k_hat=k_hat, o=o, dout=t["dout"], q_stride=HD, k_stride=HD, v_stride=HD,
                           dout_stride=HD, gains=t["gains"], lse=lse, rstd=rstd, workspace=ws,
                           stages=stages, **g)
        grads[mode] = g
        tails.append((f"backward workspace past {need} bytes ({mode})", ws, need))
    tails.append((f"forward workspace past {fws_need} bytes", fws, fws_need))
    bad = G.check()
    for label, ws, need in tails:
        if not bool((ws[need:] == PATTERN).all()):
            bad.append(label)
    assert pam.mmdit_device_faults() == 0
    assert not bad, f"written outside their bounds: {bad}"
    ref = run_oracle(inp)
    fails = []
    host = lambda x: x.double().cpu().numpy()
    for key, got in (("o", o), ("q_hat", q_hat), ("k_hat", k_hat)):
        _, msg = check(key, host(got), ref[key], dtype, failures=fails)
        _say("   " + msg)
    assert torch.equal(o, o2), "inference forward differs from the stored forward"
    for mode, g in grads.items():
        for key in ("dq", "dk", "dv"):
            _, msg = check(f"{key} ({mode})", host(g[key]), ref[key], dtype, failures=fails)
            _say("   " + msg)
        _, msg = check(f"dgains ({mode})", host(g["dgains"]), ref["dgains"], dtype, l2_only=True,
                       failures=fails)
        _say("   " + msg)
    assert not fails, fails


def test_adaln_guard_bands():
    """adaLN forward and backward outputs between guard bands, its workspace
    handed over larger than needed: nothing written outside."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(64, heads=1, head_dim=64, dtype="bf16", text=[13, 40],
                                grids=[(5, 7), (0, 0)])
    pack, _ = _pack_and_inputs(inp)
    N, S, D = pack.N, pack.plan.num_samples, 448
    a = workloads.draw_adaln(5, N, S, D, "bf16")
    up = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(x).cuda()
    x, y, dh, dz = up(a["x"]), up(a["y"]), up(a["dh"]), up(a["dz"])
    shift, scale, gate = f32(a["shift"]), f32(a["scale"]), f32(a["gate"])
    G = Guarded()
    z, h = G.empty("z", (N, D), torch.bfloat16), G.empty("h", (N, D), torch.bfloat16)
    stats = G.empty("stats", (N, 2), torch.float32)
    pam.mmdit_adaln_fwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=D, y_stride=D, shift=shift,
                        scale=scale, gate=gate, model_dim=D, z=z, h=h, stats=stats)
    need = pack.plan.num_mod_chunks * 3 * D * 4
    ws = torch.full((need + 65536,), PATTERN, dtype=torch.uint8, device="cuda")
    dx, dy = G.empty("dx", (N, D), torch.bfloat16), G.empty("dy", (N, D), torch.bfloat16)
    dsh, dsc, dg = (G.empty(n, (S, 2, D), torch.float32) for n in ("dshift", "dscale", "dgate"))
    pam.mmdit_adaln_bwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=D, y_stride=D, scale=scale,
                        gate=gate, model_dim=D, stats=stats, dh=dh, dz=dz, dh_stride=D, dz_stride=D,
                        dx=dx, dy=dy, dshift=dsh, dscale=dsc, dgate=dg, workspace=ws)
    bad = G.check()
    if not bool((ws[need:] == PATTERN).all()):
        bad.append("adaLN workspace tail")
    assert not bad, f"written outside their bounds: {bad}"


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
CLOSED_PACK = dict(text=[45, 0, 130, 1], grids=[(13, 11), (9, 7), (2, 5), (0, 0)])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_zero_gains_closed_form(dtype, d):
    """Zero gains: Q-hat = K-hat = 0 exactly, every score is 0, so O is the
    mean of V over the token's own sample and lse = ln L; dQ-hat = dS K-hat
    and dK-hat = dS^T Q-hat vanish, so dq = dk = 0 and dgains = 0 exactly;
    dV is the mean of dO over the sample."""
    import dataclasses
    inp = workloads.random_pack(81, heads=3, head_dim=d, dtype=dtype, **CLOSED_PACK)
    inp = dataclasses.replace(inp, gains=np.zeros_like(inp.gains))
    _say(f"zero gains {dtype} d={d} N={inp.num_tokens}")
    gpu = run_gpu(inp)
    L = inp.seqlens().astype(np.int64)
    off = np.concatenate([[0], np.cumsum(L)])
    seg = np.repeat(np.arange(len(L)), L)
    mean_v = np.stack([inp.v[off[i]:off[i + 1]].astype(np.float64).mean(0) for i in range(len(L))])[seg]
    mean_do = np.stack([inp.dout[off[i]:off[i + 1]].astype(np.float64).mean(0) for i in range(len(L))])[seg]
    assert not np.any(gpu["q_hat"]) and not np.any(gpu["k_hat"])
    assert not np.any(gpu["dq"]) and not np.any(gpu["dk"]) and not np.any(gpu["dgains"])
    fails = []
    for key, got, want in (("o", gpu["o"], mean_v), ("dv", gpu["dv"], mean_do)):
        _, msg = check(key + " vs segment mean", got, want, dtype, failures=fails)
        _say("   " + msg)
    lse_err = float(np.max(np.abs(gpu["lse"] - np.log(L[seg].astype(np.float64))[:, None])))
    _say(f"   lse vs ln L: max_abs={lse_err:.3e}")
    if lse_err > 1e-5 * np.log(L.max()) + 1e-6:
        fails.append(f"lse {lse_err:.3e}")
    assert not fails, fails


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_constant_v_closed_form(dtype, d):
    """V constant over each sample (per head): every output row equals that
    constant (bf16: up to the rounding of P and O), and dS = P (dP - D) with
    dP_ij = dO_i . v = D_i, so dq, dk and dgains vanish up to rounding. Their
    bar: 2e-2 of the largest value the same pack's gradients reach with
    random V (the bf16 rounding of O alone leaves about 2e-3)."""
    import dataclasses
    inp = workloads.random_pack(82, heads=3, head_dim=d, dtype=dtype, **CLOSED_PACK)
    L = inp.seqlens().astype(np.int64)
    off = np.concatenate([[0], np.cumsum(L)])
    rng = np.random.default_rng(83)
    v = np.empty_like(inp.v)
    for i in range(len(L)):
        row = rng.standard_normal((inp.heads, d)).astype(np.float32)
        if dtype == "bf16":
            row = workloads.bf16_round(row)
        v[off[i]:off[i + 1]] = row
    const = dataclasses.replace(inp, v=v)
    _say(f"constant V {dtype} d={d} N={inp.num_tokens}")
    gpu = run_gpu(const)
    base = run_gpu(inp)
    fails = []
    _, msg = check("o vs the constant", gpu["o"], v.astype(np.float64), dtype, failures=fails)
    _say("   " + msg)
    for key in ("dq", "dk", "dgains"):
        scale = float(np.max(np.abs(base[key])))
        got = float(np.max(np.abs(gpu[key])))
        _say(f"   {key}: max_abs={got:.3e} (random-V scale {scale:.3e})")
        if got > 2e-2 * scale:
            fails.append(f"{key} {got:.3e} not small against {scale:.3e}")
    assert not fails, fails


# ---------------------------------------------------------------------------
# a device blob of another pack; an explicit side stream
# ---------------------------------------------------------------------------
def test_stale_blob_is_refused_on_the_device():
    """Kernels given the device blob of another pack (same geometry, another
    RoPE base, so another fingerprint and nothing out of range even if a
    kernel read it) write nothing and record the fault; with the right blob
    the same calls work and record none."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(85, heads=2, head_dim=128, dtype="bf16",
                                text=[30, 4], grids=[(7, 9), (5, 5)])
    pack, t = _pack_and_inputs(inp)
    other = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, "bf16",
                     rope_theta=500.0)
    assert other.plan.fingerprint != pack.plan.fingerprint
    assert other.blob_dev.numel() == pack.blob_dev.numel()
    N, H, d = pack.N, pack.H, pack.d
    HD = H * d
    canary = lambda shape, dt: torch.full(shape, 7.0, dtype=dt, device="cuda")
    outs = dict(o=canary((N, H, d), torch.bfloat16), lse=canary((H, N), torch.float32),
                q_hat=canary((N, H, d), torch.bfloat16), k_hat=canary((N, H, d), torch.bfloat16),
                rstd=canary((2, N, H), torch.float32))
    fa = dict(q=t["q"], k=t["k"], v=t["v"], q_stride=HD, k_stride=HD, v_stride=HD, gains=t["gains"])
    pam.mmdit_attn_fwd(pack.plan, other.blob_dev, **fa, **outs)
    grads = dict(dq=canary((N, H, d), torch.bfloat16), dk=canary((N, H, d), torch.bfloat16),
                 dv=canary((N, H, d), torch.bfloat16), dgains=canary((4, d), torch.float32))
    ws = pack.workspace("bwd")
    ba = dict(q=t["q"], k=t["k"], v=t["v"], q_hat=outs["q_hat"], k_hat=outs["k_hat"], o=outs["o"],
              dout=t["dout"], q_stride=HD, k_stride=HD, v_stride=HD, dout_stride=HD, gains=t["gains"],
              lse=outs["lse"], rstd=outs["rstd"], workspace=ws)
    pam.mmdit_attn_bwd(pack.plan, other.blob_dev, **ba, **grads)
    faults = pam.mmdit_device_faults()
    _say(f"   faults with another pack's blob: {faults:#x}")
    assert faults == pam.DEVICE_FAULT_STALE_BLOB
    for n, x in list(outs.items()) + list(grads.items()):
        assert bool((x == 7.0).all()), f"{n} was written with another pack's blob"
    assert pam.mmdit_device_faults() == 0  # the read cleared it
    pam.mmdit_attn_fwd(pack.plan, pack.blob_dev, **fa, **outs)
    pam.mmdit_attn_bwd(pack.plan, pack.blob_dev, **ba, **grads)
    assert pam.mmdit_device_faults() == 0
    ref = run_oracle(inp)
    fails = []
    for key in ("o", "dq", "dk", "dv"):
        src = outs if key == "o" else grads
        _, msg = check(key, src[key].double().cpu().numpy(), ref[key], "bf16", failures=fails)
        _say("   " + msg)
    assert not fails, fails


def test_explicit_side_stream():
    """forward / backward / adaLN with stream= a side stream that is not the
    current one: outputs and workspaces are allocated on it and the results
    equal the default stream's bit for bit."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(86, heads=3, head_dim=128, dtype="bf16",
                                text=[45, 3], grids=[(13, 11), (2, 5)])
    pack, t = _pack_and_inputs(inp)
    ref_f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    ref_b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], ref_f, t["dout"])
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"], stream=side)
    b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], f, t["dout"], stream=side)
    side.synchronize()
    for k in ("o", "lse", "q_hat", "k_hat"):
        assert torch.equal(f[k], ref_f[k]), k
    for k in ("dq", "dk", "dv", "dgains"):
        assert torch.equal(b[k], ref_b[k]), k
    # a raw stream handle works the same way
    f2 = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"], stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(f2["o"], ref_f["o"])


def test_fault_injection_hook_on_the_gpu(monkeypatch):
    """With MMDIT_FAULT_INJECT=launch the calls fail with MMDIT_ERR_HIP and
    write nothing; with the variable cleared, the same calls in the same
    process give the results of a run before it was set."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(3, heads=2, head_dim=128, dtype="bf16", text=[21, 0], grids=[(6, 11), (9, 4)])
    _say(f"fault injection N={inp.num_tokens}")
    pack, t = _pack_and_inputs(inp)
    ref = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    refb = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], ref, t["dout"])
    torch.cuda.synchronize()
    monkeypatch.setenv("MMDIT_FAULT_INJECT", "launch")
    o = torch.full_like(ref["o"], 3.0)
    with pytest.raises(pam.MmditError) as e:
        pam.mmdit_attn_fwd(pack.plan, pack.blob_dev, q=t["q"], k=t["k"], v=t["v"], q_stride=pack.H * pack.d,
                           k_stride=pack.H * pack.d, v_stride=pack.H * pack.d, gains=t["gains"], o=o,
                           lse=torch.empty_like(ref["lse"]), q_hat=torch.empty_like(ref["q_hat"]),
                           k_hat=torch.empty_like(ref["k_hat"]), rstd=torch.empty_like(ref["rstd"]))
    assert e.value.status == 5 and "MMDIT_FAULT_INJECT" in str(e.value)
    with pytest.raises(pam.MmditError):
        pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], ref, t["dout"])
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()), "a call with an injected fault wrote its output"
    monkeypatch.delenv("MMDIT_FAULT_INJECT")
    f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], f, t["dout"])
    torch.cuda.synchronize()
    assert torch.equal(f["o"], ref["o"]) and torch.equal(b["dq"], refb["dq"]) and torch.equal(b["dgains"], refb["dgains"])
