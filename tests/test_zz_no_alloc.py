"""GPU test of mmdit_attn_bwd_noalloc, the backward for callers that cannot
allocate device memory: through the C ABI, against mmdit_attn_bwd (recompute
mode, caller workspace) bit for bit, on two calls in a row with the second on a
smaller pack, and stage by stage. Collected last (its library-owned workspace
persists across calls on the GPU)."""
import sys

import numpy as np
import pytest

import workloads
from parity import check, run_oracle, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_attention_nr_amd as pam
    pam.lib()  # must load: no fallback


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _both(inp, stage_calls=None):
    """Forward once, then the backward with the caller workspace and with the
    library's own; returns the two gradient dicts (torch tensors)."""
    import packed_attention_nr_amd as pam
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, inp.dtype)
    t = to_device(inp)
    saved = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    ref = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], saved, t["dout"],
                       workspace=pack.workspace("bwd"))
    out = {n: torch.full_like(ref[n], float("nan")) for n in ("dq", "dk", "dv", "dgains")}
    N, H, d = pack.N, pack.H, pack.d
    args = dict(q=t["q"], k=t["k"], v=t["v"], q_hat=saved["q_hat"], k_hat=saved["k_hat"],
                o=saved["o"], dout=t["dout"], q_stride=H * d, k_stride=H * d, v_stride=H * d,
                dout_stride=H * d, gains=t["gains"], lse=saved["lse"], rstd=saved["rstd"], **out)
    for st in stage_calls or [0]:
        pam.mmdit_attn_bwd_noalloc(pack.plan, pack.blob_dev, stages=st, **args)
    torch.cuda.synchronize()
    return ref, out, pack


def _same(ref, out, label):
    for n in ("dq", "dk", "dv", "dgains"):
        same = torch.equal(ref[n], out[n])
        _say(f"   {label} {n}: bitwise equal to mmdit_attn_bwd: {same}")
        assert same, (label, n)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_noalloc_matches_workspace_backward(dtype, d):
    """Two calls in a row, the second on a smaller pack: each equals
    mmdit_attn_bwd bit for bit, and the larger one also meets the oracle's
    tolerances."""
    big = workloads.random_pack(71, heads=3, head_dim=d, dtype=dtype,
                                text=[45, 3, 130, 0], grids=[(13, 11), (2, 5), (7, 19), (16, 16)])
    small = workloads.random_pack(72, heads=2, head_dim=d, dtype=dtype,
                                  text=[9, 1], grids=[(3, 4), (0, 0)])
    _say(f"no-alloc backward {dtype} d={d}: first N={big.num_tokens}, then N={small.num_tokens}")
    ref, out, _ = _both(big)
    _same(ref, out, "first call")
    orc = run_oracle(big)
    fails = []
    for n in ("dq", "dk", "dv"):
        _, msg = check(n, out[n].double().cpu().numpy(), orc[n], dtype, failures=fails)
        _say("   oracle " + msg)
    _, msg = check("dgains", out["dgains"].double().cpu().numpy(), orc["dgains"], dtype,
                   l2_only=True, failures=fails)
    _say("   oracle " + msg)
    assert not fails, fails
    ref2, out2, _ = _both(small)
    _same(ref2, out2, "second call (smaller pack)")


def test_noalloc_stage_calls():
    """The stages as separate calls (DQ, then DKDV, then GAINS): the array
    keeps the D and the partials of the calls before."""
    import packed_attention_nr_amd as pam
    B = pam.BWD_STAGES
    inp = workloads.random_pack(73, heads=2, head_dim=128, dtype="bf16",
                                text=[20, 64], grids=[(9, 9), (8, 16)])
    _say(f"no-alloc backward stage by stage N={inp.num_tokens}")
    ref, out, _ = _both(inp, stage_calls=[B["dq"], B["dkdv"], B["gains"]])
    _same(ref, out, "stage calls")


def test_noalloc_full_size_mixed_pack():
    """The mixed-resolution training pack (20,436 tokens, 24 heads, a 7.7 MiB
    workspace) against mmdit_attn_bwd, bit for bit."""
    inp = workloads.draw("mixed6")
    _say(f"no-alloc backward mixed6 N={inp.num_tokens}")
    ref, out, pack = _both(inp)
    assert pack.plan.bwd_workspace_bytes <= 64 << 20
    _same(ref, out, "mixed6")
