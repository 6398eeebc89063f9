"""Invariants of the HIP path that hold bit for bit at any size: repeated
runs agree; samples do not interact, so a sample alone or in another pack
order gives the same rows; changing one sample changes only its own rows;
q, k, v given as views into a fused [N][3][H][d] tensor give the dense
inputs' results. Marked ``gpu``: needs an MI355X and the built library."""
import sys

import numpy as np
import pytest

import workloads
from parity import run_gpu, subset_samples

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROW_KEYS = ("o", "q_hat", "k_hat", "lse", "rstd_q", "rstd_k", "dq", "dk", "dv")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_attention_nr_amd as pam
    pam.lib()  # must load: no fallback


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pack(seed, dtype, d=128):
    return workloads.random_pack(seed, max_samples=5, max_text=200, max_side=20, heads=3,
                                 head_dim=d, dtype=dtype)


def _same_rows(a, b, rows_a, rows_b, keys=ROW_KEYS):
    bad = []
    for k in keys:
        if not np.array_equal(a[k][rows_a], b[k][rows_b]):
            bad.append(k)
    return bad


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_repeat_runs_bitwise(dtype):
    inp = _pack(11, dtype)
    _say(f"repeat {dtype} N={inp.num_tokens} L={inp.seqlens().tolist()}")
    a, b = run_gpu(inp), run_gpu(inp)
    bad = [k for k in a if not np.array_equal(a[k], b[k])]
    assert not bad, f"outputs differ between identical runs: {bad}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_alone_matches_pack(dtype):
    inp = _pack(12, dtype)
    S = len(inp.text_len)
    _say(f"alone {dtype} N={inp.num_tokens} L={inp.seqlens().tolist()}")
    full = run_gpu(inp)
    for i in range(S):
        sub, rows = subset_samples(inp, [i])
        alone = run_gpu(sub)
        bad = _same_rows(full, alone, rows, slice(None))
        assert not bad, f"sample {i} alone differs from its rows in the pack: {bad}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pack_order_permutes_rows(dtype):
    inp = _pack(13, dtype)
    S = len(inp.text_len)
    order = list(range(S))[::-1]
    _say(f"permute {dtype} N={inp.num_tokens} order={order}")
    full = run_gpu(inp)
    perm, rows = subset_samples(inp, order)
    out = run_gpu(perm)
    bad = _same_rows(full, out, rows, slice(None))
    assert not bad, f"reordered pack differs: {bad}"
    # the gain gradients are sums over all tokens: same up to summation order
    assert np.allclose(full["dgains"], out["dgains"], rtol=1e-4, atol=1e-3)


def test_changing_one_sample_leaves_the_others():
    inp = workloads.random_pack(14, heads=3, head_dim=128, dtype="bf16",
                                text=[40, 100, 7], grids=[(9, 13), (5, 5), (12, 3)])
    S = len(inp.text_len)
    full = run_gpu(inp)
    off = np.concatenate([[0], np.cumsum(inp.seqlens())])
    j = S // 2
    v2 = inp.v.copy()
    v2[off[j]:off[j + 1]] = workloads.bf16_round(v2[off[j]:off[j + 1]] * 0.5 + 0.25)
    import dataclasses
    out = run_gpu(dataclasses.replace(inp, v=v2))
    others = np.concatenate([np.arange(off[i], off[i + 1]) for i in range(S) if i != j])
    own = np.arange(off[j], off[j + 1])
    bad = _same_rows(full, out, others, others)
    assert not bad, f"rows of untouched samples changed: {bad}"
    assert not np.array_equal(full["o"][own], out["o"][own]), "the changed sample's output did not change"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_qkv_views_match_dense(dtype):
    import packed_attention_nr_amd as pam
    inp = _pack(15, dtype)
    N, H, d = inp.num_tokens, inp.heads, inp.head_dim
    dense = run_gpu(inp)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qkv = torch.empty((N, 3, H, d), dtype=dt, device="cuda")
    for i, a in enumerate((inp.q, inp.k, inp.v)):
        qkv[:, i] = torch.from_numpy(a).to(device="cuda", dtype=dt)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    gains = torch.from_numpy(inp.gains).to("cuda")
    dout = torch.from_numpy(inp.dout).to(device="cuda", dtype=dt)
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, H, d, dtype, inp.rope_theta, inp.rms_eps,
                    device="cuda")
    saved = pam.forward(pack, q, k, v, gains)
    g = pam.backward(pack, q, k, v, gains, saved, dout)
    torch.cuda.synchronize()
    host = lambda t: t.detach().to(torch.float64).cpu().numpy()
    got = {"o": host(saved["o"]), "dq": host(g["dq"]), "dk": host(g["dk"]), "dv": host(g["dv"]),
           "dgains": host(g["dgains"])}
    bad = [k for k in got if not np.array_equal(got[k], dense[k])]
    assert not bad, f"strided views differ from dense inputs: {bad}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_side_stream_matches_default_stream(dtype):
    """Forward and backward enqueued on a side stream (default priority) give
    the default stream's bits: every launch goes to the caller's stream."""
    import packed_attention_nr_amd as pam
    from parity import to_device
    inp = _pack(15, dtype)
    _say(f"side stream {dtype} N={inp.num_tokens}")
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, dtype)
    t = to_device(inp)
    ref_f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    ref_b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], ref_f, t["dout"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
        b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], f, t["dout"])
    side.synchronize()
    bad = [k for k in f if not torch.equal(f[k], ref_f[k])]
    bad += [k for k in ("dq", "dk", "dv", "dgains") if not torch.equal(b[k], ref_b[k])]
    assert not bad, bad


def test_graph_capture_replays_match_eager():
    """Forward + backward captured in one HIP graph (the library allocates,
    clears and synchronises nothing, so its launches are capturable) and
    replayed three times, with eager work and synchronisation between the
    replays: every replay gives the eager bits."""
    import packed_attention_nr_amd as pam
    from parity import to_device
    inp = _pack(16, "bf16")
    _say(f"graph capture N={inp.num_tokens}")
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, "bf16")
    t = to_device(inp)
    eager_f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    eager_b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], eager_f, t["dout"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
        b = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], f, t["dout"])
    for rep in range(3):
        for k in ("o", "lse"):  # clobber the outputs so each replay must rewrite them
            f[k].fill_(float("nan"))
        for k in ("dq", "dk", "dv", "dgains"):
            b[k].fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda") * 2.0  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = [k for k in ("o", "lse", "q_hat", "k_hat", "rstd") if not torch.equal(f[k], eager_f[k])]
        bad += [k for k in ("dq", "dk", "dv", "dgains") if not torch.equal(b[k], eager_b[k])]
        _say(f"   replay {rep}: {'bitwise equal' if not bad else bad} (noise {float(noise.sum()):.1f})")
        assert not bad, (rep, bad)
