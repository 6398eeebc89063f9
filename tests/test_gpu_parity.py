"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Marked ``gpu``: needs an MI355X and the built library."""
import dataclasses
import sys

import numpy as np
import pytest

import workloads
from parity import check, run_gpu, run_oracle, subset_heads

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


def _compare(inp, gpu, ref, heads=None, backward=True, extra=()):
    """Check every output of the oracle against the GPU's (on `heads`)."""
    hs = slice(None) if heads is None else list(heads)
    fails = []
    keys = ["q_hat", "k_hat", "o", "rstd_q", "rstd_k"] + list(extra)
    if backward and inp.dout is not None:
        keys += ["dv", "dq", "dk"]
        if heads is None:
            keys += ["dgains"]
    for k in keys:
        g = gpu[k] if k == "dgains" else gpu[k][:, hs]
        ok, msg = check(k, g, ref[k], inp.dtype, l2_only=(k == "dgains"), failures=fails)
        _say("   " + msg)
    # lse: natural-log logsumexp, absolute error (bf16) / normwise (fp32)
    e = np.max(np.abs(gpu["lse"][:, hs] - ref["lse"]))
    _say(f"   lse: max_abs={e:.3e}")
    if e > (2e-2 if inp.dtype == "bf16" else 1e-5 * np.max(np.abs(ref["lse"]))):
        fails.append(f"lse max_abs {e:.3e}")
    assert not fails, fails


# ---------------------------------------------------------------------------
# small packs: every output, all heads
# ---------------------------------------------------------------------------
EDGE_PACKS = {
    "one_token_samples": dict(text=[1, 0, 1], grids=[(0, 0), (1, 1), (0, 0)]),
    "text_only_and_image_only": dict(text=[37, 0], grids=[(0, 0), (9, 7)]),
    "exact_tiles": dict(text=[64, 0], grids=[(8, 8), (16, 8)]),
    "ragged_multi_tile": dict(text=[45, 3, 130], grids=[(13, 11), (2, 5), (7, 19)]),
    "wide_4to1": dict(text=[20], grids=[(8, 32)]),
    "tile_plus_one": dict(text=[1], grids=[(16, 8)]),
    "single_token_pack": dict(text=[1], grids=[(0, 0)]),
    "single_pixel_pack": dict(text=[0], grids=[(1, 1)]),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(EDGE_PACKS))
def test_edge_packs(case, d, dtype):
    spec = EDGE_PACKS[case]
    inp = workloads.random_pack(sorted(EDGE_PACKS).index(case), heads=3, head_dim=d, dtype=dtype,
                                text=spec["text"], grids=spec["grids"])
    _say(f"edge pack {case} d={d} {dtype} N={inp.num_tokens}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("mode", ["recompute", "stored_ds"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["one_token_samples", "exact_tiles", "ragged_multi_tile", "wide_4to1"])
def test_backward_modes(case, d, mode):
    """Both bf16 backward modes at both head sizes: dQ with S and dP formed
    again per query tile (the default), and dQ from the dS that the dK/dV
    kernel stores (selected by the stored-dS flag). The other cases run the
    default."""
    spec = EDGE_PACKS[case]
    inp = workloads.random_pack(40 + sorted(EDGE_PACKS).index(case), heads=3, head_dim=d, dtype="bf16",
                                text=spec["text"], grids=spec["grids"])
    _say(f"backward {mode} {case} d={d} N={inp.num_tokens}")
    _compare(inp, run_gpu(inp, bwd_mode=mode), run_oracle(inp))


def test_stored_ds_stage_calls_match_one_call():
    """The stored-dS backward as separate stage calls (D, dK/dV, dQ, gains,
    each with the mode flag) gives bitwise the results of one call."""
    import packed_attention_nr_amd as pam
    from parity import to_device
    inp = workloads.random_pack(23, heads=2, head_dim=128, dtype="bf16",
                                text=[45, 3, 130], grids=[(13, 11), (2, 5), (7, 19)])
    _say(f"stored-dS stage calls N={inp.num_tokens}")
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, "bf16")
    assert pack.plan.bwd_ds_workspace_bytes > pack.plan.bwd_workspace_bytes
    t = to_device(inp)
    saved = pam.forward(pack, t["q"], t["k"], t["v"], t["gains"])
    one = pam.backward(pack, t["q"], t["k"], t["v"], t["gains"], saved, t["dout"], mode="stored_ds")
    N, H, d = pack.N, pack.H, pack.d
    out = {n: torch.empty_like(one[n]) for n in ("dq", "dk", "dv", "dgains")}
    ws = pack.workspace("bwd_ds")
    B = pam.BWD_STAGES
    for st in (B["d"] | B["store_ds"], B["dkdv"] | B["store_ds"], B["dq"] | B["store_ds"], B["gains"]):
        pam.mmdit_attn_bwd(pack.plan, pack.blob_dev, q=t["q"], k=t["k"], v=t["v"], q_hat=saved["q_hat"],
                           k_hat=saved["k_hat"], o=saved["o"], dout=t["dout"], q_stride=H * d,
                           k_stride=H * d, v_stride=H * d, dout_stride=H * d, gains=t["gains"],
                           lse=saved["lse"], rstd=saved["rstd"], workspace=ws, stages=st, **out)
    torch.cuda.synchronize()
    for n in out:
        assert torch.equal(out[n], one[n]), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_random_packs(seed, dtype):
    inp = workloads.random_pack(100 + seed, max_samples=6, max_text=300, max_side=24,
                                heads=2, head_dim=128 if seed % 2 else 64, dtype=dtype)
    _say(f"random pack seed={seed} {dtype} d={inp.head_dim} N={inp.num_tokens} "
         f"L={inp.seqlens().tolist()}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_many_heads(dtype, d):
    """40 heads (token stride 40*d): head-indexed strides, block maps and the
    gain-gradient sums over more heads than the workloads use."""
    inp = workloads.random_pack(17, heads=40, head_dim=d, dtype=dtype,
                                text=[33, 7], grids=[(9, 10), (4, 4)])
    _say(f"many heads {dtype} d={d} N={inp.num_tokens}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


def test_largest_grid_sides():
    """Grid sides of 32,767 (the largest the packing accepts): a 1 x 32767
    strip after 5 text tokens and a 32767 x 1 column, so row and column
    indices reach their 15-bit maximum in the token words and the RoPE table
    has 32,767 rows. One head, d = 64, bf16, forward and backward."""
    inp = workloads.random_pack(11, heads=1, head_dim=64, dtype="bf16",
                                text=[5, 0], grids=[(1, 32767), (32767, 1)])
    _say(f"largest grid sides N={inp.num_tokens} L={inp.seqlens().tolist()}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


SCORE_PATTERNS = ("jump", "ramp_up", "gentle", "ramp_down", "random")


def _score_pattern_pack(d, seed=5):
    """Text-only samples (no RoPE) of 401 tokens whose scores follow a chosen
    course along the keys, in one pack: q and k rows are +-1 vectors and all
    gains equal g, so Q-hat and K-hat are +-g up to a relative 5e-7 (exactly
    +-g once rounded to bf16) and every score g^2 (d - 2 f) is exact in fp32,
    f being the number of sign flips between the query and the key. Per head,
    every query is a base vector u with 0..3 flips; key j of a sample has f_j
    flips of u:
      jump      - the first 64 keys are -u, the rest have 0..6 flips: the later
                  scores exceed the first tile's by ~150 (log2 units), past
                  the fp32 range of exp2;
      ramp_up   - f from d down to 0: the maximum rises by ~26 per 64 keys;
      gentle    - f from d/2 + a down to d/2 - a: a rise of 5..8 over the
                  sample, so later keys weigh up to ~2^7 against the first;
      ramp_down - f from 0 up to d: the first keys hold the maximum;
      random    - f uniform in 0..d.
    g = 2.25 (d = 128) or 2.75 (d = 64) makes 1 unit of s_int = d - 2f worth
    0.65 or 1.36 in log2 units."""
    T = 401
    S = len(SCORE_PATTERNS)
    g = 2.25 if d == 128 else 2.75
    inp = workloads.random_pack(seed, heads=2, head_dim=d, dtype="bf16", backward=False,
                                text=[T] * S, grids=[(0, 0)] * S)
    rng = np.random.default_rng(seed + 1000)
    H = inp.heads
    j = np.arange(T)
    a = 3 if d == 128 else 1
    flips = {
        "jump": np.where(j < 64, d, rng.integers(0, 7, T)),
        "ramp_up": np.rint(d * (1 - j / (T - 1))),
        "gentle": np.rint(d / 2 + a - 2 * a * j / (T - 1)),
        "ramp_down": np.rint(d * j / (T - 1)),
        "random": rng.integers(0, d + 1, T),
    }
    q = np.empty_like(inp.q)
    k = np.empty_like(inp.k)

    def flipped(u, f):
        x = u.copy()
        x[rng.permutation(d)[:int(f)]] *= -1
        return x

    for h in range(H):
        u = rng.choice([-1.0, 1.0], d).astype(np.float32)
        for i, name in enumerate(SCORE_PATTERNS):
            for t in range(T):
                q[i * T + t, h] = flipped(u, rng.integers(0, 4))
                k[i * T + t, h] = flipped(u, flips[name][t])
    gains = np.full_like(inp.gains, g)
    return dataclasses.replace(inp, q=q, k=k, gains=gains)


@pytest.mark.parametrize("d", [64, 128])
def test_score_patterns(d):
    """The forward's running reference (P formed against the current one, kept
    while P stays bounded, the reference raised from the row maxima otherwise)
    on scores that jump past exp2's range, climb steeply or gently, fall, or
    scatter: Q-hat, K-hat, O and lse against the oracle. Forward only: with
    these keys a gradient is the small remainder of hundreds of near-parallel
    terms, and a key that takes the weight of all 401 queries gets a dV near 20
    whose bf16 rounding alone passes the absolute bar; the backward reads the
    forward only through the lse checked here."""
    inp = _score_pattern_pack(d)
    _say(f"score patterns d={d} N={inp.num_tokens} {SCORE_PATTERNS}")
    _compare(inp, run_gpu(inp, backward=False), run_oracle(inp, backward=False), backward=False)


INFER_PACKS = [
    ("ragged_multi_tile", 128, dict(text=[45, 3, 130], grids=[(13, 11), (2, 5), (7, 19)]), None),
    ("wide_4to1", 64, dict(text=[20], grids=[(8, 32)]), None),
    ("edit_mixed", 128, dict(text=[20, 0, 64], grids=[(5, 5), (8, 16), (3, 3)]),
     [(0, 0), (16, 8), (11, 2)]),
]


@pytest.mark.parametrize("name,d,spec,src", INFER_PACKS, ids=[c[0] for c in INFER_PACKS])
def test_inference_forward_in_workspace(name, d, spec, src):
    """A bf16 forward that keeps no Q-hat / K-hat (they live in the caller's
    workspace): O and lse against the oracle, and bit for bit against the
    forward that stores them."""
    import packed_attention_nr_amd as pam
    inp = workloads.random_pack(31, heads=3, head_dim=d, dtype="bf16", backward=False,
                                text=spec["text"], grids=spec["grids"], src=src)
    _say(f"inference forward {name} d={d} N={inp.num_tokens}")
    pack = pam.Pack(inp.text_len, inp.grid_h, inp.grid_w, inp.heads, inp.head_dim, "bf16",
                    src_h=inp.src_h, src_w=inp.src_w)
    up = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    gains = torch.from_numpy(inp.gains).cuda()
    inf = pam.forward(pack, q, k, v, gains, save_for_backward=False)
    trn = pam.forward(pack, q, k, v, gains, save_for_backward=True)
    torch.cuda.synchronize()
    ref = run_oracle(inp, backward=False)
    fails = []
    o = inf["o"].double().cpu().numpy()
    _, msg = check("o (workspace)", o, ref["o"], "bf16", failures=fails)
    _say("   " + msg)
    e = float(np.max(np.abs(inf["lse"].double().cpu().numpy().T - ref["lse"])))
    _say(f"   lse (workspace): max_abs={e:.3e}")
    if e > 2e-2:
        fails.append(f"lse {e:.3e}")
    for key in ("o", "lse"):
        if not torch.equal(inf[key], trn[key]):
            fails.append(f"{key} differs between the workspace and the stored forward")
    assert not fails, fails


def test_tiny_fp32_workload():
    inp = workloads.draw("tiny_fp32")
    _say(f"tiny_fp32 N={inp.num_tokens}")
    _compare(inp, run_gpu(inp, backward=False), run_oracle(inp, backward=False))


# ---------------------------------------------------------------------------
# full-size workloads: complete outputs for a subset of heads; the gain
# gradients (sums over all heads) from a second GPU run on just those heads,
# whose per-head outputs must equal the full run's bit for bit
# ---------------------------------------------------------------------------
FULL = [("gen1024", [0, 11, 23]), ("mixed6", [0, 13, 22]), ("gen2048", [5, 11, 18]), ("small64", [0, 9, 23]),
        ("edit1024", [0, 17])]


STORED_DS_FULL = [("mixed6", [5, 19]), ("edit1024", [7]), ("small64", [3, 20]), ("gen2048", [2, 21])]


@pytest.mark.parametrize("name,heads", STORED_DS_FULL, ids=[c[0] for c in STORED_DS_FULL])
def test_full_workload_stored_ds(name, heads):
    """The stored-dS backward at full size against the oracle on sampled heads:
    the mixed-resolution pack (3.6 GiB of dS), the editing step, the 64-segment
    pack (4.1 GiB: per-(sample, head) areas at byte offsets past 4 GiB, 64
    samples of area bases) and the 2048^2 sample (12.8 GiB: one 16,896-token
    segment, the largest dS area per head; heads 2 and 21 put the checked
    areas near both ends of the buffer). The gain gradients through a
    head-subset run in the same mode, whose per-head outputs must equal the
    full run's bit for bit; and the recompute backward's dV bit for bit (dV
    does not depend on D, which the two modes sum in different orders; the
    kernel differs only in also storing dS)."""
    inp = workloads.draw(name)
    _say(f"{name} stored dS: N={inp.num_tokens} H={inp.heads} heads checked={heads}")
    gpu = run_gpu(inp, bwd_mode="stored_ds")
    ref = run_oracle(inp, heads=heads)
    _compare(inp, gpu, ref, heads=heads)
    sub = run_gpu(subset_heads(inp, heads), bwd_mode="stored_ds")
    fails = []
    _, msg = check("dgains (checked heads only)", sub["dgains"], ref["dgains"], inp.dtype,
                   l2_only=True, failures=fails)
    _say("   " + msg)
    for k in ("o", "dq", "dk", "dv"):
        if not np.array_equal(sub[k], gpu[k][:, heads]):
            fails.append(f"{k} differs between the full and the head-subset run")
    del sub
    rec = run_gpu(inp, bwd_mode="recompute")
    if not np.array_equal(gpu["dv"], rec["dv"]):
        fails.append("dv differs from the recompute backward's")
    assert not fails, fails


@pytest.mark.parametrize("name,heads", FULL, ids=[f[0] for f in FULL])
def test_full_workload(name, heads):
    w = workloads.get(name)
    inp = workloads.draw(name)
    _say(f"{name}: N={inp.num_tokens} H={inp.heads} heads checked={heads}")
    gpu = run_gpu(inp, backward=w.backward)
    ref = run_oracle(inp, heads=heads, backward=w.backward)
    _compare(inp, gpu, ref, heads=heads, backward=w.backward)
    if w.backward:
        sub = run_gpu(subset_heads(inp, heads))
        fails = []
        _, msg = check("dgains (checked heads only)", sub["dgains"], ref["dgains"], inp.dtype,
                       l2_only=True, failures=fails)
        _say("   " + msg)
        for k in ("o", "dq", "dk", "dv"):
            same = np.array_equal(sub[k], gpu[k][:, heads])
            _say(f"   {k}: head-subset run bitwise equal: {same}")
            if not same:
                fails.append(f"{k} differs between the full and the head-subset run")
        assert not fails, fails
