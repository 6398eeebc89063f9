"""Packed classifier-free guidance on the GPU: one pack holding the
conditional samples and their unconditional twins (same latent grids, a null
prompt of null_text_len tokens) is one forward pass whose rows equal, bit for
bit, the two branches run as separate packs, and match the oracle. Marked
``gpu``: needs an MI355X and the built library."""
import sys

import numpy as np
import pytest

import workloads
from parity import check, run_gpu, run_oracle, subset_samples

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROW_KEYS = ("o", "q_hat", "k_hat", "lse", "rstd_q", "rstd_k")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_attention_nr_amd as pam
    pam.lib()  # must load: no fallback


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cfg_inputs(seed, text, grids, null_text_len, heads, d, dtype):
    import packed_attention_nr_amd as pam
    t, h, w = pam.mmdit_cfg_pack_desc(text, [g[0] for g in grids], [g[1] for g in grids], null_text_len)
    return workloads.random_pack(seed, heads=heads, head_dim=d, dtype=dtype, backward=False,
                                 text=t.tolist(), grids=list(zip(h.tolist(), w.tolist())))


def _branches_match(inp, full, S):
    for name, order in (("conditional", list(range(S))), ("unconditional", list(range(S, 2 * S)))):
        sub, rows = subset_samples(inp, order)
        alone = run_gpu(sub, backward=False)
        bad = [k for k in ROW_KEYS if not np.array_equal(full[k][rows], alone[k])]
        assert not bad, f"{name} branch differs from its rows in the packed pass: {bad}"


@pytest.mark.parametrize("null_text_len", [0, 9])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_cfg_pack_matches_oracle_and_branches(null_text_len, dtype, d):
    text = [37, 0, 120]
    grids = [(9, 7), (5, 5), (12, 3)]
    inp = _cfg_inputs(21, text, grids, null_text_len, 3, d, dtype)
    S = len(text)
    _say(f"cfg {dtype} d={d} null={null_text_len} L={inp.seqlens().tolist()}")
    assert inp.text_len[S:].tolist() == [null_text_len] * S
    assert inp.grid_h[S:].tolist() == [g[0] for g in grids]
    full = run_gpu(inp, backward=False)
    ref = run_oracle(inp, backward=False)
    fails = []
    for k in ("q_hat", "k_hat", "o", "rstd_q", "rstd_k"):
        _, msg = check(k, full[k], ref[k], inp.dtype, failures=fails)
        _say("   " + msg)
    e = np.max(np.abs(full["lse"] - ref["lse"]))
    if e > (2e-2 if dtype == "bf16" else 1e-5 * np.max(np.abs(ref["lse"]))):
        fails.append(f"lse max_abs {e:.3e}")
    assert not fails, fails
    _branches_match(inp, full, S)


def test_cfg_pack_1024_branches_bitwise():
    """The 1024^2 generation sample (512 text tokens + 64x64 latents, H=24,
    d=128) with an empty-prompt twin, as one pass and as two."""
    inp = _cfg_inputs(3, [512], [(64, 64)], 0, 24, 128, "bf16")
    _say(f"cfg 1024^2 N={inp.num_tokens} L={inp.seqlens().tolist()}")
    full = run_gpu(inp, backward=False)
    _branches_match(inp, full, 1)
