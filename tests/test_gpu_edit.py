"""Editing packs on the GPU (3D RoPE: each sample's source latents follow its
target latents on a second frame): every output of the HIP path against the
oracle on small packs, generation samples mixed into editing packs, and each
sample's rows equal, bit for bit, to that sample run alone. Marked ``gpu``:
needs an MI355X and the built library."""
import sys

import numpy as np
import pytest

import workloads
from parity import check, run_gpu, run_oracle, subset_samples

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


def _compare(inp, gpu, ref):
    fails = []
    for k in ("q_hat", "k_hat", "o", "rstd_q", "rstd_k", "dv", "dq", "dk", "dgains"):
        _, msg = check(k, gpu[k], ref[k], inp.dtype, l2_only=(k == "dgains"), failures=fails)
        _say("   " + msg)
    e = np.max(np.abs(gpu["lse"] - ref["lse"]))
    _say(f"   lse: max_abs={e:.3e}")
    if e > (2e-2 if inp.dtype == "bf16" else 1e-5 * np.max(np.abs(ref["lse"]))):
        fails.append(f"lse max_abs {e:.3e}")
    assert not fails, fails


EDIT_PACKS = {
    # one edit, target and source of different shapes, several tiles, ragged
    "edit_two_shapes": dict(text=[37], grids=[(9, 7)], src=[(7, 9)]),
    # generation samples (no source) packed with edits
    "mixed_generation_and_edit": dict(text=[20, 0, 64], grids=[(5, 5), (8, 16), (3, 3)],
                                      src=[(0, 0), (16, 8), (11, 2)]),
    # 128 + 1 tokens: one full tile and a one-token tail, which is the source
    "source_is_the_tail": dict(text=[0], grids=[(16, 8)], src=[(1, 1)]),
    # text-only sample beside an edit with equal target and source grids
    "text_only_beside_edit": dict(text=[45, 3], grids=[(0, 0), (6, 6)], src=[(0, 0), (6, 6)]),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", sorted(EDIT_PACKS))
def test_edit_packs(case, d, dtype):
    spec = EDIT_PACKS[case]
    inp = workloads.random_pack(40 + sorted(EDIT_PACKS).index(case), heads=3, head_dim=d,
                                dtype=dtype, text=spec["text"], grids=spec["grids"],
                                src=spec["src"])
    _say(f"edit pack {case} d={d} {dtype} N={inp.num_tokens} L={inp.seqlens().tolist()}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(4))
def test_random_edit_packs(seed, dtype):
    inp = workloads.random_pack(200 + seed, max_samples=5, max_text=200, max_side=20, heads=2,
                                head_dim=64 if seed % 2 else 128, dtype=dtype, edit=True)
    _say(f"random edit pack seed={seed} {dtype} d={inp.head_dim} N={inp.num_tokens} "
         f"L={inp.seqlens().tolist()} src={list(zip(inp.src_h.tolist(), inp.src_w.tolist()))}")
    _compare(inp, run_gpu(inp), run_oracle(inp))


def test_edit_samples_alone_bitwise():
    """Each sample of a mixed editing pack, run as a pack of its own, gives
    the same bits as its rows in the pack (forward and input gradients)."""
    spec = EDIT_PACKS["mixed_generation_and_edit"]
    inp = workloads.random_pack(7, heads=2, head_dim=128, dtype="bf16", text=spec["text"],
                                grids=spec["grids"], src=spec["src"])
    full = run_gpu(inp)
    for i in range(len(spec["text"])):
        sub, rows = subset_samples(inp, [i])
        alone = run_gpu(sub)
        bad = [k for k in ("o", "q_hat", "k_hat", "lse", "dq", "dk", "dv")
               if not np.array_equal(full[k][rows], alone[k])]
        _say(f"   sample {i}: {'bitwise equal' if not bad else bad}")
        assert not bad, (i, bad)
