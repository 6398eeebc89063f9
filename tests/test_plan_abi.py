"""CPU tests of the C ABI: symbols, the host pack plan (checked against the
oracle's independent layout), and argument validation (invalid calls must
return their status code before anything is launched)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import workloads

pam = pytest.importorskip("packed_attention_nr_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    try:
        return pam.lib()
    except ImportError as e:
        pytest.fail(f"libmmdit.so must be built before the tests: {e}")


def test_exports_every_header_symbol(L):
    import glob
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        names |= set(re.findall(r"\b(mmdit_[a-z_]+)\s*\(", open(h).read()))
    assert {"mmdit_pack_plan", "mmdit_attn_fwd", "mmdit_attn_bwd", "mmdit_attn_bwd_noalloc",
            "mmdit_device_faults", "mmdit_probe_mfma", "mmdit_probe_streams"} <= names
    for n in sorted(names):
        assert hasattr(L, n), n
    assert pam.mmdit_abi_version() == pam.ABI_VERSION == 5
    assert pam.mmdit_status_str(0) == "ok"


def _blob_section(blob, off, n, dtype):
    return np.frombuffer(blob[off:off + n * np.dtype(dtype).itemsize].tobytes(), dtype=dtype)


def _check_plan(inp, dtype_code):
    H, d = inp.heads, inp.head_dim
    if inp.edit:
        plan, blob = pam.mmdit_pack_plan_edit(inp.text_len, inp.grid_h, inp.grid_w, inp.src_h,
                                              inp.src_w, H, d, dtype_code)
    else:
        plan, blob = pam.mmdit_pack_plan(inp.text_len, inp.grid_h, inp.grid_w, H, d, dtype_code)
    lay = oracle.layout(inp.text_len, inp.grid_h, inp.grid_w, inp.src_h, inp.src_w)
    N, S = lay.num_tokens, len(inp.text_len)
    assert plan.total_tokens == N and plan.num_samples == S and plan.num_heads == H
    assert plan.max_seqlen == int(np.diff(lay.cu_seqlens).max())
    cu = _blob_section(blob, plan.off_cu_seqlens, S + 1, np.int32)
    assert np.array_equal(cu, lay.cu_seqlens)
    meta = _blob_section(blob, plan.off_tok_meta, N, np.int32)
    um = meta.view(np.uint32)
    assert np.array_equal((um >> 31).astype(bool), lay.is_image)
    assert np.array_equal(((um >> 16) & 0x7FFF).astype(np.int64), lay.row)
    assert np.array_equal((um & 0x7FFF).astype(np.int64), lay.col)
    assert np.array_equal(((um >> 15) & 1).astype(np.int64), lay.frame)
    # work lists: every tile of every sample once, longest segment first
    for n_items, off, tile in ((plan.num_fwd_items, plan.off_fwd_items, plan.q_tile),
                               (plan.num_bwd_items, plan.off_bwd_items, plan.kv_tile)):
        it = _blob_section(blob, off, 4 * n_items, np.int32).reshape(-1, 4)
        expect = set()
        for s in range(S):
            for t0 in range(cu[s], cu[s + 1], tile):
                expect.add((cu[s], cu[s + 1], t0, s))
        assert set(map(tuple, it.tolist())) == expect and len(it) == len(expect)
        lens = it[:, 1] - it[:, 0]
        assert np.all(np.diff(lens) <= 0)
    # workgroup -> (item, head) maps: each pair exactly once; -1 = idle; all
    # tiles of one (sample, head) on one XCD (workgroup b runs on XCD b % 8),
    # in tile order
    for n_items, n_blocks, off_it, off_bl in ((plan.num_fwd_items, plan.num_fwd_blocks,
                                               plan.off_fwd_items, plan.off_fwd_blocks),
                                              (plan.num_bwd_items, plan.num_bwd_blocks,
                                               plan.off_bwd_items, plan.off_bwd_blocks)):
        it = _blob_section(blob, off_it, 4 * n_items, np.int32).reshape(-1, 4)
        bl = _blob_section(blob, off_bl, 2 * n_blocks, np.int32).reshape(-1, 2)
        assert n_blocks % 8 == 0
        live = bl[bl[:, 0] >= 0]
        assert np.all(bl[bl[:, 0] < 0] == -1)
        pairs = set(map(tuple, live.tolist()))
        assert len(pairs) == len(live) == n_items * H
        assert pairs == {(i, hh) for i in range(n_items) for hh in range(H)}
        xcd_of = {}
        last_pos = {}
        for b, (i, hh) in enumerate(bl.tolist()):
            if i < 0:
                continue
            key = (int(it[i, 3]), hh)          # (sample, head)
            assert xcd_of.setdefault(key, b % 8) == b % 8
            assert last_pos.get(key, (-1, -1))[0] < b   # tiles in order
            assert it[i, 2] > last_pos.get(key, (-1, -1))[1]
            last_pos[key] = (b, int(it[i, 2]))
    # RoPE table [rope_rows][d/2]: cos/sin of pos * omega_p, rounded once to
    # fp32, omega_p the frequency of pair p in the oracle's schedule (read off
    # its angles for a token at position 1 on every axis)
    rope = _blob_section(blob, plan.off_rope, plan.rope_rows * (d // 2) * 2, np.float32)
    rope = rope.reshape(plan.rope_rows, d // 2, 2)
    sides = [inp.grid_h.max(), inp.grid_w.max()]
    if inp.edit:
        sides += [inp.src_h.max(), inp.src_w.max(), 2]
    assert plan.rope_rows == max(1, int(max(sides)))
    assert plan.rope_frame_pairs == (d // 8 if inp.edit else 0)
    unit = oracle.Layout(np.array([0, 1]), np.zeros(1, np.int64), np.ones(1, bool),
                         np.ones(1, np.int64), np.ones(1, np.int64), np.ones(1, np.int64),
                         inp.edit)
    om = oracle.rope_angles(unit, d)[0]
    pos = np.arange(plan.rope_rows)[:, None].astype(np.float64)
    ang = pos * om[None, :]
    # computed in fp64 and rounded once: within one fp32 ulp of the fp64
    # value, plus what a last-bit difference in the fp64 angle (pos * omega,
    # up to 32767 rad) can move it; bit equality with numpy holds for small
    # positions only, where the two libraries' last-ulp differences in pow
    # and cos cannot flip a rounding
    for got, ref in ((rope[..., 0], np.cos(ang)), (rope[..., 1], np.sin(ang))):
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        tol = ulp + 4.0 * np.spacing(np.maximum(ang, 1.0))
        assert np.all(np.abs(got.astype(np.float64) - ref) <= tol)
        if plan.rope_rows <= 64:
            assert np.array_equal(got, ref.astype(np.float32))
    # adaLN row chunks: each inside one (sample, stream) range, at most
    # mod_chunk_rows rows, covering every token once, ranges in order
    C_ = plan.num_mod_chunks
    ch = _blob_section(blob, plan.off_mod_chunks, 4 * C_, np.int32).reshape(-1, 4)
    rg = _blob_section(blob, plan.off_mod_ranges, 2 * S + 1, np.int32)
    assert plan.mod_chunk_rows == 32 and rg[0] == 0 and rg[-1] == C_ and np.all(np.diff(rg) >= 0)
    midx = oracle.modulation_index(lay)
    cover = np.zeros(N, np.int64)
    for c, (r0, r1, r, zero) in enumerate(ch.tolist()):
        assert zero == 0 and 0 < r1 - r0 <= 32 and rg[r] <= c < rg[r + 1]
        assert np.all(midx[r0:r1] == r)
        cover[r0:r1] += 1
    assert np.all(cover == 1)
    for r in range(2 * S):   # a range's chunks are consecutive and ordered
        rows = [x for c in range(rg[r], rg[r + 1]) for x in range(ch[c, 0], ch[c, 1])]
        assert rows == np.flatnonzero(midx == r).tolist()
    # stored-dS areas: per sample and head ceil(L/32) * 4 * ceil(L/64) blocks
    # of 1 KiB, samples in pack order; the area follows the backward's
    # workspace at the next 4 KiB (bf16 packs whose samples have at most
    # 32,768 tokens; else no larger workspace is offered)
    Ls = np.diff(lay.cu_seqlens)
    per = (Ls + 31) // 32 * 4 * ((Ls + 63) // 64)
    base = _blob_section(blob, plan.off_ds_base, S + 1, np.int64)
    assert np.array_equal(base, np.concatenate([[0], np.cumsum(H * per)]))
    if dtype_code == 1 and Ls.max() <= 32768:
        assert plan.bwd_ds_workspace_bytes == (plan.bwd_workspace_bytes + 4095) // 4096 * 4096 + 1024 * int(base[-1])
    else:
        assert plan.bwd_ds_workspace_bytes == plan.bwd_workspace_bytes
    return plan


@pytest.mark.parametrize("name", workloads.ORDER)
def test_plan_matches_oracle_layout_on_workloads(L, name):
    w = workloads.get(name)
    rng = np.random.default_rng(0)
    if w.text is None:
        text = rng.integers(w.text_range[0], w.text_range[1] + 1, len(w.grids))
    else:
        text = np.array(w.text)
    src = (None, None) if w.src is None else tuple(np.array([g[i] for g in w.src], np.int32)
                                                   for i in (0, 1))
    inp = workloads.Inputs(np.asarray(text, np.int32), np.array([g[0] for g in w.grids], np.int32),
                           np.array([g[1] for g in w.grids], np.int32), None, None, None, None,
                           None, w.heads, w.head_dim, w.dtype, src_h=src[0], src_w=src[1])
    plan = _check_plan(inp, 1 if w.dtype == "bf16" else 0)
    expect_n = {"tiny_fp32": 440, "gen1024": 4608, "mixed6": 20436, "gen2048": 16896,
                "small64": 74894, "edit1024": 8704}
    assert plan.total_tokens == expect_n[name]


@pytest.mark.parametrize("seed", range(12))
def test_plan_matches_oracle_layout_random(L, seed):
    inp = workloads.random_pack(seed, max_samples=9, max_text=300, max_side=40,
                                heads=3, head_dim=64, backward=False)
    _check_plan(inp, 0)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("d", [64, 128])
def test_edit_plan_matches_oracle_layout_random(L, seed, d):
    inp = workloads.random_pack(100 + seed, max_samples=7, max_text=200, max_side=33,
                                heads=2, head_dim=d, backward=False, edit=True)
    _check_plan(inp, 1)


def test_plan_largest_grid_sides(L):
    """Rows and columns at their 15-bit maximum (sides of 32,767), also on the
    source frame of an editing pack."""
    inp = workloads.random_pack(0, heads=1, head_dim=64, backward=False, text=[5, 0],
                                grids=[(1, 32767), (32767, 1)])
    assert _check_plan(inp, 1).rope_rows == 32767
    inp = workloads.random_pack(0, heads=1, head_dim=64, backward=False, text=[2],
                                grids=[(3, 2)], src=[(1, 32767)])
    assert _check_plan(inp, 1).rope_rows == 32767


def test_edit_plan_one_pixel_grids(L):
    """1 x 1 target and source grids: rope_rows still covers frame 1."""
    inp = workloads.random_pack(0, heads=1, head_dim=64, backward=False, text=[2, 0],
                                grids=[(1, 1), (1, 1)], src=[(1, 1), (0, 0)])
    plan = _check_plan(inp, 1)
    assert plan.rope_rows == 2 and plan.total_tokens == 5


def _edit_call(text, gh, gw, sh, sw, budget=0):
    t, h, w, a, b = (np.ascontiguousarray(x, np.int32) for x in (text, gh, gw, sh, sw))
    P = C.POINTER(C.c_int32)
    desc = pam.PackDesc(len(t), t.ctypes.data_as(P), h.ctypes.data_as(P), w.ctypes.data_as(P),
                        2, 64, 1, 1e4, 1e-6, budget)
    plan = pam.Plan()
    return pam.lib().mmdit_pack_plan_edit(C.byref(desc), a.ctypes.data_as(P), b.ctypes.data_as(P),
                                          C.byref(plan), None, 0), plan


@pytest.mark.parametrize("case,code", [
    (dict(sh=[2], sw=[0]), 1),              # source h without w
    (dict(sh=[-1], sw=[-1]), 1),            # negative source grid
    (dict(sh=[40000], sw=[1]), 1),          # source side too large
    (dict(gh=[0], gw=[0], sh=[2], sw=[2]), 1),   # source without a target
    (dict(budget=15), 4),                   # 3 + 4 + 9 = 16 tokens
])
def test_edit_plan_rejects(L, case, code):
    args = dict(text=[3], gh=[2], gw=[2], sh=[3], sw=[3])
    args.update(case)
    st, _ = _edit_call(**args)
    assert st == code, pam.mmdit_last_error()
    assert pam.mmdit_last_error()


def test_edit_plan_null_arrays_and_budget(L):
    t = np.array([3], np.int32)
    P = C.POINTER(C.c_int32)
    desc = pam.PackDesc(1, t.ctypes.data_as(P), t.ctypes.data_as(P), t.ctypes.data_as(P),
                        2, 64, 1, 1e4, 1e-6, 0)
    plan = pam.Plan()
    assert pam.lib().mmdit_pack_plan_edit(C.byref(desc), None, t.ctypes.data_as(P),
                                          C.byref(plan), None, 0) == 1
    st, plan = _edit_call([3], [2], [2], [3], [3], budget=16)
    assert st == 0 and plan.total_tokens == 16 and plan.rope_frame_pairs == 8


def _desc_call(text, gh, gw, H=2, d=64, dtype=1, theta=1e4, eps=1e-6, budget=0, blob_bytes=None):
    t = np.ascontiguousarray(text, np.int32)
    h = np.ascontiguousarray(gh, np.int32)
    w = np.ascontiguousarray(gw, np.int32)
    P = C.POINTER(C.c_int32)
    desc = pam.PackDesc(len(t), t.ctypes.data_as(P), h.ctypes.data_as(P), w.ctypes.data_as(P),
                        H, d, dtype, theta, eps, budget)
    plan = pam.Plan()
    if blob_bytes is None:
        return pam.lib().mmdit_pack_plan(C.byref(desc), C.byref(plan), None, 0), plan
    buf = np.zeros(max(blob_bytes, 1), np.uint8)
    return pam.lib().mmdit_pack_plan(C.byref(desc), C.byref(plan), buf.ctypes.data, blob_bytes), plan


@pytest.mark.parametrize("case,code", [
    (dict(text=[3], gh=[2], gw=[0]), 1),                 # grid h without w
    (dict(text=[-1], gh=[2], gw=[2]), 1),                # negative text
    (dict(text=[0], gh=[0], gw=[0]), 1),                 # empty sample
    (dict(text=[3], gh=[40000], gw=[1]), 1),             # grid side too large
    (dict(text=[3], gh=[2], gw=[2], H=0), 1),            # no heads
    (dict(text=[3], gh=[2], gw=[2], d=96), 2),           # unsupported head_dim
    (dict(text=[3], gh=[2], gw=[2], d=66), 1),           # not a multiple of 4
    (dict(text=[3], gh=[2], gw=[2], dtype=7), 1),        # bad dtype
    (dict(text=[3], gh=[2], gw=[2], theta=0.0), 1),      # bad theta
    (dict(text=[3], gh=[2], gw=[2], eps=-1.0), 1),       # bad eps
    (dict(text=[3], gh=[2], gw=[2], eps=float("nan")), 1),
    (dict(text=[30, 5], gh=[4, 1], gw=[4, 1], budget=40), 4),   # over budget (52 tokens)
    (dict(text=[0, 0], gh=[20000, 20000], gw=[20000, 20000]), 1),  # over 2^29 tokens
])
def test_plan_rejects_invalid_descriptors(L, case, code):
    st, _ = _desc_call(**case)
    assert st == code, pam.mmdit_last_error()
    assert pam.mmdit_last_error()


def test_plan_budget_and_blob_size(L):
    st, plan = _desc_call([30, 5], [4, 1], [4, 1], budget=52)
    assert st == 0 and plan.total_tokens == 52
    st, _ = _desc_call([30, 5], [4, 1], [4, 1], blob_bytes=int(plan.blob_bytes) - 1)
    assert st == 3
    st, plan2 = _desc_call([30, 5], [4, 1], [4, 1], blob_bytes=int(plan.blob_bytes))
    assert st == 0 and plan2.fingerprint == plan.fingerprint


# --------------------------------------------------------------------------
# argument validation of fwd / bwd: fake (aligned, never dereferenced) device
# pointers; every call below must fail on the host before any launch.
# --------------------------------------------------------------------------
BASE = 1 << 40
SZ = 1 << 30


def _p(i):
    return BASE + i * SZ


@pytest.fixture(scope="module")
def small_plan(L):
    plan, blob = pam.mmdit_pack_plan([5, 3], [2, 3], [3, 2], 2, 64, 1)
    return plan


def _fwd(plan, **kw):
    """Call mmdit_attn_fwd with fake pointers (ints); kw overrides fields."""
    args = dict(q=_p(1), k=_p(2), v=_p(3), q_stride=128, k_stride=128, v_stride=128,
                gains=_p(4), o=_p(5), lse=_p(6), q_hat=_p(7), k_hat=_p(8), rstd=_p(9),
                stages=0, blob=_p(0), ws=None, ws_bytes=0, plan=plan)
    args.update(kw)
    a = pam.FwdArgs(args["q"], args["k"], args["v"], args["q_stride"], args["k_stride"],
                    args["v_stride"], args["gains"], args["o"], args["lse"], args["q_hat"],
                    args["k_hat"], args["rstd"], args["stages"])
    return pam.lib().mmdit_attn_fwd(C.byref(args["plan"]), args["blob"], C.byref(a),
                                    args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1),
    (dict(q=_p(1) + 8), 1),               # misaligned
    (dict(q_stride=64), 1),               # stride < H*d
    (dict(k_stride=132), 1),              # not a multiple of 8
    (dict(v_stride=(1 << 24) + 8), 1),    # above the largest accepted stride
    (dict(gains=None), 1),
    (dict(o=None), 1),
    (dict(k_hat=None), 1),                # only one of q_hat / k_hat
    (dict(o=_p(3) + 256), 1),             # output overlaps v
    (dict(lse=_p(5) + 64), 1),            # output overlaps output
    (dict(stages=8), 1),
    (dict(blob=None), 1),
    (dict(q_hat=None, k_hat=None), 1),    # needs a workspace then
    (dict(q_hat=None, k_hat=None, ws=_p(10), ws_bytes=16), 3),
    (dict(q_hat=None, k_hat=None, ws=_p(10), ws_bytes=1 << 20, stages=1), 1),
])
def test_fwd_rejects_invalid_arguments(small_plan, kw, code):
    assert _fwd(small_plan, **kw) == code, pam.mmdit_last_error()


def test_fwd_rejects_foreign_plan(small_plan):
    bad = pam.Plan.from_buffer_copy(bytes(small_plan))
    bad.total_tokens += 1
    assert _fwd(bad) == 1
    assert "fingerprint" in pam.mmdit_last_error()


def _bwd(plan, ws_bytes=None, **kw):
    names = ("q", "k", "v", "q_hat", "k_hat", "o", "dout")
    args = {n: _p(i + 1) for i, n in enumerate(names)}
    args.update(gains=_p(8), lse=_p(9), rstd=_p(10), dq=_p(11), dk=_p(12), dv=_p(13), dgains=_p(14))
    args.update(kw)
    a = pam.BwdArgs(*(args[n] for n in names), 128, 128, 128, args.get("dout_stride", 128),
                    args["gains"], args["lse"], args["rstd"], args["dq"], args["dk"], args["dv"],
                    args["dgains"], args.get("stages", 0))
    ws = args.get("ws", _p(15))
    wsb = int(plan.bwd_workspace_bytes) if ws_bytes is None else ws_bytes
    return pam.lib().mmdit_attn_bwd(C.byref(plan), _p(0), C.byref(a), ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), 1),
    (dict(lse=None), 1),
    (dict(dq=None), 1),
    (dict(dq=_p(12) + 16), 1),            # dq overlaps dk
    (dict(dv=_p(3)), 1),                  # dv overlaps v
    (dict(dout_stride=64), 1),
    (dict(dout_stride=(1 << 24) + 8), 1),
    (dict(ws=None), 1),
    (dict(stages=32), 1),                 # unknown stage bit
    (dict(stages=8), 1),                  # stage D only in the stored-dS mode
    (dict(stages=8 | 16), 3),             # stored-dS mode without room for dS
    (dict(stages=8 | 16, o=None, ws_bytes=1 << 20), 1),     # stage D reads o
    (dict(stages=8 | 16, dout=None, ws_bytes=1 << 20), 1),  # ... and dout
    (dict(stages=1 | 2 | 16, ws_bytes=1 << 20), 1),   # stored dS: DQ and DKDV need D in the call
    (dict(stages=1 | 2 | 4 | 16, ws_bytes=1 << 20), 1),
    (dict(ws_bytes=64), 3),
    (dict(stages=1, q=None), 1),          # the dQ stage writes dq from q
    (dict(stages=1, o=None), 1),          # ... and forms D from o
    (dict(stages=2, k=None), 1),          # the dK/dV stage writes dk from k
    (dict(stages=2, dk=None), 1),
    (dict(stages=2, gains=None), 1),
    (dict(stages=2, dv=_p(12)), 1),       # dv overlaps dk
    (dict(stages=4, dgains=_p(15)), 1),   # dgains overlaps the workspace
])
def test_bwd_rejects_invalid_arguments(small_plan, kw, code):
    ws_bytes = kw.pop("ws_bytes", None)
    assert _bwd(small_plan, ws_bytes=ws_bytes, **kw) == code, pam.mmdit_last_error()


def test_bwd_stored_ds_mode_needs_a_bf16_plan(L):
    """fp32 plans (and samples over 32,768 tokens) have no stored-dS mode."""
    plan, _ = pam.mmdit_pack_plan([5, 3], [2, 3], [3, 2], 2, 64, 0)
    assert plan.bwd_ds_workspace_bytes == plan.bwd_workspace_bytes
    assert _bwd(plan, ws_bytes=1 << 20, stages=2 | 16) == 2, pam.mmdit_last_error()
    assert "stored-dS" in pam.mmdit_last_error()


def _adaln_fwd(plan, **kw):
    args = dict(x=_p(1), y=_p(2), x_stride=3072, y_stride=3072, shift=_p(3), scale=_p(4),
                gate=_p(5), model_dim=3072, eps=1e-6, z=_p(6), h=_p(7), stats=_p(8), blob=_p(0))
    args.update(kw)
    a = pam.AdalnFwdArgs(*(args[n] for n, _ in pam.AdalnFwdArgs._fields_))
    return pam.lib().mmdit_adaln_fwd(C.byref(plan), args["blob"], C.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1),
    (dict(x=_p(1) + 8), 1),               # misaligned
    (dict(x_stride=3000), 1),             # stride < D
    (dict(y_stride=3074), 1),             # not a multiple of 4
    (dict(model_dim=3070), 2),            # D not a multiple of 4
    (dict(model_dim=8196, x_stride=8196, y_stride=8196), 2),  # D above 8192
    (dict(model_dim=0), 2),
    (dict(eps=-1.0), 1),
    (dict(eps=float("inf")), 1),
    (dict(shift=None), 1),
    (dict(h=None), 1),
    (dict(gate=None), 1),                 # the residual needs its gate
    (dict(z=None), 1),                    # ... and writes z
    (dict(y=None), 1),                    # gate and z given without y
    (dict(h=_p(1) + 4096), 1),            # h overlaps x
    (dict(stats=_p(7) + 64), 1),          # stats overlaps h
    (dict(blob=None), 1),
])
def test_adaln_fwd_rejects_invalid_arguments(small_plan, kw, code):
    assert _adaln_fwd(small_plan, **kw) == code, pam.mmdit_last_error()


def _adaln_bwd(plan, **kw):
    args = dict(x=_p(1), y=_p(2), x_stride=1024, y_stride=1024, scale=_p(3), gate=_p(4),
                model_dim=1024, eps=1e-6, stats=_p(5), dh=_p(6), dz=_p(7), dh_stride=1024,
                dz_stride=1024, dx=_p(8), dy=_p(9), dshift=_p(10), dscale=_p(11), dgate=_p(12))
    ws = kw.pop("ws", _p(13))
    wsb = kw.pop("ws_bytes", plan.num_mod_chunks * 3 * 1024 * 4)
    args.update(kw)
    a = pam.AdalnBwdArgs(*(args[n] for n, _ in pam.AdalnBwdArgs._fields_))
    return pam.lib().mmdit_adaln_bwd(C.byref(plan), _p(0), C.byref(a), ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dh=None), 1),
    (dict(dx=None), 1),
    (dict(dscale=None), 1),
    (dict(dgate=None), 1),                # the residual writes dgate
    (dict(y=None), 1),                    # gate, dy, dgate given without y
    (dict(dz_stride=1000), 1),
    (dict(ws=None), 1),
    (dict(ws_bytes=1024), 3),
    (dict(dx=_p(6)), 1),                  # dx overlaps dh
    (dict(dshift=_p(13)), 1),             # dshift overlaps the workspace
    (dict(model_dim=1026), 2),
])
def test_adaln_bwd_rejects_invalid_arguments(small_plan, kw, code):
    assert _adaln_bwd(small_plan, **kw) == code, pam.mmdit_last_error()


def test_fault_injection_hook(small_plan, monkeypatch):
    """MMDIT_FAULT_INJECT=launch: every entry point that launches kernels
    returns MMDIT_ERR_HIP where it would launch, after its argument checks
    (which still win) and before any HIP call, so this runs without a GPU."""
    monkeypatch.setenv("MMDIT_FAULT_INJECT", "launch")
    for call in (_fwd, _bwd, _adaln_fwd, _adaln_bwd):
        assert call(small_plan) == 5, call.__name__
        assert "MMDIT_FAULT_INJECT" in pam.mmdit_last_error()
    assert _fwd(small_plan, q=None) == 1
    assert _bwd(small_plan, dq=None) == 1
    monkeypatch.setenv("MMDIT_FAULT_INJECT", "other")
    assert _fwd(small_plan, q=None) == 1
    assert "MMDIT_FAULT_INJECT" not in pam.mmdit_last_error()


# --------------------------------------------------------------------------
# packed classifier-free guidance: descriptor of conditional + unconditional
# --------------------------------------------------------------------------
def test_cfg_pack_desc_geometry(L):
    t, h, w = pam.mmdit_cfg_pack_desc([5, 0, 12], [2, 4, 0], [3, 4, 0], null_text_len=3)
    assert t.tolist() == [5, 0, 12, 3, 3, 3]
    assert h.tolist() == [2, 4, 0, 2, 4, 0]
    assert w.tolist() == [3, 4, 0, 3, 4, 0]
    plan, blob = pam.mmdit_pack_plan(t, h, w, 2, 64, 1)
    cu = np.frombuffer(blob.tobytes(), dtype=np.int32)[plan.off_cu_seqlens // 4:][:7]
    assert cu.tolist() == [0, 11, 27, 39, 48, 67, 70]


def test_cfg_pack_desc_rejects(L):
    with pytest.raises(pam.MmditError):
        pam.mmdit_cfg_pack_desc([5], [2], [3], null_text_len=-1)
    with pytest.raises(pam.MmditError):       # text-only sample, empty null prompt
        pam.mmdit_cfg_pack_desc([5, 7], [2, 0], [3, 0], null_text_len=0)
    t = np.array([5, 1], np.int32); h = np.array([2, 3], np.int32); w = np.array([3, 3], np.int32)
    P = C.POINTER(C.c_int32)
    cond = pam.PackDesc(2, t.ctypes.data_as(P), h.ctypes.data_as(P), w.ctypes.data_as(P),
                        2, 64, 1, 1e4, 1e-6, 20)
    buf = [np.zeros(4, np.int32) for _ in range(3)]
    out = pam.PackDesc()
    st = pam.lib().mmdit_cfg_pack_desc(C.byref(cond), 0, *(b.ctypes.data_as(P) for b in buf), 3,
                                       C.byref(out))
    assert st == 1 and pam.mmdit_last_error()           # capacity below 2S
    assert not buf[0].any()                              # nothing written on error
    st = pam.lib().mmdit_cfg_pack_desc(C.byref(cond), 0, *(b.ctypes.data_as(P) for b in buf), 4,
                                       C.byref(out))
    assert st == 0 and out.num_samples == 4 and out.token_budget == 20
    plan = pam.Plan()                                    # 6 + 10 + 6 + 9 = 31 tokens > 20
    assert pam.lib().mmdit_pack_plan(C.byref(out), C.byref(plan), None, 0) == 4


def test_pack_workspace_kinds(L):
    """Pack.workspace sizes: "bwd" and "bwd_recompute" take the plan's
    backward workspace, "bwd_ds" the stored-dS one (refused over ds_limit),
    "fwd" the inference forward's; unknown kinds are refused."""
    pack = pam.Pack([5, 3], [2, 3], [3, 2], 2, 64, "bf16", device="cpu")
    p = pack.plan
    assert p.bwd_ds_workspace_bytes > p.bwd_workspace_bytes
    assert pack.workspace("bwd").numel() == p.bwd_workspace_bytes
    assert pack.workspace("bwd_recompute").numel() == p.bwd_workspace_bytes
    assert pack.workspace("bwd_ds").numel() == p.bwd_ds_workspace_bytes
    assert pack.workspace("fwd").numel() == p.fwd_workspace_bytes
    with pytest.raises(ValueError):
        pack.workspace("bwd_ds", ds_limit=p.bwd_ds_workspace_bytes - 1)
    with pytest.raises(ValueError):
        pack.workspace("bwd_dS")


def _noalloc(plan, **kw):
    names = ("q", "k", "v", "q_hat", "k_hat", "o", "dout")
    args = {n: _p(i + 1) for i, n in enumerate(names)}
    args.update(gains=_p(8), lse=_p(9), rstd=_p(10), dq=_p(11), dk=_p(12), dv=_p(13), dgains=_p(14))
    args.update(kw)
    a = pam.BwdArgs(*(args[n] for n in names), 128, 128, 128, 128, args["gains"], args["lse"],
                    args["rstd"], args["dq"], args["dk"], args["dv"], args["dgains"],
                    args.get("stages", 0))
    return pam.lib().mmdit_attn_bwd_noalloc(None if plan is None else C.byref(plan), _p(0),
                                            C.byref(a), None)


def test_noalloc_refuses_before_touching_a_device(L):
    """The allocation-free backward refuses, on the host and before any HIP
    call, the stored-dS mode and packs whose workspace exceeds its array."""
    plan, _ = pam.mmdit_pack_plan([5, 3], [2, 3], [3, 2], 1, 128, 1)
    assert _noalloc(plan, stages=2 | 16) == 2, pam.mmdit_last_error()
    assert "recompute" in pam.mmdit_last_error()
    big, _ = pam.mmdit_pack_plan([0], [512], [512], 24, 128, 1)
    assert big.bwd_workspace_bytes > 64 << 20
    assert _noalloc(big) == 3, pam.mmdit_last_error()
    assert "exceeds" in pam.mmdit_last_error()
    assert _noalloc(None) == 1


def test_stream_probe_rejects_bad_arguments(L):
    """mmdit_probe_streams checks its arguments before it launches anything
    (no GPU needed): unsupported mixes and unrolls, misaligned and
    overlapping buffers, a read-only probe without a sink."""
    import ctypes as C
    L.mmdit_probe_streams.restype = C.c_int
    L.mmdit_probe_streams.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.POINTER(C.c_void_p), C.c_int32,
                                      C.c_uint64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    base = 1 << 40
    srcs = (C.c_void_p * 4)(base, base + (1 << 30), base + (2 << 30), base + (3 << 30))
    dsts = (C.c_void_p * 2)(base + (4 << 30), base + (5 << 30))
    INVALID = 1
    for nr, nw in [(3, 1), (1, 2), (4, 1), (0, 1)]:
        assert L.mmdit_probe_streams(srcs, nr, dsts, nw, 1 << 20, 8, 1, None, None) == INVALID
    assert L.mmdit_probe_streams(srcs, 2, dsts, 2, 1 << 20, 8, 3, None, None) == INVALID     # unroll
    assert L.mmdit_probe_streams(srcs, 2, dsts, 2, (1 << 20) + 8, 8, 1, None, None) == INVALID  # bytes
    assert L.mmdit_probe_streams(srcs, 1, dsts, 0, 1 << 20, 8, 1, None, None) == INVALID     # no sink
    bad = (C.c_void_p * 4)(base + 8, base + (1 << 30), 0, 0)
    assert L.mmdit_probe_streams(bad, 2, dsts, 2, 1 << 20, 8, 1, None, None) == INVALID      # misaligned
    ovl = (C.c_void_p * 4)(base, base + (1 << 19), 0, 0)
    assert L.mmdit_probe_streams(ovl, 2, dsts, 2, 1 << 20, 8, 1, None, None) == INVALID      # overlap
    assert "overlap" in pam.mmdit_last_error()
