"""Python binding of libmmdit (packed native-resolution joint attention on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmmdit.so; torch provides device memory and the HIP stream. The
three C entry points keep their names here (``mmdit_pack_plan``,
``mmdit_attn_fwd``, ``mmdit_attn_bwd``); ``Pack``, ``forward`` and ``backward``
are small conveniences that allocate outputs with torch and call them.

Importing this module does not need a GPU. Loading the library fails loudly
(ImportError) when libmmdit.so has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "MmditError", "lib", "mmdit_pack_plan", "mmdit_pack_plan_edit", "mmdit_attn_fwd",
    "mmdit_attn_bwd", "mmdit_attn_bwd_noalloc", "mmdit_cfg_pack_desc", "mmdit_adaln_fwd", "mmdit_adaln_bwd",
    "adaln_forward", "adaln_backward",
    "mmdit_status_str", "mmdit_last_error", "mmdit_abi_version", "mmdit_device_faults", "Pack",
    "forward", "backward", "FWD_STAGES", "BWD_STAGES", "LIB_PATH",
]

ABI_VERSION = 5
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmmdit.so")

MMDIT_F32, MMDIT_BF16 = 0, 1
STAGE_PROLOGUE, STAGE_ATTENTION = 1, 2
STAGE_BWD_DQ, STAGE_BWD_DKDV, STAGE_BWD_GAINS, STAGE_BWD_D, STAGE_BWD_STORE_DS = 1, 2, 4, 8, 16
DEVICE_FAULT_STALE_BLOB = 1
FWD_STAGES = {"prologue": STAGE_PROLOGUE, "attention": STAGE_ATTENTION}
BWD_STAGES = {"dq": STAGE_BWD_DQ, "dkdv": STAGE_BWD_DKDV, "gains": STAGE_BWD_GAINS,
              "d": STAGE_BWD_D, "store_ds": STAGE_BWD_STORE_DS}


class PackDesc(C.Structure):
    _fields_ = [("num_samples", C.c_int32), ("text_len", C.POINTER(C.c_int32)),
                ("grid_h", C.POINTER(C.c_int32)), ("grid_w", C.POINTER(C.c_int32)),
                ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32),
                ("rope_theta", C.c_float), ("rms_eps", C.c_float), ("token_budget", C.c_int64)]


# Largest workspace Pack.workspace("bwd_ds") (the stored-dS backward's) allocates
# unless told otherwise.
DS_WORKSPACE_LIMIT = 16 << 30


class Plan(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_samples", "total_tokens", "max_seqlen", "num_heads", "head_dim", "dtype",
        "q_tile", "kv_tile", "num_fwd_items", "num_bwd_items", "rope_rows", "rope_frame_pairs",
        "num_fwd_blocks", "num_bwd_blocks")] + [
        ("rope_theta", C.c_float), ("rms_eps", C.c_float)] + [(n, C.c_uint64) for n in (
        "blob_bytes", "off_cu_seqlens", "off_tok_meta", "off_fwd_items", "off_bwd_items",
        "off_rope", "off_fwd_blocks", "off_bwd_blocks", "fwd_workspace_bytes",
        "bwd_workspace_bytes", "off_mod_chunks", "off_mod_ranges")] + [
        ("num_mod_chunks", C.c_int32), ("mod_chunk_rows", C.c_int32), ("off_ds_base", C.c_uint64),
        ("bwd_ds_workspace_bytes", C.c_uint64), ("fingerprint", C.c_uint64)]


class FwdArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("q_stride", C.c_int64), ("k_stride", C.c_int64), ("v_stride", C.c_int64),
                ("gains", C.c_void_p), ("o", C.c_void_p), ("lse", C.c_void_p),
                ("q_hat", C.c_void_p), ("k_hat", C.c_void_p), ("rstd", C.c_void_p),
                ("stages", C.c_uint32)]


class BwdArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
                ("q_hat", C.c_void_p), ("k_hat", C.c_void_p), ("o", C.c_void_p),
                ("dout", C.c_void_p),
                ("q_stride", C.c_int64), ("k_stride", C.c_int64), ("v_stride", C.c_int64),
                ("dout_stride", C.c_int64),
                ("gains", C.c_void_p), ("lse", C.c_void_p), ("rstd", C.c_void_p),
                ("dq", C.c_void_p), ("dk", C.c_void_p), ("dv", C.c_void_p),
                ("dgains", C.c_void_p), ("stages", C.c_uint32)]


class AdalnFwdArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("y", C.c_void_p), ("x_stride", C.c_int64),
                ("y_stride", C.c_int64), ("shift", C.c_void_p), ("scale", C.c_void_p),
                ("gate", C.c_void_p), ("model_dim", C.c_int32), ("eps", C.c_float),
                ("z", C.c_void_p), ("h", C.c_void_p), ("stats", C.c_void_p)]


class AdalnBwdArgs(C.Structure):
    _fields_ = [("x", C.c_void_p), ("y", C.c_void_p), ("x_stride", C.c_int64),
                ("y_stride", C.c_int64), ("scale", C.c_void_p), ("gate", C.c_void_p),
                ("model_dim", C.c_int32), ("eps", C.c_float), ("stats", C.c_void_p),
                ("dh", C.c_void_p), ("dz", C.c_void_p), ("dh_stride", C.c_int64),
                ("dz_stride", C.c_int64), ("dx", C.c_void_p), ("dy", C.c_void_p),
                ("dshift", C.c_void_p), ("dscale", C.c_void_p), ("dgate", C.c_void_p)]


class MmditError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{mmdit_status_str(status)} ({status}): {message}")
        self.status = status


_lib = None


def lib():
    """Load libmmdit.so (once). Raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m packed_attention_nr_amd.build` (hipcc, gfx950)")
        # torch's bundled HIP runtime has the same soname as ROCm's: loading
        # torch first makes libmmdit bind to that one runtime instead of
        # bringing a second one into the process.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        L.mmdit_pack_plan.restype = C.c_int
        L.mmdit_pack_plan.argtypes = [C.POINTER(PackDesc), C.POINTER(Plan), C.c_void_p, C.c_uint64]
        L.mmdit_pack_plan_edit.restype = C.c_int
        L.mmdit_pack_plan_edit.argtypes = [C.POINTER(PackDesc), C.POINTER(C.c_int32),
                                           C.POINTER(C.c_int32), C.POINTER(Plan), C.c_void_p,
                                           C.c_uint64]
        L.mmdit_cfg_pack_desc.restype = C.c_int
        L.mmdit_cfg_pack_desc.argtypes = [C.POINTER(PackDesc), C.c_int32, C.POINTER(C.c_int32),
                                          C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_int32,
                                          C.POINTER(PackDesc)]
        L.mmdit_attn_fwd.restype = C.c_int
        L.mmdit_attn_fwd.argtypes = [C.POINTER(Plan), C.c_void_p, C.POINTER(FwdArgs), C.c_void_p,
                                     C.c_uint64, C.c_void_p]
        L.mmdit_attn_bwd.restype = C.c_int
        L.mmdit_attn_bwd.argtypes = [C.POINTER(Plan), C.c_void_p, C.POINTER(BwdArgs), C.c_void_p,
                                     C.c_uint64, C.c_void_p]
        L.mmdit_attn_bwd_noalloc.restype = C.c_int
        L.mmdit_attn_bwd_noalloc.argtypes = [C.POINTER(Plan), C.c_void_p, C.POINTER(BwdArgs),
                                             C.c_void_p]
        L.mmdit_adaln_fwd.restype = C.c_int
        L.mmdit_adaln_fwd.argtypes = [C.POINTER(Plan), C.c_void_p, C.POINTER(AdalnFwdArgs),
                                      C.c_void_p]
        L.mmdit_adaln_bwd.restype = C.c_int
        L.mmdit_adaln_bwd.argtypes = [C.POINTER(Plan), C.c_void_p, C.POINTER(AdalnBwdArgs),
                                      C.c_void_p, C.c_uint64, C.c_void_p]
        L.mmdit_status_str.restype = C.c_char_p
        L.mmdit_status_str.argtypes = [C.c_int]
        L.mmdit_last_error.restype = C.c_char_p
        L.mmdit_last_error.argtypes = []
        L.mmdit_abi_version.restype = C.c_int32
        L.mmdit_abi_version.argtypes = []
        L.mmdit_device_faults.restype = C.c_int
        L.mmdit_device_faults.argtypes = [C.POINTER(C.c_uint32), C.c_void_p]
        if L.mmdit_abi_version() != ABI_VERSION:
            raise ImportError("libmmdit ABI version mismatch")
        _lib = L
    return _lib


def mmdit_status_str(status: int) -> str:
    return lib().mmdit_status_str(status).decode()


def mmdit_last_error() -> str:
    return lib().mmdit_last_error().decode()


def mmdit_abi_version() -> int:
    return int(lib().mmdit_abi_version())


def mmdit_device_faults(stream=None) -> int:
    """Read and clear this GPU's fault word (synchronises the stream): the OR
    of the DEVICE_FAULT_* flags the kernels recorded since the last read."""
    out = C.c_uint32(0)
    _check(lib().mmdit_device_faults(C.byref(out), _stream(stream)))
    return int(out.value)


def _check(status: int):
    if status != 0:
        raise MmditError(status, mmdit_last_error())


def _plan(text_len, grid_h, grid_w, num_heads, head_dim, dtype, rope_theta, rms_eps,
          token_budget, src_h=None, src_w=None):
    t = np.ascontiguousarray(text_len, dtype=np.int32)
    h = np.ascontiguousarray(grid_h, dtype=np.int32)
    w = np.ascontiguousarray(grid_w, dtype=np.int32)
    if not (len(t) == len(h) == len(w)):
        raise ValueError("text_len, grid_h and grid_w must have the same length")
    P = C.POINTER(C.c_int32)
    desc = PackDesc(len(t), t.ctypes.data_as(P), h.ctypes.data_as(P), w.ctypes.data_as(P),
                    int(num_heads), int(head_dim), int(dtype), float(rope_theta), float(rms_eps),
                    int(token_budget))
    plan = Plan()
    if src_h is None:
        call = lambda blob, n: lib().mmdit_pack_plan(C.byref(desc), C.byref(plan), blob, n)
    else:
        sh = np.ascontiguousarray(src_h, dtype=np.int32)
        sw = np.ascontiguousarray(src_w, dtype=np.int32)
        if not (len(sh) == len(sw) == len(t)):
            raise ValueError("src_h and src_w must have one entry per sample")
        call = lambda blob, n: lib().mmdit_pack_plan_edit(
            C.byref(desc), sh.ctypes.data_as(P), sw.ctypes.data_as(P), C.byref(plan), blob, n)
    _check(call(None, 0))
    blob = np.zeros(plan.blob_bytes, dtype=np.uint8)
    _check(call(blob.ctypes.data, blob.nbytes))
    return plan, blob


def mmdit_pack_plan(text_len: Sequence[int], grid_h: Sequence[int], grid_w: Sequence[int],
                    num_heads: int, head_dim: int, dtype: int, rope_theta: float = 10000.0,
                    rms_eps: float = 1e-6, token_budget: int = 0):
    """Run mmdit_pack_plan. Returns (plan, blob) with blob a uint8 numpy array
    holding the host copy of the plan blob."""
    return _plan(text_len, grid_h, grid_w, num_heads, head_dim, dtype, rope_theta, rms_eps,
                 token_budget)


def mmdit_pack_plan_edit(text_len: Sequence[int], grid_h: Sequence[int], grid_w: Sequence[int],
                         src_h: Sequence[int], src_w: Sequence[int], num_heads: int,
                         head_dim: int, dtype: int, rope_theta: float = 10000.0,
                         rms_eps: float = 1e-6, token_budget: int = 0):
    """Run mmdit_pack_plan_edit (editing pack: each sample's source grid
    follows its target grid, on frame 1 of a 3D RoPE). Returns (plan, blob)."""
    if src_h is None or src_w is None:
        raise ValueError("src_h and src_w are required")
    return _plan(text_len, grid_h, grid_w, num_heads, head_dim, dtype, rope_theta, rms_eps,
                 token_budget, src_h, src_w)


def mmdit_cfg_pack_desc(text_len: Sequence[int], grid_h: Sequence[int], grid_w: Sequence[int],
                        null_text_len: int = 0):
    """Run mmdit_cfg_pack_desc on a conditional pack's geometry. Returns the
    (text_len, grid_h, grid_w) int32 arrays of the packed conditional +
    unconditional pack: the conditional samples first, then their twins with
    the same grids and null_text_len text tokens."""
    t = np.ascontiguousarray(text_len, dtype=np.int32)
    h = np.ascontiguousarray(grid_h, dtype=np.int32)
    w = np.ascontiguousarray(grid_w, dtype=np.int32)
    if not (len(t) == len(h) == len(w)):
        raise ValueError("text_len, grid_h and grid_w must have the same length")
    P = C.POINTER(C.c_int32)
    cond = PackDesc(len(t), t.ctypes.data_as(P), h.ctypes.data_as(P), w.ctypes.data_as(P),
                    1, 64, MMDIT_BF16, 10000.0, 1e-6, 0)
    n = 2 * len(t)
    ot, oh, ow = (np.zeros(max(n, 1), dtype=np.int32) for _ in range(3))
    out = PackDesc()
    _check(lib().mmdit_cfg_pack_desc(C.byref(cond), int(null_text_len), ot.ctypes.data_as(P),
                                     oh.ctypes.data_as(P), ow.ctypes.data_as(P), n, C.byref(out)))
    assert out.num_samples == n
    return ot[:n].copy(), oh[:n].copy(), ow[:n].copy()


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on_stream(stream):
    """Context for the conveniences below: with `stream` (a torch stream or a
    raw hipStream_t handle) made current, every buffer they allocate (outputs
    and the workspace they drop on return) belongs to the stream the kernels
    run on, so torch's caching allocator cannot hand it to other work while
    the kernels still use it."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def mmdit_attn_fwd(plan: Plan, blob_dev, *, q=None, k=None, v=None, q_stride=0, k_stride=0,
                   v_stride=0, gains=None, o=None, lse=None, q_hat=None, k_hat=None, rstd=None,
                   workspace=None, stages: int = 0, stream=None):
    """Run mmdit_attn_fwd with torch tensors (device pointers taken from them)."""
    a = FwdArgs(_ptr(q), _ptr(k), _ptr(v), int(q_stride), int(k_stride), int(v_stride),
                _ptr(gains), _ptr(o), _ptr(lse), _ptr(q_hat), _ptr(k_hat), _ptr(rstd), int(stages))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mmdit_attn_fwd(C.byref(plan), _ptr(blob_dev), C.byref(a), _ptr(workspace),
                                ws_bytes, _stream(stream)))


def mmdit_attn_bwd(plan: Plan, blob_dev, *, q=None, k=None, v=None, q_hat=None, k_hat=None,
                   o=None, dout=None, q_stride=0, k_stride=0, v_stride=0, dout_stride=0,
                   gains=None, lse=None, rstd=None, dq=None, dk=None, dv=None, dgains=None,
                   workspace=None, stages: int = 0, stream=None):
    """Run mmdit_attn_bwd with torch tensors (device pointers taken from them)."""
    a = BwdArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(q_hat), _ptr(k_hat), _ptr(o), _ptr(dout),
                int(q_stride), int(k_stride), int(v_stride), int(dout_stride), _ptr(gains),
                _ptr(lse), _ptr(rstd), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgains), int(stages))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mmdit_attn_bwd(C.byref(plan), _ptr(blob_dev), C.byref(a), _ptr(workspace),
                                ws_bytes, _stream(stream)))


def mmdit_attn_bwd_noalloc(plan: Plan, blob_dev, *, q=None, k=None, v=None, q_hat=None,
                           k_hat=None, o=None, dout=None, q_stride=0, k_stride=0, v_stride=0,
                           dout_stride=0, gains=None, lse=None, rstd=None, dq=None, dk=None,
                           dv=None, dgains=None, stages: int = 0, stream=None):
    """Run mmdit_attn_bwd_noalloc (the recompute backward with the library's
    own per-GPU workspace; no workspace argument)."""
    a = BwdArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(q_hat), _ptr(k_hat), _ptr(o), _ptr(dout),
                int(q_stride), int(k_stride), int(v_stride), int(dout_stride), _ptr(gains),
                _ptr(lse), _ptr(rstd), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgains), int(stages))
    _check(lib().mmdit_attn_bwd_noalloc(C.byref(plan), _ptr(blob_dev), C.byref(a),
                                        _stream(stream)))


def mmdit_adaln_fwd(plan: Plan, blob_dev, *, x=None, y=None, x_stride=0, y_stride=0, shift=None,
                    scale=None, gate=None, model_dim=0, eps=1e-6, z=None, h=None, stats=None,
                    stream=None):
    """Run mmdit_adaln_fwd with torch tensors (device pointers taken from them)."""
    a = AdalnFwdArgs(_ptr(x), _ptr(y), int(x_stride), int(y_stride), _ptr(shift), _ptr(scale),
                     _ptr(gate), int(model_dim), float(eps), _ptr(z), _ptr(h), _ptr(stats))
    _check(lib().mmdit_adaln_fwd(C.byref(plan), _ptr(blob_dev), C.byref(a), _stream(stream)))


def mmdit_adaln_bwd(plan: Plan, blob_dev, *, x=None, y=None, x_stride=0, y_stride=0, scale=None,
                    gate=None, model_dim=0, eps=1e-6, stats=None, dh=None, dz=None, dh_stride=0,
                    dz_stride=0, dx=None, dy=None, dshift=None, dscale=None, dgate=None,
                    workspace=None, stream=None):
    """Run mmdit_adaln_bwd with torch tensors (device pointers taken from them)."""
    a = AdalnBwdArgs(_ptr(x), _ptr(y), int(x_stride), int(y_stride), _ptr(scale), _ptr(gate),
                     int(model_dim), float(eps), _ptr(stats), _ptr(dh), _ptr(dz), int(dh_stride),
                     int(dz_stride), _ptr(dx), _ptr(dy), _ptr(dshift), _ptr(dscale), _ptr(dgate))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mmdit_adaln_bwd(C.byref(plan), _ptr(blob_dev), C.byref(a), _ptr(workspace),
                                 ws_bytes, _stream(stream)))


# ---------------------------------------------------------------------------
# Conveniences: a pack with its device blob; forward / backward with torch-
# allocated outputs.
# ---------------------------------------------------------------------------
def _torch_dtype(dtype: int):
    import torch
    return torch.bfloat16 if dtype == MMDIT_BF16 else torch.float32


def _token_stride(t, N, H, d, name):
    if t.dim() != 3 or tuple(t.shape) != (N, H, d):
        raise ValueError(f"{name} must have shape ({N}, {H}, {d}), got {tuple(t.shape)}")
    if t.stride(2) != 1 or (H > 1 and t.stride(1) != d):  # a lone head's stride is immaterial
        raise ValueError(f"{name}: heads and head_dim must be contiguous")
    return t.stride(0)


class Pack:
    """Plan of one pack plus its device blob (copied once)."""

    def __init__(self, text_len, grid_h, grid_w, num_heads, head_dim, dtype="bf16",
                 rope_theta=10000.0, rms_eps=1e-6, token_budget=0, device="cuda",
                 src_h=None, src_w=None):
        """src_h, src_w (per-sample source grids) make an editing pack
        (mmdit_pack_plan_edit); None makes a generation pack."""
        import torch
        self.dtype_code = MMDIT_BF16 if dtype in ("bf16", MMDIT_BF16) else MMDIT_F32
        if src_h is None and src_w is None:
            self.plan, self.blob = mmdit_pack_plan(text_len, grid_h, grid_w, num_heads, head_dim,
                                                   self.dtype_code, rope_theta, rms_eps,
                                                   token_budget)
        else:
            self.plan, self.blob = mmdit_pack_plan_edit(text_len, grid_h, grid_w, src_h, src_w,
                                                        num_heads, head_dim, self.dtype_code,
                                                        rope_theta, rms_eps, token_budget)
        self.blob_dev = torch.from_numpy(self.blob).to(device)
        self.N = self.plan.total_tokens
        self.H = self.plan.num_heads
        self.d = self.plan.head_dim
        self.device = device
        self.torch_dtype = _torch_dtype(self.dtype_code)

    def workspace(self, kind: str, model_dim: int = 0, ds_limit: int = DS_WORKSPACE_LIMIT):
        """Workspace of the attention forward ("fwd"), backward ("bwd") or
        the adaLN backward ("adaln", for model width model_dim). "bwd" (and
        "bwd_recompute") is the workspace with which the backward forms S and
        dP again for dQ; "bwd_ds" is large enough for it to store dS and form
        dQ from it (bf16 plans that offer that mode), when that needs at most
        ds_limit bytes."""
        import torch
        if kind == "adaln":
            n = self.plan.num_mod_chunks * 3 * int(model_dim) * 4
        elif kind == "fwd":
            n = self.plan.fwd_workspace_bytes
        elif kind in ("bwd", "bwd_recompute"):
            n = self.plan.bwd_workspace_bytes
        elif kind == "bwd_ds":
            n = self.plan.bwd_ds_workspace_bytes
            if n > ds_limit:
                raise ValueError(f"the stored-dS workspace needs {n} bytes, over ds_limit={ds_limit}")
        else:
            raise ValueError(f"unknown workspace kind {kind!r}")
        return torch.empty(max(int(n), 16), dtype=torch.uint8, device=self.device)


def forward(pack: Pack, q, k, v, gains, *, save_for_backward: bool = True, stream=None):
    """O (and lse, q_hat, k_hat, rstd when saving for the backward). With
    `stream`, outputs and workspace are allocated on it and the kernels run on
    it."""
    with _on_stream(stream):
        return _forward(pack, q, k, v, gains, save_for_backward)


def _forward(pack, q, k, v, gains, save_for_backward):
    import torch
    N, H, d = pack.N, pack.H, pack.d
    qs = _token_stride(q, N, H, d, "q")
    ks = _token_stride(k, N, H, d, "k")
    vs = _token_stride(v, N, H, d, "v")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != pack.torch_dtype:
            raise TypeError(f"{n} must be {pack.torch_dtype}")
    if gains.dtype != torch.float32 or tuple(gains.shape) != (4, d) or not gains.is_contiguous():
        raise TypeError("gains must be a contiguous float32 tensor of shape (4, d)")
    dev = q.device
    o = torch.empty((N, H, d), dtype=pack.torch_dtype, device=dev)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    out = dict(o=o, lse=lse)
    if save_for_backward:
        q_hat = torch.empty_like(o)
        k_hat = torch.empty_like(o)
        rstd = torch.empty((2, N, H), dtype=torch.float32, device=dev)
        mmdit_attn_fwd(pack.plan, pack.blob_dev, q=q, k=k, v=v, q_stride=qs, k_stride=ks,
                       v_stride=vs, gains=gains, o=o, lse=lse, q_hat=q_hat, k_hat=k_hat,
                       rstd=rstd)
        out.update(q_hat=q_hat, k_hat=k_hat, rstd=rstd)
    else:
        ws = pack.workspace("fwd")
        mmdit_attn_fwd(pack.plan, pack.blob_dev, q=q, k=k, v=v, q_stride=qs, k_stride=ks,
                       v_stride=vs, gains=gains, o=o, lse=lse, workspace=ws)
    return out


def backward(pack: Pack, q, k, v, gains, saved: dict, dout, *, workspace=None,
             mode: str = "recompute", stream=None):
    """dq, dk, dv (w.r.t. the pre-norm inputs) and dgains for loss sum(dout * o).
    mode "recompute" (dQ with S and dP formed again) or "stored_ds" (dQ from
    the dS the dK/dV kernel stores; needs Pack.workspace("bwd_ds")); the
    workspace defaults to the mode's. With `stream`, outputs and workspace are
    allocated on it and the kernels run on it."""
    with _on_stream(stream):
        return _backward(pack, q, k, v, gains, saved, dout, workspace, mode)


def _backward(pack, q, k, v, gains, saved, dout, workspace, mode):
    import torch
    if mode not in ("recompute", "stored_ds"):
        raise ValueError(f"unknown backward mode {mode!r}")
    N, H, d = pack.N, pack.H, pack.d
    qs = _token_stride(q, N, H, d, "q")
    ks = _token_stride(k, N, H, d, "k")
    vs = _token_stride(v, N, H, d, "v")
    gs = _token_stride(dout, N, H, d, "dout")
    if dout.dtype != pack.torch_dtype:
        raise TypeError(f"dout must be {pack.torch_dtype}")
    dev = q.device
    dq = torch.empty((N, H, d), dtype=pack.torch_dtype, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    dgains = torch.empty((4, d), dtype=torch.float32, device=dev)
    ds = mode == "stored_ds"
    ws = pack.workspace("bwd_ds" if ds else "bwd") if workspace is None else workspace
    mmdit_attn_bwd(pack.plan, pack.blob_dev, q=q, k=k, v=v, q_hat=saved["q_hat"],
                   k_hat=saved["k_hat"], o=saved["o"], dout=dout, q_stride=qs, k_stride=ks,
                   v_stride=vs, dout_stride=gs, gains=gains, lse=saved["lse"],
                   rstd=saved.get("rstd"), dq=dq, dk=dk, dv=dv, dgains=dgains, workspace=ws,
                   stages=STAGE_BWD_STORE_DS if ds else 0)
    return dict(dq=dq, dk=dk, dv=dv, dgains=dgains, workspace=ws)


def _rows_stride(t, N, name):
    if t.dim() != 2 or t.shape[0] != N or t.stride(1) != 1:
        raise ValueError(f"{name} must be a [N={N}, D] tensor with unit column stride")
    return t.stride(0)


def adaln_forward(pack: Pack, x, shift, scale, *, y=None, gate=None, eps: float = 1e-6,
                  save_stats: bool = True, stream=None):
    """h = adaLN(z) with z = x (+ gate * y); returns dict with h, z (with y)
    and stats ([N, 2] mean and rstd, when saved). With `stream`, outputs are
    allocated on it and the kernels run on it."""
    with _on_stream(stream):
        return _adaln_forward(pack, x, shift, scale, y, gate, eps, save_stats)


def _adaln_forward(pack, x, shift, scale, y, gate, eps, save_stats):
    import torch
    N, D = pack.N, int(x.shape[-1])
    xs = _rows_stride(x, N, "x")
    ys = 0 if y is None else _rows_stride(y, N, "y")
    h = torch.empty((N, D), dtype=pack.torch_dtype, device=x.device)
    z = None if y is None else torch.empty_like(h)
    stats = torch.empty((N, 2), dtype=torch.float32, device=x.device) if save_stats else None
    mmdit_adaln_fwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=xs, y_stride=ys, shift=shift,
                    scale=scale, gate=gate, model_dim=D, eps=eps, z=z, h=h, stats=stats)
    out = dict(h=h)
    if z is not None:
        out["z"] = z
    if stats is not None:
        out["stats"] = stats
    return out


def adaln_backward(pack: Pack, x, scale, dh, *, y=None, gate=None, dz=None, stats=None,
                   eps: float = 1e-6, workspace=None, stream=None):
    """dx (= dz_total), dy, dshift, dscale, dgate of ``adaln_forward``. With
    `stream`, outputs and workspace are allocated on it and the kernels run on
    it."""
    with _on_stream(stream):
        return _adaln_backward(pack, x, scale, dh, y, gate, dz, stats, eps, workspace)


def _adaln_backward(pack, x, scale, dh, y, gate, dz, stats, eps, workspace):
    import torch
    N, D = pack.N, int(x.shape[-1])
    S = pack.plan.num_samples
    dx = torch.empty((N, D), dtype=pack.torch_dtype, device=x.device)
    dy = None if y is None else torch.empty_like(dx)
    f32 = dict(dtype=torch.float32, device=x.device)
    dshift, dscale = torch.empty((S, 2, D), **f32), torch.empty((S, 2, D), **f32)
    dgate = None if y is None else torch.empty((S, 2, D), **f32)
    ws = pack.workspace("adaln", D) if workspace is None else workspace
    mmdit_adaln_bwd(pack.plan, pack.blob_dev, x=x, y=y, x_stride=_rows_stride(x, N, "x"),
                    y_stride=0 if y is None else _rows_stride(y, N, "y"), scale=scale, gate=gate,
                    model_dim=D, eps=eps, stats=stats, dh=dh, dz=dz,
                    dh_stride=_rows_stride(dh, N, "dh"),
                    dz_stride=0 if dz is None else _rows_stride(dz, N, "dz"), dx=dx, dy=dy,
                    dshift=dshift, dscale=dscale, dgate=dgate, workspace=ws)
    out = dict(dx=dx, dshift=dshift, dscale=dscale)
    if y is not None:
        out.update(dy=dy, dgate=dgate)
    return out
