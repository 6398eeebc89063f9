"""The measurement probes' results on the GPU: the stream probe writes, for
every destination w, the XOR of its sources' 16-byte words with w added to
the first 32-bit component, for each supported mix, unroll and a grid that
leaves a ragged tail; the copy probe copies. Marked ``gpu``."""
import ctypes as C
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import packed_attention_nr_amd as pam
    L = pam.lib()
    L.mmdit_probe_streams.restype = C.c_int
    L.mmdit_probe_streams.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.POINTER(C.c_void_p), C.c_int32,
                                      C.c_uint64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    L.mmdit_probe_copy.restype = C.c_int
    L.mmdit_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_int32, C.c_void_p]
    return L


@pytest.mark.parametrize("unroll", [1, 2])
@pytest.mark.parametrize("mix", [(1, 0), (1, 1), (2, 1), (2, 2), (4, 2)])
def test_stream_probe_values(L, mix, unroll):
    nr, nw = mix
    n16 = 3 * 256 * 2 * 5 + 7          # several grid-stride steps of 3 workgroups, ragged tail
    print(f"stream probe {nr}r{nw}w unroll={unroll} words={n16}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(10 * nr + nw + unroll)
    src = [rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint32) for _ in range(nr)]
    d_src = [torch.from_numpy(s.view(np.int32)).to("cuda") for s in src]
    d_dst = [torch.full((n16, 4), -1, dtype=torch.int32, device="cuda") for _ in range(nw)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    srcs = (C.c_void_p * 4)(*[t.data_ptr() for t in d_src])
    dsts = (C.c_void_p * 2)(*[t.data_ptr() for t in d_dst])
    st = L.mmdit_probe_streams(srcs, nr, dsts, nw, n16 * 16, 3, unroll, sink.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    x = src[0].copy()
    for s in src[1:]:
        x ^= s
    for w, t in enumerate(d_dst):
        want = x.copy()
        want[:, 0] += np.uint32(w)
        assert np.array_equal(t.cpu().numpy().view(np.uint32), want), f"destination {w}"


def test_copy_probe_copies(L):
    n = (1 << 20) + 16 * 37
    a = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    b = torch.zeros_like(a)
    assert L.mmdit_probe_copy(a.data_ptr(), b.data_ptr(), n, 5, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, b)
