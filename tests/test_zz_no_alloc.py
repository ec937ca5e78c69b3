"""GPU: w4a8_linear_noalloc (static device scratch, no workspace argument)
against w4a8_linear with a caller workspace, through the C ABI.

The two run the same kernels, so the outputs must be the same bits; each is
also checked against the oracle on a window.  Calls come in pairs, the second
smaller than the first, so a call that reused stale scratch contents from the
larger one would show.  Paths covered: the prefill tail slices (the largest
scratch use), the M <= 16 kernel with and without in-kernel quantisation, and
the GEMV with split K (its scale slot lives in the scratch).
"""
import ctypes
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 4e-3


@pytest.fixture(scope="module")
def w4():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_amd as w4
    w4.load()
    return w4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_tensor(lin):
    x = lin["x"]
    if x.dtype == np.uint16:
        return dev(x.view(np.int16)).view(torch.bfloat16)
    return dev(x)


def noalloc(w4, x, W, y):
    lib = w4.load()
    dt = 0 if x.dtype == torch.bfloat16 else 1
    M, K = x.shape
    return lib.w4a8_linear_noalloc(x.data_ptr(), dt, W.buf.data_ptr(), W.buf.numel(), M, W.N, K,
                                   128, y.data_ptr(), torch.cuda.current_stream().cuda_stream)


PAIRS = [((512, 3584, 18944), (300, 1024, 4096)),
         ((4, 18944, 3584), (2, 3584, 512)),
         ((1, 18944, 512), (1, 3584, 512)),
         ((16, 18944, 3584), (5, 1024, 272))]


@pytest.mark.parametrize("pair", PAIRS, ids=[f"M{a[0]}_K{a[1]}_N{a[2]}_then_M{b[0]}" for a, b in PAIRS])
def test_noalloc_equals_linear(w4, pair):
    for i, (M, K, N) in enumerate(pair):
        say(f"noalloc call {i + 1}: M={M} K={K} N={N}")
        spec = synth.LinearSpec(f"noalloc_{M}_{K}_{N}", M, K, N, seed=900 + M + K + N)
        lin = synth.make_linear(spec)
        W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
        x = x_tensor(lin)
        y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        rc = noalloc(w4, x, W, y)
        assert rc == 0, w4.load().w4a8_last_error()
        ref_lib = w4.linear(x, W)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref_lib.view(torch.int16))
        qa_ref, sa_ref = oracle.quant_act(lin["x"])
        m1 = min(M, 4)
        ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(0, m1))
        ok, err, bound = oracle.tolerance_ok(y[:m1].float().cpu().numpy(), ref, REL)
        assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"


def test_noalloc_rejects_oversize(w4):
    """A shape whose workspace exceeds the static scratch is refused before
    anything is enqueued; the output is untouched."""
    M, K, N = 8192, 8192, 256
    lib = w4.load()
    assert lib.w4a8_linear_workspace_bytes(M, N, K, 128) > w4.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    W = w4.PackedWeight(torch.zeros(w4.packed_weight_bytes(N, K), dtype=torch.uint8, device="cuda"),
                        N, K, 128, lib.w4a8_layout_version())
    y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc(w4, x, W, y) == -4
    assert b"static scratch" in lib.w4a8_last_error()
    torch.cuda.synchronize()
    assert torch.all(y.float() == 5.0)
