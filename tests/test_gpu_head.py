"""GPU parity for the 7B-shaped output head, K = 3584 -> N = 152064, at full
width ("The 4-bit CPU path", section "W4A8": left unquantised, the head alone
costs 2.97 ms per step, so it is packed like every other linear).

At M = 1 the head runs the decode GEMV on a grid of several rounds of
workgroups over the compute units; at M = 512 the prefill tiles fill whole
rounds plus part of one, whose tiles (the last column tiles) run as K slices
reduced by a second kernel.  Bars: per-group int32 partials bit-exact for
every channel, bf16 y within 4e-3 * max|y_ref| over whole rows.
"""
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 4e-3
K, N = 3584, 152064


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
    return dev(lin["x"].view(np.int16)).view(torch.bfloat16)


def head(w4, M):
    spec = next(s for s in synth.layer_specs(M) if s.name.startswith("layer_head"))
    assert (spec.K, spec.N) == (K, N)
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    return lin, W, qa_ref, sa_ref


def check_rows(y, lin, qa_ref, sa_ref, m0, m1):
    ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(m0, m1))
    ok, err, bound = oracle.tolerance_ok(y[m0:m1].float().cpu().numpy(), ref, REL)
    assert ok, f"rows {m0}:{m1}: max|y - y_ref| = {err:.3e} > {bound:.3e}"


def test_head_decode_full_width(w4):
    say("head M=1: GEMV partials for all 9504 channel blocks, y over the whole row")
    lin, W, qa_ref, sa_ref = head(w4, 1)
    assert w4.select_path(1, N, K) == w4.PATH_GEMV
    x = x_tensor(lin)
    qa, sa = w4.quant_act(x)
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_ref.view(np.uint32))
    P, y_dbg = w4.gemm_debug(qa, sa, W, path=w4.PATH_GEMV)
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa_ref, lin["q"], lin["z"]))
    y = w4.gemm(qa, sa, W)
    assert torch.equal(y_dbg.view(torch.int16), y.view(torch.int16))
    check_rows(y, lin, qa_ref, sa_ref, 0, 1)
    # the fused decode step (quantisation inside the GEMV) is the same bits
    assert torch.equal(w4.linear(x, W).view(torch.int16), y.view(torch.int16))


def test_head_prefill_full_width(w4):
    M = 512
    say("head M=512: prefill partials across both row tiles, every column")
    lin, W, qa_ref, sa_ref = head(w4, M)
    assert w4.select_path(M, N, K) == w4.PATH_PREFILL
    assert w4.workspace_bytes(M, N, K) > 0        # the partial round's K slices
    qa, sa = dev(qa_ref), dev(sa_ref)
    y = w4.gemm(qa, sa, W)
    rows = (254, 258)                            # two rows of each 256-row tile
    P, y_dbg = w4.gemm_debug(qa, sa, W, path=w4.PATH_PREFILL, rows=rows)
    P_ref = oracle.group_partials(qa_ref, lin["q"], lin["z"], m0=rows[0], m1=rows[1])
    assert np.array_equal(P.cpu().numpy(), P_ref)
    assert torch.equal(y_dbg.view(torch.int16), y.view(torch.int16))
    say("head M=512: y over whole rows of both row tiles")
    for m0, m1 in ((0, 2), (255, 257), (510, 512)):
        check_rows(y, lin, qa_ref, sa_ref, m0, m1)
    # the layer entry point (quantisation, then the GEMM) gives the same bits
    assert torch.equal(w4.linear(x_tensor(lin), W).view(torch.int16), y.view(torch.int16))
