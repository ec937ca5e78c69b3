"""GPU parity of the two-launch linears at 12 <= M <= 16 on the M <= 16
kernel, where the workspace holds the codes in the 16-row tiled layout
([K / 16][16 rows][16 B]) that the kernel reads as matrix-core operands.

The codes and the GEMM arithmetic are those of w4a8_quant_act + w4a8_gemm
(row-major codes), so the bar is bitwise equality with that pair, plus
max|y - y_ref| <= 4e-3 * max|y_ref| against the oracle on sampled rows.
"The 4-bit CPU path", section "W4A8": per-token int8 activations times the
int4 weights.  The shapes: the 7B down projection at M = 16 (K = 18944 ->
N = 3584), M = 12 with float input, a K split (K = 8192 -> N = 2048), more
channel blocks than compute units with a K past the weight-streaming grid
(K = 5120 -> N = 8192), and the rotated linear.  Rows M..15 of the tiled
layout are never written: the workspace is filled with random bytes first,
and a call at M = 16 runs before one at M = 12 on the same workspace.
"""
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


def round256(v):
    return (v + 255) // 256 * 256


def tiled_workspace(w4, M, N, K, seed):
    """A workspace of the linear's size, filled with random bytes; its size
    shows the tiled route (16 K bytes of codes) is the one taken."""
    need = w4.linear_workspace_bytes(M, N, K)
    assert need == round256(16 * K) + round256(4 * M) + w4.workspace_bytes(M, N, K)
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=g)


# (M, K, N, x dtype): down projection; M = 12 float; K split; N / 16 > CUs
SHAPES = [(16, 18944, 3584, "bf16_outliers"), (12, 18944, 3584, "f32"),
          (13, 8192, 2048, "bf16_outliers"), (14, 5120, 8192, "bf16_outliers")]


@pytest.mark.parametrize("M,K,N,xd", SHAPES, ids=[f"M{m}_K{k}_N{n}_{d}" for m, k, n, d in SHAPES])
def test_tiled_linear(w4, M, K, N, xd):
    say(f"tiled linear M={M} K={K} N={N} {xd}")
    spec = synth.LinearSpec(f"tiled_{M}_{K}_{N}", M, K, N, seed=1200 + M + K // 128, act=xd)
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = x_tensor(lin)
    ws = tiled_workspace(w4, M, N, K, seed=M)
    y = w4.linear(x, W, workspace=ws)
    qa, sa = w4.quant_act(x)
    y_two = w4.gemm(qa, sa, W)
    assert torch.equal(y.view(torch.int16), y_two.view(torch.int16))
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    yn = y.float().cpu().numpy()
    for rows in ((0, 1), (M - 1, M)):
        ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=rows)
        ok, err, bound = oracle.tolerance_ok(yn[rows[0]:rows[1]], ref, REL)
        assert ok, f"rows {rows}: max|y - y_ref| = {err:.3e} > {bound:.3e}"


def test_tiled_stale_rows(w4):
    """M = 16 then M = 12 on one workspace: rows 12..15 of the tiled codes
    still hold the first call's codes, and the second output is unchanged by
    them (bitwise that of quant + gemm)."""
    K, N = 18944, 3584
    lin16 = synth.make_linear(synth.LinearSpec("tiled_stale16", 16, K, N, seed=1301))
    lin12 = synth.make_linear(synth.LinearSpec("tiled_stale12", 12, K, N, seed=1302))
    W = w4.pack_weights(dev(lin12["q"]), dev(lin12["z"]), dev(lin12["s"]))
    ws = tiled_workspace(w4, 16, N, K, seed=5)
    assert ws.numel() >= w4.linear_workspace_bytes(12, N, K)
    w4.linear(x_tensor(lin16), W, workspace=ws)
    x12 = x_tensor(lin12)
    y = w4.linear(x12, W, workspace=ws)
    qa, sa = w4.quant_act(x12)
    assert torch.equal(y.view(torch.int16), w4.gemm(qa, sa, W).view(torch.int16))


def test_tiled_hadamard(w4):
    """The rotated linear at M = 12 takes the same route: bitwise the output
    of w4a8_quant_act_hadamard + w4a8_gemm."""
    M, K, N = 12, 18944, 3584
    lin = synth.make_linear(synth.LinearSpec("tiled_had", M, K, N, seed=1310))
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = x_tensor(lin)
    y = w4.linear_hadamard(x, W)
    qa, sa = w4.quant_act_hadamard(x)
    assert torch.equal(y.view(torch.int16), w4.gemm(qa, sa, W).view(torch.int16))


def test_tiled_w8a8(w4):
    """The W8A8 linear's two-launch route at M = 16 and 14 takes the tiled
    codes too: bitwise the output of w4a8_quant_act + w8a8_gemm, and within
    the bar of the oracle's W8A8 product on the first and last rows."""
    K, N = 18944, 3584
    for M in (16, 14):
        say(f"tiled w8a8 M={M}")
        lin = synth.make_w8_linear(synth.LinearSpec(f"tiled_w8_{M}", M, K, N, seed=1320 + M))
        W = w4.w8a8_pack_weights(dev(lin["qw"]), dev(lin["sw"]))
        need = w4.w8a8_linear_workspace_bytes(M, N, K)
        assert need == round256(16 * K) + round256(4 * M) + w4.w8a8_workspace_bytes(M, N, K)
        x = x_tensor(lin)
        y = w4.w8a8_linear(x, W)
        qa, sa = w4.quant_act(x)
        assert torch.equal(y.view(torch.int16), w4.w8a8_gemm(qa, sa, W).view(torch.int16))
        qa_ref, sa_ref = oracle.quant_act(lin["x"])
        yn = y.float().cpu().numpy()
        for rows in ((0, 1), (M - 1, M)):
            ref = oracle.w8a8_linear(qa_ref, sa_ref, lin["qw"], lin["sw"], rows=rows)
            ok, err, bound = oracle.tolerance_ok(yn[rows[0]:rows[1]], ref, REL)
            assert ok, f"M={M} rows {rows}: max|y - y_ref| = {err:.3e} > {bound:.3e}"
