"""GPU parity of the W4A16 linear (bf16 activations x the packed int4
weights) through the C ABI against the CPU oracle.

"The 4-bit CPU path", section "W4A16": the activations stay bf16, and small
and large batches take different kernels.  Each group's products are summed
in float32 on the bf16 matrix cores and scaled by the group's scale, so the
output is held to max|y - y_ref| <= 4e-3 * max|y_ref| against the oracle's
unrounded float64 value (no integer stage to compare bit for bit).
"""
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 4e-3
GEMV, SKINNY, PREFILL = 1, 2, 3


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


def _check(y, lin, rows):
    m0, m1 = rows
    ref = oracle.w4a16_linear(lin["x"], lin["q"], lin["z"], lin["s"], rows=(m0, m1))
    ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy()[m0:m1], ref, REL)
    assert ok, f"rows {m0}:{m1}: max|y - y_ref| = {err:.3e} > {bound:.3e}"


# M <= 16: every row bucket, rows staged in LDS where they fit and A operands
# loaded straight from memory where they do not (m4/m16 down, m6, m13: the
# last with a K split to fill the machine), ragged and small N; M > 16:
# prefill tiles of 128 tokens with ragged M and N, split K, full size
A16_SPECS = [
    synth.LinearSpec("a16_m1_up", 1, 3584, 18944, seed=110),
    synth.LinearSpec("a16_m1_k", 1, 3584, 512, seed=111),
    synth.LinearSpec("a16_m1_down", 1, 18944, 3584, seed=123),
    synth.LinearSpec("a16_m1_tiny", 1, 128, 16, seed=124),
    synth.LinearSpec("a16_m1_kmax", 1, 32768, 256, seed=125),
    synth.LinearSpec("a16_m1_ragged", 1, 1152, 4112, seed=126),
    synth.LinearSpec("a16_m2", 2, 640, 272, seed=112),
    synth.LinearSpec("a16_m3", 3, 1024, 512, seed=113),
    synth.LinearSpec("a16_m4_down", 4, 18944, 3584, seed=114),
    synth.LinearSpec("a16_m8", 8, 4096, 1024, seed=115),
    synth.LinearSpec("a16_m16_down", 16, 18944, 3584, seed=116),
    synth.LinearSpec("a16_m16_small_k", 16, 256, 2048, seed=117),
    synth.LinearSpec("a16_m6_direct", 6, 24576, 4096, seed=128),
    synth.LinearSpec("a16_m13_direct_ksplit", 13, 18944, 400, seed=129),
    synth.LinearSpec("a16_m17", 17, 512, 272, seed=118),
    synth.LinearSpec("a16_m300", 300, 1024, 528, seed=119),
    synth.LinearSpec("a16_m512_ksplit", 512, 3584, 512, seed=120),
    synth.LinearSpec("a16_m2048_up", 2048, 3584, 18944, seed=121),
    # 2384 tiles: 9 rounds and 80 tiles, the last column tile ragged; the
    # partial round runs as K slices
    synth.LinearSpec("a16_m2048_tail_ragged", 2048, 3584, 18960, seed=130),
]


def _rows(M):
    return [(0, M)] if M <= 64 else [(0, 24), (M - 24, M)]


@pytest.mark.parametrize("spec", A16_SPECS, ids=[s.name for s in A16_SPECS])
def test_w4a16_linear(w4, spec):
    say(f"w4a16 {spec}")
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = dev(lin["x"].view(np.int16)).view(torch.bfloat16)
    y = w4.w4a16_linear(x, W)
    for rows in _rows(spec.M):
        _check(y, lin, rows)
    assert torch.equal(w4.w4a16_linear(x, W), y)          # deterministic
    if spec.M == 1:
        assert w4.w4a16_select_path(spec.M, spec.N, spec.K) == GEMV
        ys = w4.w4a16_linear(x, W, path=SKINNY)           # the M <= 16 kernel, same row
        _check(ys, lin, (0, 1))
    if 1 < spec.M <= 16:
        ys = w4.w4a16_linear(x, W, path=SKINNY)           # both M <= 16 paths, same rows
        _check(ys, lin, (0, spec.M))
    if spec.M <= 16:
        yp = w4.w4a16_linear(x, W, path=PREFILL)
        _check(yp, lin, (0, spec.M))


def test_w4a16_symmetric_grid(w4):
    say("w4a16 symmetric grid")
    lin = synth.make_linear(synth.LinearSpec("a16_sym", 5, 1024, 512, seed=122))
    W = w4.pack_weights(dev(lin["q"]), None, dev(lin["s"]))
    x = dev(lin["x"].view(np.int16)).view(torch.bfloat16)
    y = w4.w4a16_linear(x, W)
    z8 = np.full_like(lin["z"], 8)
    ref = oracle.w4a16_linear(lin["x"], lin["q"], z8, lin["s"])
    ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"


def test_w4a16_gemv_symmetric_and_zero_token(w4):
    """M == 1 GEMV: symmetric grid (constant zero point 8), and an all-zero
    token gives exactly zero."""
    say("w4a16 gemv symmetric + zero token")
    lin = synth.make_linear(synth.LinearSpec("a16_m1_sym", 1, 2048, 1024, seed=127))
    W = w4.pack_weights(dev(lin["q"]), None, dev(lin["s"]))
    x = dev(lin["x"].view(np.int16)).view(torch.bfloat16)
    assert w4.w4a16_select_path(1, 1024, 2048) == GEMV
    y = w4.w4a16_linear(x, W, path=GEMV)
    z8 = np.full_like(lin["z"], 8)
    ref = oracle.w4a16_linear(lin["x"], lin["q"], z8, lin["s"])
    ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"
    y0 = w4.w4a16_linear(torch.zeros_like(x), W, path=GEMV)
    assert not torch.any(y0.float() != 0.0)
