"""GPU parity of the W8A8 int8-dynamic linear through the C ABI against the
CPU oracle.

"Serve a pre-quantized int8 weight-only DiT ...", comment "Round two ...":
int8 weights with per-channel scales, activations quantised to int8 at run
time, an integer product scaled afterwards, checked one linear at a time
against a reference that carries the activation scale.

Bars: the packed bytes and the int32 totals P[m][n] bit-exact on every path;
max|y - y_ref| <= 4e-3 * max|y_ref| per tensor for the bf16 output (y_ref the
oracle's unrounded float64); and, since P is exact and the epilogue fixed,
y bitwise equal across paths and between w8a8_linear and quant + gemm.
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


def x_tensor(lin):
    x = lin["x"]
    if x.dtype == np.uint16:
        return dev(x.view(np.int16)).view(torch.bfloat16)
    return dev(x)


def _setup(w4, spec):
    lin = synth.make_w8_linear(spec)
    W = w4.w8a8_pack_weights(dev(lin["qw"]), dev(lin["sw"]))
    return lin, W


def _windows(M):
    if M <= 64:
        return [(0, M)]
    return [(0, 24), (M // 2 - 5, M // 2 + 5), (M - 24, M)]


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (512, 3584), (3584, 18944)])
def test_w8_pack_bytes_and_round_trip(w4, N, K):
    say(f"w8 pack N={N} K={K}")
    rng = np.random.Generator(np.random.PCG64(N * 7 + K))
    qw, sw = synth.draw_w8_weights(rng, N, K)
    W = w4.w8a8_pack_weights(dev(qw), dev(sw))
    assert np.array_equal(W.buf.cpu().numpy(), oracle.w8_layout_pack(qw, sw))
    qw2, sw2 = w4.w8a8_unpack_weights(W)
    assert np.array_equal(qw2.cpu().numpy(), qw)
    assert np.array_equal(sw2.cpu().numpy().view(np.uint32), sw.view(np.uint32))


# M across the buckets and the kernels' edges: M = 1 (decode), every
# power-of-two row bucket of the M <= 16 kernel and its neighbours, prefill
# tile edges (256 rows, 128 channels, ragged N), split K on both paths, and
# the decode / skinny / prefill shapes of the 7B layer at full size.
W8_SPECS = [
    synth.LinearSpec("w8_m1_decode_up", 1, 3584, 18944, seed=80),
    synth.LinearSpec("w8_m1_ksplit", 1, 18944, 512, seed=81),
    synth.LinearSpec("w8_m1_ragged", 1, 1152, 4112, seed=97),
    synth.LinearSpec("w8_m1_down", 1, 18944, 3584, seed=98),
    synth.LinearSpec("w8_m2", 2, 256, 256, seed=82, act="f32"),
    synth.LinearSpec("w8_m3", 3, 640, 272, seed=83),
    synth.LinearSpec("w8_m4", 4, 1024, 512, seed=84),
    synth.LinearSpec("w8_m8", 8, 3584, 1024, seed=85),
    synth.LinearSpec("w8_m9", 9, 384, 4096, seed=86),
    synth.LinearSpec("w8_m16_down", 16, 18944, 3584, seed=87),
    synth.LinearSpec("w8_m17", 17, 512, 272, seed=88),
    synth.LinearSpec("w8_m300", 300, 1024, 528, seed=89, act="f32"),
    synth.LinearSpec("w8_m512_ksplit", 512, 3584, 512, seed=90),
    synth.LinearSpec("w8_m2048_up", 2048, 3584, 18944, seed=91),
    # one round of tiles plus a partial one: the partial round runs as K slices
    synth.LinearSpec("w8_m512_tail", 512, 3584, 18944, seed=99),
    synth.LinearSpec("w8_m300_tail_ragged", 300, 1024, 18992, seed=100),
]


@pytest.mark.parametrize("spec", W8_SPECS, ids=[s.name for s in W8_SPECS])
def test_w8_totals_and_output(w4, spec):
    say(f"w8 totals {spec}")
    lin, W = _setup(w4, spec)
    qa, sa = w4.quant_act(x_tensor(lin))
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_ref.view(np.uint32))
    paths = ([GEMV] if spec.M == 1 else []) + ([SKINNY] if spec.M <= 16 else []) + [PREFILL]
    ys = {}
    for path in paths:
        for (m0, m1) in _windows(spec.M):
            P, y = w4.w8a8_gemm_debug(qa, sa, W, path=path, rows=(m0, m1))
            P_ref = oracle.w8a8_totals(qa_ref, lin["qw"], m0=m0, m1=m1)
            assert np.array_equal(P.cpu().numpy(), P_ref), (path, m0, m1)
            ref = oracle.w8a8_linear(qa_ref, sa_ref, lin["qw"], lin["sw"], rows=(m0, m1))
            got = y.float().cpu().numpy()[m0:m1]
            ok, err, bound = oracle.tolerance_ok(got, ref, REL)
            assert ok, f"path {path} rows {m0}:{m1}: max|y - y_ref| = {err:.3e} > {bound:.3e}"
        ys[path] = y
    y_auto = w4.w8a8_gemm(qa, sa, W)
    for path, y in ys.items():
        assert torch.equal(y, y_auto), f"path {path} differs from AUTO"


W8_LINEAR_SPECS = [
    synth.LinearSpec("w8l_m1", 1, 3584, 3584, seed=92),
    synth.LinearSpec("w8l_m1_ksplit_f32", 1, 18944, 512, seed=99, act="f32"),
    synth.LinearSpec("w8l_m4_fused", 4, 18944, 3584, seed=93),
    synth.LinearSpec("w8l_m16_fused_f32", 16, 2048, 2048, seed=94, act="f32"),
    synth.LinearSpec("w8l_m16_two_launch", 16, 18944, 512, seed=95),
    synth.LinearSpec("w8l_m100", 100, 1024, 1024, seed=96),
]


@pytest.mark.parametrize("spec", W8_LINEAR_SPECS, ids=[s.name for s in W8_LINEAR_SPECS])
def test_w8_linear_matches_quant_then_gemm(w4, spec):
    say(f"w8 linear {spec}")
    lin, W = _setup(w4, spec)
    x = x_tensor(lin)
    y = w4.w8a8_linear(x, W)
    qa, sa = w4.quant_act(x)
    assert torch.equal(y, w4.w8a8_gemm(qa, sa, W))
    assert torch.equal(w4.w8a8_linear(x, W), y)
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    m1 = min(spec.M, 24)
    ref = oracle.w8a8_linear(qa_ref, sa_ref, lin["qw"], lin["sw"], rows=(0, m1))
    ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy()[:m1], ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"


def test_w8_extreme_values(w4):
    """Full-range codes: +127 activations against -127 weights on every k,
    the largest |P| a K = 8192 product can reach (127 * 127 * 8192), on both
    paths."""
    say("w8 extremes")
    M, K, N = 16, 8192, 256
    x = np.full((M, K), 1.0, np.float32)
    x[1::2] *= -1.0
    qw = np.full((N, K), -127, np.int8)
    qw[::3] = 127
    sw = np.full((N,), 0.5, np.float32)
    W = w4.w8a8_pack_weights(dev(qw), dev(sw))
    qa, sa = w4.quant_act(dev(x))
    P_ref = oracle.w8a8_totals(oracle.quant_act(x)[0], qw)
    assert np.abs(P_ref.astype(np.int64)).max() == 127 * 127 * K
    for path in (SKINNY, PREFILL):
        P, _ = w4.w8a8_gemm_debug(qa, sa, W, path=path)
        assert np.array_equal(P.cpu().numpy(), P_ref), path
    for m in (0, 1):  # one row at a time through the GEMV
        P, _ = w4.w8a8_gemm_debug(qa[m:m + 1].clone(), sa[m:m + 1].clone(), W, path=GEMV)
        assert np.array_equal(P.cpu().numpy(), P_ref[m:m + 1]), ("gemv", m)
