"""GPU parity of the online Hadamard rotation + per-token quantisation (and
the layer built on it) through the C ABI against the CPU oracle.

The packed QuaRot model of "EgoPQ Real-Serving Handoff" (section "1. Source
Checkpoint") rotates activations before quantising them.  Here each group of
128 input channels is multiplied by the unnormalised 128 x 128
Walsh-Hadamard matrix in float32 by butterflies of increasing stride, on both
sides, so the rotated values and hence the codes are compared bit for bit;
the layer's bf16 output is held to max|y - y_ref| <= 4e-3 * max|y_ref|.
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


def x_tensor(x):
    if x.dtype == np.uint16:
        return dev(x.view(np.int16)).view(torch.bfloat16)
    return dev(x)


# every quantiser variant: one row per workgroup holding 1, 2, 4 or 8 chunks
# of eight per thread (ragged and exact), the two-pass kernel for many rows
# and for long rows, bf16 with outlier channels and float32
HAD_CASES = [(1, 3584, "bf16_outliers"), (3, 8192, "bf16_outliers"), (2, 8320, "f32"),
             (4, 18944, "bf16_outliers"), (5, 32896, "f32"), (1, 65536, "bf16_outliers"),
             (2, 65664, "bf16_outliers"), (65, 1024, "f32"), (300, 3584, "bf16_outliers"),
             (2048, 3584, "bf16_outliers"), (100, 8192, "f32"), (80, 16384, "bf16_outliers"),
             (70, 16512, "bf16_outliers")]


@pytest.mark.parametrize("M,K,act", HAD_CASES, ids=[f"M{m}_K{k}_{a[:4]}" for m, k, a in HAD_CASES])
def test_hadamard_quant_bit_exact(w4, M, K, act):
    say(f"hadamard quant M={M} K={K} {act}")
    lin = synth.make_linear(synth.LinearSpec("had", M, K, 16, seed=M * 3 + K, act=act),
                            with_weights=False)
    qa, sa = w4.quant_act_hadamard(x_tensor(lin["x"]))
    qa_ref, sa_ref = oracle.hadamard_quant_act(lin["x"])
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(qa.cpu().numpy(), qa_ref)


def test_hadamard_special_rows(w4):
    """A zero row (scale 0, codes 0), a unit row (every code +-127 in its
    group), and integer rows whose rotation is exact."""
    say("hadamard special rows")
    K = 512
    rng = np.random.Generator(np.random.PCG64(43))
    x = np.zeros((4, K), np.float32)
    x[1, 130] = 1.0
    x[2] = rng.integers(-50, 51, size=K)
    x[3] = rng.standard_normal(K)
    qa, sa = w4.quant_act_hadamard(dev(x))
    qa_ref, sa_ref = oracle.hadamard_quant_act(x)
    assert np.array_equal(qa.cpu().numpy(), qa_ref)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_ref.view(np.uint32))
    q = qa.cpu().numpy()
    assert sa_ref[0] == 0 and not q[0].any()
    assert np.all(np.abs(q[1, 128:256].astype(int)) == 127) and not q[1, :128].any()


# M = 1 and the M <= 16 kernels quantise (and rotate) in the kernel: bf16 and
# f32, one and two token batches (K = 32768), every row bucket; M = 16 at
# K = 18944 and M = 300 take the two-launch path.
LIN_CASES = [synth.LinearSpec("hadl_m1", 1, 3584, 18944, seed=97),
             synth.LinearSpec("hadl_m1_k32768_f32", 1, 32768, 256, seed=101, act="f32"),
             synth.LinearSpec("hadl_m2_f32", 2, 4096, 1024, seed=102, act="f32"),
             synth.LinearSpec("hadl_m4", 4, 18944, 3584, seed=98),
             synth.LinearSpec("hadl_m9", 9, 2048, 512, seed=103),
             synth.LinearSpec("hadl_m16_k3584", 16, 3584, 512, seed=104),
             synth.LinearSpec("hadl_m16_two_launch", 16, 18944, 256, seed=105),
             synth.LinearSpec("hadl_m300", 300, 1024, 528, seed=99, act="f32")]


@pytest.mark.parametrize("spec", LIN_CASES, ids=[s.name for s in LIN_CASES])
def test_hadamard_linear(w4, spec):
    say(f"hadamard linear {spec}")
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = x_tensor(lin["x"])
    y = w4.linear_hadamard(x, W)
    qa, sa = w4.quant_act_hadamard(x)
    assert torch.equal(y, w4.gemm(qa, sa, W))
    qa_ref, sa_ref = oracle.hadamard_quant_act(lin["x"])
    m1 = min(spec.M, 16)
    ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(0, m1))
    ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy()[:m1], ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"


# The M = 1 GEMV quantises (or stages) the token in several batches when K is
# large, and its quantiser wavefronts then stream runs that read codes and
# sums the other quantisers wrote: every one of them must wait for all.  The
# fused step is repeated and compared bit for bit with quantise + GEMM (and,
# for W4A16, with its own first result), so a wavefront that ran ahead would
# show as a mismatch.
@pytest.mark.parametrize("act,had", [("f32", True), ("f32", False), ("bf16_outliers", True),
                                     ("bf16_outliers", False)])
def test_gemv_multibatch_token_repeat(w4, act, had):
    say(f"gemv multibatch token act={act} hadamard={had}")
    spec = synth.LinearSpec(f"gemv_mb_{act}", 1, 32768, 512, seed=131, act=act)
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = x_tensor(lin["x"])
    quant = w4.quant_act_hadamard if had else w4.quant_act
    linear = w4.linear_hadamard if had else w4.linear
    qa, sa = quant(x)
    ref = w4.gemm(qa, sa, W)
    for i in range(12):
        assert torch.equal(linear(x, W), ref), f"repeat {i}"
    if not had and act == "bf16_outliers":  # (W4A16 takes bf16 activations)
        first = w4.w4a16_linear(x, W)
        for i in range(12):
            assert torch.equal(w4.w4a16_linear(x, W), first), f"w4a16 repeat {i}"
