"""GPU: no kernel writes outside the buffers it is given.

"Serve a pre-quantized int8 weight-only DiT ...", comment "Directive ...":
stripes at the borders of parallel output tiles were that page's symptom of a
kernel writing where it should not.  Every output, debug-partials and
workspace buffer here sits between two guard bands of a known byte pattern,
inside one larger allocation; after each call (on every path, at ragged M and
N, with split K, with the prefill's tail slices, and on the fused entry
points) the guards must be unchanged and the result must still match the
oracle.  Nothing here is meant to fault: the kernels run on valid inputs.
"""
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 4e-3
GUARD = 4096


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


class Guarded:
    """nbytes of device memory between two GUARD-byte bands of a pattern."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        pat = (np.arange(2 * GUARD + self.n, dtype=np.int64) * 37 + 11) % 251
        self.full = dev(pat.astype(np.uint8))
        self.inner = self.full[GUARD:GUARD + self.n]

    def view(self, dtype, shape):
        return self.inner.view(dtype).view(shape)

    def check(self, what):
        torch.cuda.synchronize()
        pat = (np.arange(2 * GUARD + self.n, dtype=np.int64) * 37 + 11) % 251
        got = self.full.cpu().numpy()
        lo = np.flatnonzero(got[:GUARD] != pat[:GUARD])
        hi = np.flatnonzero(got[GUARD + self.n:] != pat[GUARD + self.n:])
        assert lo.size == 0 and hi.size == 0, (
            f"{what}: guard bytes changed (before: {lo[:8]}, after: {hi[:8]})")


def _check_y(y, lin, qa_ref, sa_ref, rows=None):
    m0, m1 = rows if rows else (0, lin["spec"].M)
    ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(m0, m1))
    ok, err, bound = oracle.tolerance_ok(y[m0:m1].float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"


def _paths(M):
    return [3, 4, 5] + ([2] if M <= 16 else []) + ([1] if M == 1 else [])


# (M, K, N): the M buckets and tile edges with a ragged N; split K on the
# GEMV and the M <= 16 kernel; the prefill's tail slices with a ragged last
# column tile; a GEMV grid of several rounds; 256 x 256 tiles whose partial
# round runs as 256 x 128 half tiles; the M <= 16 weight-streaming grid
# (N / 16 >= compute units, K <= 4096) with a ragged block split; the
# two-launch linear with the codes in the 16-row tiled layout (12 <= M <= 16)
SHAPES = [(1, 384, 208), (2, 384, 208), (5, 384, 208), (16, 384, 208), (17, 384, 208),
          (33, 384, 208), (129, 384, 208), (300, 384, 208), (1, 18944, 512), (8, 10240, 512),
          (300, 1024, 18992), (1, 3584, 38912), (2048, 1024, 9472),
          (3, 1280, 4112), (16, 4096, 9600), (14, 18944, 208)]


@pytest.mark.parametrize("M,K,N", SHAPES, ids=[f"M{m}_K{k}_N{n}" for m, k, n in SHAPES])
def test_w4a8_guards(w4, M, K, N):
    say(f"guards w4a8 M={M} K={K} N={N}")
    spec = synth.LinearSpec(f"guard_{M}_{K}_{N}", M, K, N, seed=500 + M + K + N)
    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    qa, sa = dev(qa_ref), dev(sa_ref)
    G = K // 128
    lib = w4.load()
    # plain GEMM (automatic path)
    yg = Guarded(M * N * 2)
    wsg = Guarded(max(w4.workspace_bytes(M, N, K), 16))
    y = w4.gemm(qa, sa, W, out=yg.view(torch.bfloat16, (M, N)), workspace=wsg.inner)
    yg.check("gemm y")
    wsg.check("gemm workspace")
    rows = (0, M) if M * N <= 300 * 208 else (0, 4)
    _check_y(y, lin, qa_ref, sa_ref, rows)
    # every forced path with guarded partials over a row window
    m0, m1 = (0, M) if M <= 20 else (M // 2 - 3, M // 2 + 5)
    P_ref = oracle.group_partials(qa_ref, lin["q"], lin["z"], m0=m0, m1=m1)
    for path in _paths(M):
        pg = Guarded((m1 - m0) * N * G * 4)
        yg2 = Guarded(M * N * 2)
        wsg2 = Guarded(max(w4.workspace_bytes(M, N, K), 16))
        P = pg.view(torch.int32, (m1 - m0, N, G))
        y2 = yg2.view(torch.bfloat16, (M, N))
        rc = lib.w4a8_gemm_debug(qa.data_ptr(), sa.data_ptr(), W.buf.data_ptr(), W.buf.numel(),
                                 M, N, K, 128, path, m0, m1, P.data_ptr(), y2.data_ptr(),
                                 wsg2.inner.data_ptr(), wsg2.n,
                                 torch.cuda.current_stream().cuda_stream)
        assert rc == 0, lib.w4a8_last_error()
        pg.check(f"partials path {path}")
        yg2.check(f"debug y path {path}")
        wsg2.check(f"debug workspace path {path}")
        assert np.array_equal(P.cpu().numpy(), P_ref), f"path {path}"
    # the fused entry point (one launch at M == 1 and for small M that fit)
    x = x_tensor(lin)
    yg3 = Guarded(M * N * 2)
    lws = Guarded(max(w4.linear_workspace_bytes(M, N, K), 16))
    y3 = w4.linear(x, W, out=yg3.view(torch.bfloat16, (M, N)), workspace=lws.inner)
    yg3.check("linear y")
    lws.check("linear workspace")
    assert torch.equal(y3.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(1, 384, 208), (4, 1024, 272), (17, 384, 208),
                                   (300, 1024, 18992), (16, 18944, 208)])
def test_w8a8_and_w4a16_guards(w4, M, K, N):
    say(f"guards w8a8/w4a16 M={M} K={K} N={N}")
    spec = synth.LinearSpec(f"guard8_{M}_{K}_{N}", M, K, N, seed=700 + M + K + N)
    lin8 = synth.make_w8_linear(spec)
    W8 = w4.w8a8_pack_weights(dev(lin8["qw"]), dev(lin8["sw"]))
    x8 = x_tensor(lin8)
    yg = Guarded(M * N * 2)
    ws = Guarded(max(w4.w8a8_linear_workspace_bytes(M, N, K), 16))
    y = w4.w8a8_linear(x8, W8, out=yg.view(torch.bfloat16, (M, N)), workspace=ws.inner)
    yg.check("w8a8 y")
    ws.check("w8a8 workspace")
    qa_ref, sa_ref = oracle.quant_act(lin8["x"])
    rows = (0, min(M, 4))
    ref = oracle.w8a8_linear(qa_ref, sa_ref, lin8["qw"], lin8["sw"], rows=rows)
    ok, err, bound = oracle.tolerance_ok(y[rows[0]:rows[1]].float().cpu().numpy(), ref, REL)
    assert ok, f"w8a8: {err:.3e} > {bound:.3e}"

    lin = synth.make_linear(spec)
    W = w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))
    x = x_tensor(lin)
    yg = Guarded(M * N * 2)
    ws = Guarded(max(w4.w4a16_workspace_bytes(M, N, K), 16))
    y = w4.w4a16_linear(x, W, out=yg.view(torch.bfloat16, (M, N)), workspace=ws.inner)
    yg.check("w4a16 y")
    ws.check("w4a16 workspace")
    ref = oracle.w4a16_linear(lin["x"][rows[0]:rows[1]], lin["q"], lin["z"], lin["s"])
    ok, err, bound = oracle.tolerance_ok(y[rows[0]:rows[1]].float().cpu().numpy(), ref, REL)
    assert ok, f"w4a16: {err:.3e} > {bound:.3e}"


def test_quant_guards(w4):
    say("guards quantiser")
    for M, K in ((1, 3584), (5, 18944), (300, 3584), (3, 70016)):
        lin = synth.make_linear(synth.LinearSpec("gq", M, K, 16, seed=M + K), with_weights=False)
        qg, sg = Guarded(M * K), Guarded(M * 4)
        qa = qg.view(torch.int8, (M, K))
        sa = sg.view(torch.float32, (M,))
        w4.quant_act(x_tensor(lin), qa, sa)
        qg.check(f"qa M={M} K={K}")
        sg.check(f"sa M={M} K={K}")
        qa_ref, sa_ref = oracle.quant_act(lin["x"])
        assert np.array_equal(qa.cpu().numpy(), qa_ref)
        w4.quant_act_hadamard(x_tensor(lin), qa, sa)
        qg.check(f"hadamard qa M={M} K={K}")
        sg.check(f"hadamard sa M={M} K={K}")
