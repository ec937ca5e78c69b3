"""GPU: activation matrices of 2^31 bytes or more on the prefill paths.

The prefill kernels address one launch's activations with 32-bit offsets, so
the library runs a taller matrix as consecutive row chunks of whole 256-row
tiles.  Each test builds such a matrix on the GPU by repeating a seeded block
of R = 4099 rows (so the rows on either side of a chunk boundary differ) and
checks it against the oracle:
- bit-exact per-group partials (W4A8) or int32 totals (W8A8) over a row
  window that straddles the first chunk boundary;
- the bf16 output on sampled rows (the first, around the boundary, the last)
  to max|y - y_ref| <= 4e-3 * max|y_ref|;
- the plain entry point's output equal, byte for byte, to the debug call's.
"""
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL = 4e-3
R = 4099        # rows of the repeated block
K, N = 128, 16
LIMIT = 2**31 - 1


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


def tiled(block: np.ndarray, M: int) -> torch.Tensor:
    """Row m of the result is row m % R of the block (built on the GPU)."""
    b = dev(block)
    idx = torch.arange(M, device="cuda") % R
    out = b[idx]
    del idx
    return out


def first_chunk_rows(bytes_per_row: int) -> int:
    rows = LIMIT // bytes_per_row
    return rows // 256 * 256


def sample_rows(M: int, B: int) -> np.ndarray:
    return np.unique(np.r_[0:8, B - 8:B + 8, M - 8:M])


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy()


def test_w4a8_prefill_row_chunks(w4):
    M = 1 << 24                      # the largest M the library takes; M*K = 2^31 bytes
    B = first_chunk_rows(K)
    assert M * K > LIMIT and B < M
    say(f"w4a8 prefill row chunks M={M} K={K} N={N} boundary={B}")
    rng = np.random.Generator(np.random.PCG64(2031))
    xb, _ = synth.draw_activations(rng, R, K, "bf16_outliers")
    qa_b, sa_b = oracle.quant_act(xb)
    q, z, s = synth.draw_weights(rng, N, K)
    W = w4.pack_weights(dev(q), dev(z), dev(s))
    qa, sa = tiled(qa_b, M), tiled(sa_b, M)
    window = (B - 8, B + 8)
    P, y = w4.gemm_debug(qa, sa, W, path=w4.PATH_PREFILL, rows=window)
    wrows = np.arange(*window) % R
    assert np.array_equal(P.cpu().numpy(), oracle.group_partials(qa_b[wrows], q, z))
    rows = sample_rows(M, B)
    rows_t = torch.from_numpy(rows).cuda()
    ref = oracle.linear(qa_b[rows % R], sa_b[rows % R], q, z, s)
    ok, err, bound = oracle.tolerance_ok(y[rows_t].float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"
    y2 = w4.gemm(qa, sa, W)
    assert np.array_equal(bits(y2[rows_t]), bits(y[rows_t]))
    del qa, sa, y, y2
    torch.cuda.empty_cache()


def test_w8a8_prefill_row_chunks(w4):
    M = 1 << 24
    B = first_chunk_rows(K)
    say(f"w8a8 prefill row chunks M={M} K={K} N={N} boundary={B}")
    rng = np.random.Generator(np.random.PCG64(2032))
    xb, _ = synth.draw_activations(rng, R, K, "bf16_outliers")
    qa_b, sa_b = oracle.quant_act(xb)
    qw, sw = synth.draw_w8_weights(rng, N, K)
    W = w4.w8a8_pack_weights(dev(qw), dev(sw))
    qa, sa = tiled(qa_b, M), tiled(sa_b, M)
    window = (B - 8, B + 8)
    T, y = w4.w8a8_gemm_debug(qa, sa, W, path=w4.PATH_PREFILL, rows=window)
    wrows = np.arange(*window) % R
    assert np.array_equal(T.cpu().numpy(), oracle.w8a8_totals(qa_b[wrows], qw))
    rows = sample_rows(M, B)
    rows_t = torch.from_numpy(rows).cuda()
    ref = oracle.w8a8_linear(qa_b[rows % R], sa_b[rows % R], qw, sw)
    ok, err, bound = oracle.tolerance_ok(y[rows_t].float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"
    y2 = w4.w8a8_gemm(qa, sa, W)
    assert np.array_equal(bits(y2[rows_t]), bits(y[rows_t]))
    del qa, sa, y, y2
    torch.cuda.empty_cache()


def test_w4a16_prefill_row_chunks(w4):
    B = first_chunk_rows(2 * K)      # bf16 rows: two bytes per value
    M = B + 300
    assert 2 * M * K > LIMIT
    say(f"w4a16 prefill row chunks M={M} K={K} N={N} boundary={B}")
    rng = np.random.Generator(np.random.PCG64(2033))
    xb, _ = synth.draw_activations(rng, R, K, "bf16_outliers")
    q, z, s = synth.draw_weights(rng, N, K)
    W = w4.pack_weights(dev(q), dev(z), dev(s))
    x = tiled(xb.view(np.int16), M).view(torch.bfloat16)
    assert w4.w4a16_select_path(M, N, K) == w4.PATH_PREFILL
    y = w4.w4a16_linear(x, W)
    rows = sample_rows(M, B)
    rows_t = torch.from_numpy(rows).cuda()
    ref = oracle.w4a16_linear(xb[rows % R], q, z, s)
    ok, err, bound = oracle.tolerance_ok(y[rows_t].float().cpu().numpy(), ref, REL)
    assert ok, f"max|y - y_ref| = {err:.3e} > {bound:.3e}"
    del x, y
    torch.cuda.empty_cache()
