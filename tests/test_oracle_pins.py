"""Pins for the CPU oracle: each check ties it to something other than itself.

- golden worked examples of the quantiser's rounding rule (tests/golden);
- invariants of symmetric per-token quantisation;
- brute force of the per-group integer products against numpy int64 matmul;
- zero-point shift equivalence, all-zero weights, in-group permutation;
- the float64 result against numpy dequant-then-matmul ("Serve a
  pre-quantized int8 weight-only DiT ...", comment "Directive ...": isolate
  one linear against a reference dequant-then-matmul; comment "Round two ...":
  that reference must carry the activation scale);
- the identity-scale case, which reduces to an exact integer GEMM;
- the packed layout against hand-worked bytes and a round trip;
- for the W8A8 linear: integer totals against numpy int64 matmul and closed
  forms, the float64 result against numpy dequant-then-matmul, and the exact
  agreement with the W4A8 oracle on weights both can express (int8 weights
  q - z with a per-channel scale repeated over every group);
- the W8A8 packed layout against hand-worked bytes and a round trip;
- for the online Hadamard rotation: unit rows give the rows of the
  Sylvester matrix (closed form), rotating twice gives 128 x the input
  (H H = 128 I) exactly on integer rows, and the float32 result matches a
  float64 block-diagonal matrix product within float32 rounding.

Every pin is a plain function taking ``mutant``; ``test_mutants_are_caught``
rebuilds the oracle with one planted mistake at a time and checks that at
least one pin fails for each.
"""
import os

import numpy as np
import pytest

import oracle
from bit_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_quant_ties():
    rows = []
    with open(os.path.join(GOLDEN, "quant_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, sa, qs = (p.split() for p in line.split("|"))
            rows.append((np.array([float(v) for v in xs], np.float32), float(sa[0]),
                         np.array([int(v) for v in qs], np.int8)))
    return rows


def _tiny_case(seed=11, M=3, K=256, N=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    q, z, s = synth.draw_weights(rng, N, K)
    return x, q, z, s


def _p_numpy(qa, q, z, group=128):
    """Per-group products with numpy int64 matmul, one group at a time."""
    M, K = qa.shape
    N = q.shape[0]
    G = K // group
    P = np.empty((M, N, G), np.int64)
    for g in range(G):
        a = qa[:, g * group:(g + 1) * group].astype(np.int64)
        w = q[:, g * group:(g + 1) * group].astype(np.int64) - z[:, g:g + 1].astype(np.int64)
        P[:, :, g] = a @ w.T
    return P


# --------------------------------------------------------------------------- pins

def pin_quant_golden(mutant=0):
    for x, sa_exp, q_exp in _read_quant_ties():
        qa, sa = oracle.quant_act(x[None, :], mutant=mutant)
        assert sa[0] == np.float32(sa_exp), (x, sa[0], sa_exp)
        assert np.array_equal(qa[0], q_exp), (x, qa[0], q_exp)


def pin_quant_invariants(mutant=0):
    lin = synth.make_linear(synth.LinearSpec("pin", 6, 512, 16, seed=5), with_weights=False)
    xf = synth.x_as_f32(lin)
    for x in (xf, lin["x"]):                      # float32 and bf16 entry points
        qa, sa = oracle.quant_act(x, mutant=mutant)
        assert qa.min() >= -127
        assert np.all(np.abs(qa).max(axis=1) == 127)
        err = np.abs(xf.astype(np.float64) - sa[:, None].astype(np.float64) * qa)
        assert np.all(err <= sa[:, None].astype(np.float64) / 2 * (1 + 2.0 ** -22))
    qa, sa = oracle.quant_act(xf, mutant=mutant)
    for j in (-3, 2, 5):                           # exact power-of-two rescaling
        qa2, sa2 = oracle.quant_act((xf * np.float32(2.0 ** j)).astype(np.float32), mutant=mutant)
        assert np.array_equal(qa2, qa)
        assert np.array_equal(sa2, (sa * np.float32(2.0 ** j)).astype(np.float32))


def pin_partials_brute(mutant=0):
    x, q, z, s = _tiny_case()
    qa, _ = oracle.quant_act(x, mutant=mutant)
    P = oracle.group_partials(qa, q, z, mutant=mutant)
    assert np.array_equal(P.astype(np.int64), _p_numpy(qa, q, z))
    # extremes: |P| reaches 128*127*15 and no further
    K, N = 256, 16
    qa = np.full((2, K), 127, np.int8)
    qa[1] = -127
    q = np.zeros((N, K), np.uint8)
    q[: N // 2] = 15
    z = np.zeros((N, 2), np.uint8)
    z[N // 2:] = 15
    P = oracle.group_partials(qa, q, z, mutant=mutant)
    assert np.array_equal(P.astype(np.int64), _p_numpy(qa, q, z))
    assert P.max() == oracle.P_BOUND and P.min() == -oracle.P_BOUND


def pin_zero_shift_and_identity(mutant=0):
    x, q, z, s = _tiny_case(seed=12)
    qa, _ = oracle.quant_act(x, mutant=mutant)
    P = oracle.group_partials(qa, q, z, mutant=mutant).astype(np.int64)
    # sum qa*(q-z) == sum qa*q - z * sum qa, from numpy alone
    G = q.shape[1] // 128
    rs = qa.astype(np.int64).reshape(qa.shape[0], G, 128).sum(axis=2)
    Pq = _p_numpy(qa, q, np.zeros_like(z))
    assert np.array_equal(P, Pq - z.astype(np.int64)[None, :, :] * rs[:, None, :])
    # shifting codes and zeros together (codes kept in 0..15) leaves P unchanged
    qc = np.minimum(q, 10).astype(np.uint8)
    zc = np.minimum(z, 10).astype(np.uint8)
    P0 = oracle.group_partials(qa, qc, zc, mutant=mutant)
    for c in (1, 5):
        Pc = oracle.group_partials(qa, qc + c, zc + c, mutant=mutant)
        assert np.array_equal(P0, Pc)


def pin_zero_weights(mutant=0):
    x, q, z, s = _tiny_case(seed=13)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    zq = np.repeat(z, 128, axis=1).astype(np.uint8)          # q == z everywhere
    assert not oracle.group_partials(qa, zq, z, mutant=mutant).any()
    y = oracle.linear(qa, sa, zq, z, s, mutant=mutant)
    assert np.all(y == 0.0)
    y = oracle.linear(qa, sa, q, z, np.zeros_like(s), mutant=mutant)
    assert np.all(y == 0.0)


def pin_group_permutation(mutant=0):
    x, q, z, s = _tiny_case(seed=14)
    qa, _ = oracle.quant_act(x, mutant=mutant)
    P = oracle.group_partials(qa, q, z, mutant=mutant)
    rng = np.random.Generator(np.random.PCG64(99))
    perm = np.concatenate([g * 128 + rng.permutation(128) for g in range(q.shape[1] // 128)])
    P2 = oracle.group_partials(np.ascontiguousarray(qa[:, perm]), np.ascontiguousarray(q[:, perm]),
                               z, mutant=mutant)
    assert np.array_equal(P, P2)


def pin_dequant_matmul(mutant=0):
    x, q, z, s = _tiny_case(seed=15, M=4, K=384, N=24)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    y = oracle.linear(qa, sa, q, z, s, mutant=mutant)
    w = np.repeat(s.astype(np.float64), 128, axis=1) * (
        q.astype(np.float64) - np.repeat(z.astype(np.float64), 128, axis=1))
    ref = (sa.astype(np.float64)[:, None] * qa.astype(np.float64)) @ w.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # a window of rows and columns is the same slice of the full result
    yw = oracle.linear(qa, sa, q, z, s, rows=(1, 3), cols=(5, 17), mutant=mutant)
    assert np.array_equal(yw, y[1:3, 5:17])


def pin_identity_scale(mutant=0):
    """s == 1 and integer rows with absmax 127: sa == 1, qa == x, y is an exact
    integer GEMM (numpy int64 matmul)."""
    rng = np.random.Generator(np.random.PCG64(16))
    M, K, N = 5, 512, 32
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, 7] = 127
    x = xi.astype(np.float32)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=(N, K // 128), dtype=np.uint8)
    s = np.ones((N, K // 128), np.float32)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    assert np.all(sa == 1.0) and np.array_equal(qa.astype(np.int64), xi)
    y = oracle.linear(qa, sa, q, z, s, mutant=mutant)
    exact = xi @ (q.astype(np.int64) - np.repeat(z.astype(np.int64), 128, axis=1)).T
    assert np.array_equal(y, exact.astype(np.float64))


def _w8_case(seed, M, K, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    qw, sw = synth.draw_w8_weights(rng, N, K)
    return x, qw, sw


def pin_w8_totals_brute(mutant=0):
    """W8A8 integer totals: numpy int64 matmul, and two closed forms."""
    x, qw, sw = _w8_case(31, 4, 384, 24)
    qa, _ = oracle.quant_act(x, mutant=mutant)
    P = oracle.w8a8_totals(qa, qw, mutant=mutant)
    assert np.array_equal(P.astype(np.int64), qa.astype(np.int64) @ qw.astype(np.int64).T)
    K = 1024
    ones = np.ones((2, K), np.int8)
    assert np.all(oracle.w8a8_totals(ones, np.ones((16, K), np.int8), mutant=mutant) == K)
    # +127 activations against -127 weights: every product is -16129
    a = np.full((1, K), 127, np.int8)
    w = np.full((16, K), -127, np.int8)
    assert np.all(oracle.w8a8_totals(a, w, mutant=mutant) == -16129 * K)
    P2 = oracle.w8a8_totals(qa, qw, m0=1, m1=3, mutant=mutant)
    assert np.array_equal(P2, P[1:3])


def pin_w8_dequant_matmul(mutant=0):
    """W8A8 float64 result against numpy dequant-then-matmul (activation and
    weight scales both applied)."""
    x, qw, sw = _w8_case(32, 5, 512, 32)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    y = oracle.w8a8_linear(qa, sa, qw, sw, mutant=mutant)
    ref = (sa.astype(np.float64)[:, None] * qa.astype(np.float64)) @ (
        sw.astype(np.float64)[:, None] * qw.astype(np.float64)).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    yw = oracle.w8a8_linear(qa, sa, qw, sw, rows=(2, 4), cols=(3, 19), mutant=mutant)
    assert np.array_equal(yw, y[2:4, 3:19])


def pin_w8_equals_w4_special_case(mutant=0):
    """Int4 weights with zero points are int8 weights q - z; with the group
    scale equal for every group of a channel, the W4A8 and W8A8 results are
    the same exact float64 values (every product of a float32 scale and an
    integer below 2^29 is exact, so the two summation orders agree)."""
    x, q, z, s = _tiny_case(seed=33, M=3, K=512, N=32)
    sw = s[:, 0].copy()
    s_rep = np.repeat(sw[:, None], 512 // 128, axis=1)
    qw = (q.astype(np.int16) - np.repeat(z.astype(np.int16), 128, axis=1)).astype(np.int8)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    y4 = oracle.linear(qa, sa, q, z, s_rep, mutant=mutant)
    y8 = oracle.w8a8_linear(qa, sa, qw, sw, mutant=mutant)
    assert np.array_equal(y4, y8)
    P4 = oracle.group_partials(qa, q, z, mutant=mutant).astype(np.int64).sum(axis=2)
    assert np.array_equal(P4, oracle.w8a8_totals(qa, qw, mutant=mutant).astype(np.int64))


def _sylvester(n):
    i = np.arange(n)
    return np.array([[(-1) ** bin(a & b).count("1") for b in i] for a in i], np.float64)


def pin_hadamard_unit_rows(mutant=0):
    """A unit row e_k (k in group g) becomes row k % 128 of H in group g."""
    K = 384
    H = _sylvester(128)
    ks = [0, 1, 5, 64, 127, 130, 255, 300]
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    xr = oracle.hadamard_rows(x, mutant=mutant)
    for r, k in enumerate(ks):
        g = k // 128
        want = np.zeros(K)
        want[128 * g:128 * g + 128] = H[k % 128]
        assert np.array_equal(xr[r].astype(np.float64), want), k


def pin_hadamard_twice(mutant=0):
    """H H = 128 I: on small integer rows (exact in float32) rotating twice
    returns 128 x the row, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(41))
    x = rng.integers(-100, 101, size=(3, 256)).astype(np.float32)
    twice = oracle.hadamard_rows(oracle.hadamard_rows(x, mutant=mutant), mutant=mutant)
    assert np.array_equal(twice, 128.0 * x)


def pin_hadamard_matmul(mutant=0):
    """Float32 butterflies against a float64 block-diagonal product, from bf16
    and float32 inputs; the codes are the quantiser's on the rotated rows."""
    rng = np.random.Generator(np.random.PCG64(42))
    H = _sylvester(128)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    x[:, 77] *= 20.0
    for xin in (x, synth.bf16_round_bits(x)):
        xr = oracle.hadamard_rows(xin, mutant=mutant).astype(np.float64)
        x64 = synth.bf16_bits_to_f32(xin).astype(np.float64) if xin.dtype == np.uint16 else \
            xin.astype(np.float64)
        ref = np.concatenate([x64[:, 128 * g:128 * g + 128] @ H for g in range(4)], axis=1)
        assert np.max(np.abs(xr - ref)) <= 1e-5 * np.max(np.abs(ref))
        qa, sa = oracle.hadamard_quant_act(xin, mutant=mutant)
        qa2, sa2 = oracle.quant_act(oracle.hadamard_rows(xin, mutant=mutant), mutant=mutant)
        assert np.array_equal(qa, qa2) and np.array_equal(sa, sa2)


def pin_w4a16_dequant_matmul(mutant=0):
    """W4A16 float64 result against numpy dequant-then-matmul (bf16 and f32
    activations), with windows; zero weights give zeros."""
    x, q, z, s = _tiny_case(seed=44, M=4, K=384, N=24)
    w = np.repeat(s.astype(np.float64), 128, axis=1) * (
        q.astype(np.float64) - np.repeat(z.astype(np.float64), 128, axis=1))
    for xin in (x, synth.bf16_round_bits(x)):
        x64 = synth.bf16_bits_to_f32(xin).astype(np.float64) if xin.dtype == np.uint16 else \
            xin.astype(np.float64)
        y = oracle.w4a16_linear(xin, q, z, s, mutant=mutant)
        ref = x64 @ w.T
        assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
        assert np.array_equal(oracle.w4a16_linear(xin, q, z, s, rows=(1, 3), cols=(2, 10),
                                                  mutant=mutant), y[1:3, 2:10])
    zq = np.broadcast_to(np.repeat(z, 128, axis=1), q.shape).astype(np.uint8)
    assert not oracle.w4a16_linear(x, zq, z, s, mutant=mutant).any()


def pin_w4a16_equals_w4a8_on_integer_rows(mutant=0):
    """Integer activation rows with absmax 127 quantise to themselves with
    scale 1, so W4A16 and W4A8 compute the same exact float64 values."""
    rng = np.random.Generator(np.random.PCG64(45))
    M, K, N = 3, 512, 32
    xi = rng.integers(-127, 128, size=(M, K))
    xi[:, 3] = -127
    x = xi.astype(np.float32)
    q, z, s = synth.draw_weights(rng, N, K)
    qa, sa = oracle.quant_act(x, mutant=mutant)
    assert np.array_equal(oracle.w4a16_linear(x, q, z, s, mutant=mutant),
                          oracle.linear(qa, sa, q, z, s, mutant=mutant))


PINS = [pin_quant_golden, pin_quant_invariants, pin_partials_brute, pin_zero_shift_and_identity,
        pin_zero_weights, pin_group_permutation, pin_dequant_matmul, pin_identity_scale,
        pin_w8_totals_brute, pin_w8_dequant_matmul, pin_w8_equals_w4_special_case,
        pin_hadamard_unit_rows, pin_hadamard_twice, pin_hadamard_matmul, pin_w4a16_dequant_matmul,
        pin_w4a16_equals_w4a8_on_integer_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(0)


MUTANTS = {1: "zero point dropped", 2: "ties away from zero", 3: "scale absmax/128",
           4: "zero plane transposed", 5: "activation scale missing", 6: "weights shifted by one k",
           7: "W8A8 weight scale dropped", 8: "W8A8 weights read unsigned",
           9: "Hadamard upper half not negated", 10: "W4A16 zero point dropped"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_mutants_are_caught(mutant):
    caught = []
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
        except oracle.OracleError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{MUTANTS[mutant]}' passed every pin"


def test_nonfinite_rejected():
    x = np.zeros((1, 128), np.float32)
    x[0, 3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quant_act(x)


# --------------------------------------------------------------------------- layout

def _read_layout_golden():
    entries = {"bytes": [], "zeros": [], "scalars": {}}
    with open(os.path.join(GOLDEN, "layout_v1.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "zeros":
                entries["zeros"].append((int(parts[1]), int(parts[2], 16)))
            elif parts[0] in ("scales_offset", "total_bytes"):
                entries["scalars"][parts[0]] = int(parts[1])
            else:
                entries["bytes"].append((int(parts[0]), int(parts[4], 16)))
    return entries


def test_layout_golden():
    gold = _read_layout_golden()
    N, K = 16, 128
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    q = ((3 * n + k + 5 * (k // 16)) % 16).astype(np.uint8)
    z = np.arange(16, dtype=np.uint8)[:, None]
    s = np.linspace(0.5, 2.0, 16, dtype=np.float32)[:, None]
    buf = oracle.layout_pack(q, z, s)
    assert buf.size == gold["scalars"]["total_bytes"]
    for off, b in gold["bytes"]:
        assert buf[off] == b, (off, hex(buf[off]), hex(b))
    for off, b in gold["zeros"]:
        assert buf[off] == b, (off, hex(buf[off]), hex(b))
    s0 = gold["scalars"]["scales_offset"]
    assert np.array_equal(buf[s0:s0 + 64].view(np.float32), s[:, 0])


def test_layout_round_trip_and_bijection():
    rng = np.random.Generator(np.random.PCG64(21))
    N, K = 48, 384
    q, z, s = synth.draw_weights(rng, N, K)
    buf = oracle.layout_pack(q, z, s)
    q2, z2, s2 = oracle.layout_unpack(buf, N, K)
    assert np.array_equal(q, q2) and np.array_equal(z, z2)
    assert np.array_equal(s.view(np.uint32), s2.view(np.uint32))
    # every code lands in exactly one nibble: a single 1 among zeros sets one bit group
    codes_end = N * K // 2
    seen = set()
    for (nn, kk) in [(0, 0), (0, 64), (1, 0), (15, 127), (16, 0), (47, 383), (20, 200), (33, 65)]:
        qq = np.zeros((N, K), np.uint8)
        qq[nn, kk] = 1
        b = oracle.layout_pack(qq, np.zeros_like(z), np.zeros_like(s))[:codes_end]
        nz = np.flatnonzero(b)
        assert nz.size == 1 and b[nz[0]] in (0x01, 0x10)
        pos = (int(nz[0]), int(b[nz[0]]))
        assert pos not in seen
        seen.add(pos)


def test_w8_layout_golden():
    entries, scalars = [], {}
    with open(os.path.join(GOLDEN, "layout_w8_v1.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] in ("scales_offset", "total_bytes"):
                scalars[parts[0]] = int(parts[1])
            else:
                entries.append((int(parts[0]), int(parts[7]), int(parts[8], 16)))
    N, K = 16, 128
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    qw = (((5 * n + 3 * k) % 255) - 127).astype(np.int8)
    sw = np.linspace(0.25, 4.0, N, dtype=np.float32)
    buf = oracle.w8_layout_pack(qw, sw)
    assert buf.size == scalars["total_bytes"]
    for off, value, b in entries:
        assert (value & 0xFF) == b
        assert buf[off] == b, (off, hex(buf[off]), hex(b))
    s0 = scalars["scales_offset"]
    assert np.array_equal(buf[s0:s0 + 4 * N].view(np.float32), sw)


def test_w8_layout_round_trip_and_bijection():
    rng = np.random.Generator(np.random.PCG64(34))
    N, K = 48, 384
    qw, sw = synth.draw_w8_weights(rng, N, K)
    buf = oracle.w8_layout_pack(qw, sw)
    qw2, sw2 = oracle.w8_layout_unpack(buf, N, K)
    assert np.array_equal(qw, qw2) and np.array_equal(sw.view(np.uint32), sw2.view(np.uint32))
    seen = set()
    for (nn, kk) in [(0, 0), (0, 64), (1, 0), (15, 127), (16, 0), (47, 383), (20, 200), (33, 65)]:
        q1 = np.zeros((N, K), np.int8)
        q1[nn, kk] = 1
        b = oracle.w8_layout_pack(q1, np.zeros_like(sw))[:N * K]
        nz = np.flatnonzero(b)
        assert nz.size == 1 and b[nz[0]] == 1
        assert int(nz[0]) not in seen
        seen.add(int(nz[0]))
