"""GPU: every route of the linear entry points captured in a HIP graph.

Each route is captured once (on torch's capture stream, with the input,
output and workspace allocated beforehand), then replayed several times with
new activations copied into the input between replays, with the program's
own eager work and synchronisations in between; every replay must equal the
eager call on the same input bit for bit.  The bench times every figure from
such replays, and graph capture is what the allocation-free entry point is
for, so a route that kept state across launches, or recorded work that does
not replay, would show here.
"""
import sys

import numpy as np
import pytest

from bit_quantized_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def _w4(w4, lin):
    return w4.pack_weights(dev(lin["q"]), dev(lin["z"]), dev(lin["s"]))


# (id, M, K, N, kind): kind picks the entry point and weight format
CASES = [
    ("gemv_fused", 1, 3584, 4096, "w4a8"),
    ("gemv_split_k", 1, 18944, 512, "w4a8"),
    ("skinny_fused", 4, 3584, 2048, "w4a8"),
    ("skinny_two_launch_split_k_tiled", 16, 18944, 1024, "w4a8"),
    ("skinny_stream_grid", 8, 3584, 18944, "w4a8"),
    ("prefill_narrow_split_k", 512, 3584, 512, "w4a8"),
    ("prefill_wide_half_tile_tail", 2048, 1024, 18944, "w4a8"),
    ("w8a8_prefill", 300, 1024, 4096, "w8a8"),
    ("w8a8_gemv", 1, 3584, 4096, "w8a8"),
    ("w8a8_skinny_tiled", 16, 18944, 1024, "w8a8"),
    ("w4a16_skinny", 4, 3584, 2048, "w4a16"),
    ("w4a16_prefill", 300, 1024, 2048, "w4a16"),
    ("hadamard_gemv", 1, 3584, 2048, "hadamard"),
    ("hadamard_skinny", 4, 3584, 2048, "hadamard"),
]


def _route(w4, kind, spec):
    """(weight, run(x, out, workspace), workspace bytes)."""
    M, K, N = spec.M, spec.K, spec.N
    if kind == "w8a8":
        lin = synth.make_w8_linear(spec)
        W = w4.w8a8_pack_weights(dev(lin["qw"]), dev(lin["sw"]))
        return W, (lambda x, out, ws: w4.w8a8_linear(x, W, out=out, workspace=ws)), \
            w4.w8a8_linear_workspace_bytes(M, N, K)
    lin = synth.make_linear(spec)
    W = _w4(w4, lin)
    if kind == "w4a16":
        return W, (lambda x, out, ws: w4.w4a16_linear(x, W, out=out, workspace=ws)), \
            w4.w4a16_workspace_bytes(M, N, K)
    if kind == "hadamard":
        nb = int(w4.load().w4a8_linear_hadamard_workspace_bytes(M, N, K, 128))
        return W, (lambda x, out, ws: w4.linear_hadamard(x, W, out=out, workspace=ws)), nb
    return W, (lambda x, out, ws: w4.linear(x, W, out=out, workspace=ws)), \
        w4.linear_workspace_bytes(M, N, K)


@pytest.mark.parametrize("name,M,K,N,kind", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(w4, name, M, K, N, kind):
    spec = synth.LinearSpec(f"graph_{name}", M, K, N, seed=500 + M + N)
    say(f"graph {name} {spec}")
    W, run, nb = _route(w4, kind, spec)
    xs = [x_tensor(synth.make_linear(synth.LinearSpec(f"graph_{name}_{r}", M, K, N,
                                                      seed=600 + 7 * r + M), with_weights=False)["x"])
          for r in range(4)]
    ws = torch.empty(max(int(nb), 16), dtype=torch.uint8, device="cuda")
    refs = []
    for x in xs:
        refs.append(run(x, torch.empty((M, N), dtype=torch.bfloat16, device="cuda"), ws).clone())
    xbuf = xs[0].clone()
    ybuf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    scratch = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(xbuf, ybuf, ws)
    torch.cuda.synchronize()
    for rep, r in enumerate((1, 0, 3, 2, 1)):
        xbuf.copy_(xs[r])
        run(xs[(r + 1) % 4], scratch, ws)  # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ybuf.view(torch.int16), refs[r].view(torch.int16)), f"replay {rep} (input {r})"
        assert torch.equal(scratch.view(torch.int16), refs[(r + 1) % 4].view(torch.int16)), rep
