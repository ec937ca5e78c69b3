"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host (no GPU needed: a
rejected call returns before anything is enqueued)."""
import ctypes
import glob
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b((?:w4a8|w8a8|w4a16)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_amd import _lib
    return _lib.load()


def test_header_symbols_exported(lib):
    from bit_quantized_amd import _lib
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def test_versions_and_status(lib):
    assert lib.w4a8_abi_version() == 1
    assert lib.w4a8_layout_version() == 1
    assert lib.w4a8_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4, -5):
        assert lib.w4a8_status_string(s) != b"unknown status"


@pytest.mark.parametrize("N,K", [(16, 128), (256, 256), (512, 3584), (18944, 3584), (3584, 18944),
                                 (48, 384)])
def test_packed_size_matches_spec(lib, N, K):
    assert lib.w4a8_packed_weight_bytes(N, K, 128) == oracle.layout_bytes(N, K)


def test_packed_size_unsupported(lib):
    assert lib.w4a8_packed_weight_bytes(80 + 4, 128, 128) == 0
    assert lib.w4a8_packed_weight_bytes(64, 100, 128) == 0
    assert lib.w4a8_packed_weight_bytes(64, 256, 64) == 0
    assert lib.w4a8_packed_weight_bytes(0, 256, 128) == 0


FAKE = ctypes.c_void_p(1 << 20)          # 16-byte aligned, never dereferenced
FAKE2 = ctypes.c_void_p(1 << 24)
MIS = ctypes.c_void_p((1 << 20) + 4)


def test_pack_rejections(lib):
    f = lib.w4a8_pack_weights
    big = 1 << 30
    assert f(FAKE, FAKE, FAKE, 16, 100, 128, FAKE2, big, None) == -2     # K % 128
    assert f(FAKE, FAKE, FAKE, 20, 128, 128, FAKE2, big, None) == -2     # N tail
    assert f(FAKE, FAKE, FAKE, 16, 128, 64, FAKE2, big, None) == -2      # group
    assert f(None, FAKE, FAKE, 16, 128, 128, FAKE2, big, None) == -1
    assert f(MIS, FAKE, FAKE, 16, 128, 128, FAKE2, big, None) == -3
    assert f(FAKE, FAKE, FAKE, 16, 128, 128, FAKE2, 100, None) == -4
    assert b"too small" in lib.w4a8_last_error() or b"need" in lib.w4a8_last_error()


def test_quant_rejections(lib):
    f = lib.w4a8_quant_act
    assert f(FAKE, 0, 0, 128, FAKE2, FAKE2, None) == -1
    assert f(FAKE, 7, 1, 128, FAKE2, FAKE2, None) == -1
    assert f(FAKE, 0, 1, 130, FAKE2, FAKE2, None) == -2
    assert f(MIS, 0, 1, 128, FAKE2, ctypes.c_void_p((1 << 24) + 4096), None) == -3
    assert f(FAKE, 0, 4, 128, FAKE, FAKE2, None) == -1                  # qa aliases x


def test_gemm_rejections(lib):
    f = lib.w4a8_gemm
    pb = lib.w4a8_packed_weight_bytes(256, 256, 128)
    y = ctypes.c_void_p(1 << 28)
    args = dict(qa=FAKE, sa=ctypes.c_void_p((1 << 20) + 65536), packed=FAKE2, pb=pb)

    def call(M=4, N=256, K=256, group=128, pb=pb, y=y, qa=FAKE, ws=None, wsb=0):
        return f(qa, args["sa"], args["packed"], pb, M, N, K, group, y, ws, wsb, None)

    assert call(M=0) == -1
    assert call(N=250) == -2
    assert call(K=200) == -2
    assert call(group=32) == -2
    assert call(pb=pb - 1) == -4
    assert call(qa=None) == -1
    assert call(qa=MIS) == -3
    assert call(y=None) == -1
    assert call(y=FAKE2) == -1                                            # y aliases packed
    # split-K workspace required but missing
    need = lib.w4a8_gemm_workspace_bytes(4, 256, 18944, 128)
    assert need > 0
    pb2 = lib.w4a8_packed_weight_bytes(256, 18944, 128)
    assert f(FAKE, args["sa"], FAKE2, pb2, 4, 256, 18944, 128, y, None, 0, None) == -4


def test_debug_path_rejections(lib):
    f = lib.w4a8_gemm_debug
    pb = lib.w4a8_packed_weight_bytes(256, 256, 128)
    sa = ctypes.c_void_p((1 << 20) + 65536)
    y = ctypes.c_void_p(1 << 28)
    P = ctypes.c_void_p(1 << 29)
    assert f(FAKE, sa, FAKE2, pb, 4, 256, 256, 128, 1, 0, 4, P, y, None, 0, None) == -1  # GEMV M!=1
    assert f(FAKE, sa, FAKE2, pb, 17, 256, 256, 128, 2, 0, 4, P, y, None, 0, None) == -1  # SKINNY M>16
    assert f(FAKE, sa, FAKE2, pb, 4, 256, 256, 128, 9, 0, 4, P, y, None, 0, None) == -1   # bad path
    assert f(FAKE, sa, FAKE2, pb, 4, 256, 256, 128, 3, 2, 5, P, y, None, 0, None) == -1   # window


def test_select_path(lib):
    assert lib.w4a8_select_path(1, 18944, 3584) == 1
    assert lib.w4a8_select_path(2, 3584, 18944) == 2
    assert lib.w4a8_select_path(16, 3584, 18944) == 2
    assert lib.w4a8_select_path(17, 3584, 18944) == 3
    assert lib.w4a8_select_path(2048, 18944, 3584) == 3


def test_linear_rejections(lib):
    f = lib.w4a8_linear
    pb = lib.w4a8_packed_weight_bytes(256, 256, 128)
    y = ctypes.c_void_p(1 << 28)
    assert f(None, 0, FAKE2, pb, 1, 256, 256, 128, y, None, 0, None) == -1
    assert f(FAKE, 5, FAKE2, pb, 1, 256, 256, 128, y, None, 0, None) == -1
    assert f(FAKE, 0, FAKE2, pb, 1, 250, 256, 128, y, None, 0, None) == -2
    assert f(FAKE, 0, FAKE2, pb - 16, 1, 256, 256, 128, y, None, 0, None) == -4
    assert f(FAKE, 0, FAKE2, pb, 4, 256, 256, 128, y, None, 0, None) == -4     # needs workspace
    assert lib.w4a8_linear_workspace_bytes(1, 18944, 3584, 128) == 0          # one launch
    assert lib.w4a8_linear_workspace_bytes(4, 256, 256, 128) >= 4 * 256 + 16


def test_linear_workspace_codes_region(lib):
    """The two-launch linear's workspace: the codes (16 K bytes in the tiled
    layout at 12 <= M <= 16 on the M <= 16 kernel, else M K), the scales, then
    the GEMM's own workspace."""
    def r(v):
        return (v + 255) // 256 * 256
    gw = lib.w4a8_gemm_workspace_bytes
    for M, K, N in ((16, 18944, 3584), (12, 18944, 3584), (13, 8192, 2048)):
        assert lib.w4a8_linear_workspace_bytes(M, N, K, 128) == r(16 * K) + r(4 * M) + gw(M, N, K, 128)
        assert lib.w4a8_linear_hadamard_workspace_bytes(M, N, K, 128) == \
            r(16 * K) + r(4 * M) + gw(M, N, K, 128)
    for M, K, N in ((8, 18944, 3584), (11, 18944, 3584), (17, 18944, 3584)):
        assert lib.w4a8_linear_workspace_bytes(M, N, K, 128) == r(M * K) + r(4 * M) + gw(M, N, K, 128)
    w8 = lib.w8a8_gemm_workspace_bytes
    assert lib.w8a8_linear_workspace_bytes(16, 3584, 18944) == r(16 * 18944) + r(64) + w8(16, 3584, 18944)
    assert lib.w8a8_linear_workspace_bytes(13, 3584, 18944) == r(13 * 18944) + r(52) + w8(13, 3584, 18944)


def test_pack_into_rejections(lib):
    f = lib.w4a8_pack_weights_into
    big = 1 << 30
    assert f(FAKE, FAKE, FAKE, 16, 128, 128, FAKE2, big, 64, 8, None) == -1     # offset % 16
    assert f(FAKE, FAKE, FAKE, 32, 128, 128, FAKE2, big, 64, 48, None) == -1    # past N_total
    assert f(FAKE, FAKE, FAKE, 16, 128, 128, FAKE2, big, 64, -16, None) == -1   # negative
    assert f(FAKE, FAKE, FAKE, 16, 128, 128, FAKE2, big, 70, 0, None) == -2     # N_total tail
    assert f(FAKE, FAKE, FAKE, 20, 128, 128, FAKE2, big, 64, 0, None) == -2     # part tail
    pb = lib.w4a8_packed_weight_bytes(64, 128, 128)
    assert f(FAKE, FAKE, FAKE, 16, 128, 128, FAKE2, pb - 1, 64, 0, None) == -4  # sized for N_total


# ------------------------------------------------------------------ W8A8

@pytest.mark.parametrize("N,K", [(16, 128), (512, 3584), (3584, 18944), (48, 384)])
def test_w8_packed_size_matches_spec(lib, N, K):
    assert lib.w8a8_packed_weight_bytes(N, K) == oracle.w8_layout_bytes(N, K)


def test_w8_packed_size_unsupported(lib):
    assert lib.w8a8_packed_weight_bytes(84, 128) == 0
    assert lib.w8a8_packed_weight_bytes(64, 100) == 0
    assert lib.w8a8_packed_weight_bytes(16, 131072 + 128) == 0       # exact int32 totals
    assert lib.w8a8_packed_weight_bytes(16, 131072) > 0
    assert lib.w8a8_layout_version() == 1


def test_w8_pack_rejections(lib):
    f = lib.w8a8_pack_weights
    pb = lib.w8a8_packed_weight_bytes(32, 256)
    assert f(None, FAKE, 32, 256, FAKE2, pb, None) == -1
    assert f(FAKE, FAKE, 32, 250, FAKE2, pb, None) == -2
    assert f(FAKE, FAKE, 32, 131200, FAKE2, 1 << 40, None) == -2
    assert f(MIS, FAKE, 32, 256, FAKE2, pb, None) == -3
    assert f(FAKE, FAKE2, 32, 256, FAKE2, pb, None) == -1                # packed aliases sw
    assert f(FAKE, FAKE2, 32, 256, ctypes.c_void_p(1 << 26), pb - 16, None) == -4
    u = lib.w8a8_unpack_weights
    assert u(FAKE, pb - 1, 32, 256, FAKE2, ctypes.c_void_p(1 << 26), None) == -4
    assert u(FAKE, pb, 32, 256, FAKE2, FAKE2, None) == -1                 # qw aliases sw


def test_w8_gemm_rejections(lib):
    f = lib.w8a8_gemm
    pb = lib.w8a8_packed_weight_bytes(256, 256)
    y = ctypes.c_void_p(1 << 28)
    assert f(None, FAKE, FAKE2, pb, 4, 256, 256, y, None, 0, None) == -1
    assert f(FAKE, FAKE, FAKE2, pb, 0, 256, 256, y, None, 0, None) == -1
    assert f(FAKE, FAKE, FAKE2, pb, 4, 250, 256, y, None, 0, None) == -2
    assert f(FAKE, FAKE, FAKE2, pb - 16, 4, 256, 256, y, None, 0, None) == -4
    assert f(FAKE, MIS, FAKE2, pb, 4, 256, 256, y, None, 0, None) == -3
    assert f(FAKE, FAKE, FAKE2, pb, 4, 256, 256, FAKE2, None, 0, None) == -1   # y aliases packed
    # small N with long K splits K on the M <= 16 path: the int32 partials
    # need a workspace (device_cus() reads 256 when no device is present)
    pb2 = lib.w8a8_packed_weight_bytes(512, 18944)
    need = lib.w8a8_gemm_workspace_bytes(1, 512, 18944)
    assert need >= 2 * 512 * 4
    assert f(FAKE, FAKE, FAKE2, pb2, 1, 512, 18944, y, None, 0, None) == -4
    # (the M <= 16 kernel splits K four ways here: 4 x 1 x 512 int32 partials)
    assert f(FAKE, FAKE, FAKE2, pb2, 1, 512, 18944, y, ctypes.c_void_p(1 << 32), 4 * 512 * 4 - 16,
             None) == -4
    assert lib.w8a8_gemm_workspace_bytes(1, 18944, 3584) == 0


def test_w8_debug_and_path_rejections(lib):
    f = lib.w8a8_gemm_debug
    pb = lib.w8a8_packed_weight_bytes(256, 256)
    y = ctypes.c_void_p(1 << 28)
    assert f(FAKE, FAKE, FAKE2, pb, 4, 256, 256, 1, 0, 4, None, y, None, 0, None) == -2   # GEMV: M == 1
    assert f(FAKE, FAKE, FAKE2, pb, 1, 256, 256, 9, 0, 1, None, y, None, 0, None) == -1   # no such path
    assert f(FAKE, FAKE, FAKE2, pb, 17, 256, 256, 2, 0, 17, None, y, None, 0, None) == -1  # SKINNY M
    assert f(FAKE, FAKE, FAKE2, pb, 4, 256, 256, 0, 2, 5, None, y, None, 0, None) == -1   # window
    assert f(FAKE, FAKE, FAKE2, pb, 4, 256, 256, 7, 0, 4, None, y, None, 0, None) == -1   # enum
    assert f(FAKE, FAKE, FAKE2, pb, 4, 256, 256, 0, 0, 4, MIS, y, None, 0, None) == -3
    assert lib.w8a8_select_path(1, 18944, 3584) == 1                           # GEMV
    assert lib.w8a8_select_path(1, 256, 65536) == 2                            # K past the GEMV
    assert lib.w8a8_select_path(16, 3584, 18944) == 2
    assert lib.w8a8_select_path(17, 3584, 18944) == 3


def test_w8_linear_rejections(lib):
    f = lib.w8a8_linear
    pb = lib.w8a8_packed_weight_bytes(256, 256)
    y = ctypes.c_void_p(1 << 28)
    assert f(None, 0, FAKE2, pb, 1, 256, 256, y, None, 0, None) == -1
    assert f(FAKE, 5, FAKE2, pb, 1, 256, 256, y, None, 0, None) == -1
    assert f(FAKE, 0, FAKE2, pb, 1, 250, 256, y, None, 0, None) == -2
    assert f(FAKE, 0, FAKE2, pb, 4, 256, 256, y, None, 0, None) == -4       # needs workspace
    assert lib.w8a8_linear_workspace_bytes(4, 256, 256) >= 4 * 256 + 16


def test_hadamard_rejections(lib):
    f = lib.w4a8_quant_act_hadamard
    assert f(None, 0, 4, 256, FAKE2, FAKE, None) == -1
    assert f(FAKE, 3, 4, 256, FAKE2, ctypes.c_void_p(1 << 26), None) == -1
    assert f(FAKE, 0, 4, 200, FAKE2, ctypes.c_void_p(1 << 26), None) == -2
    assert f(MIS, 0, 4, 256, FAKE2, ctypes.c_void_p(1 << 26), None) == -3
    g = lib.w4a8_linear_hadamard
    pb = lib.w4a8_packed_weight_bytes(256, 256, 128)
    y = ctypes.c_void_p(1 << 28)
    need = lib.w4a8_linear_hadamard_workspace_bytes(1, 256, 256, 128)
    assert need >= 256 + 4
    assert g(FAKE, 0, FAKE2, pb, 1, 256, 256, 128, y, None, 0, None) == -4     # codes need room
    assert g(FAKE, 0, FAKE2, pb, 1, 256, 256, 128, y, ctypes.c_void_p(1 << 32), need - 16,
             None) == -4
    assert g(FAKE, 0, FAKE2, pb - 16, 1, 256, 256, 128, y, ctypes.c_void_p(1 << 32), need,
             None) == -4
    assert g(FAKE, 0, FAKE2, pb, 1, 256, 256, 64, y, ctypes.c_void_p(1 << 32), need, None) == -2


def test_w4a16_rejections(lib):
    f = lib.w4a16_linear
    pb = lib.w4a8_packed_weight_bytes(256, 256, 128)
    y = ctypes.c_void_p(1 << 28)
    assert f(None, FAKE2, pb, 4, 256, 256, 128, y, None, 0, None) == -1
    assert f(FAKE, FAKE2, pb, 4, 250, 256, 128, y, None, 0, None) == -2
    assert f(MIS, FAKE2, pb, 4, 256, 256, 128, y, None, 0, None) == -3
    assert f(FAKE, FAKE2, pb - 16, 4, 256, 256, 128, y, None, 0, None) == -4
    assert f(FAKE, FAKE2, pb, 4, 256, 256, 128, FAKE2, None, 0, None) == -1   # y aliases packed
    g = lib.w4a16_linear_path
    assert g(FAKE, FAKE2, pb, 4, 256, 256, 128, 1, y, None, 0, None) == -2    # GEMV needs M == 1
    assert g(FAKE, FAKE2, pb, 1, 256, 256, 128, 9, y, None, 0, None) == -1    # no such path
    assert g(FAKE, FAKE2, pb, 17, 256, 256, 128, 2, y, None, 0, None) == -2   # SKINNY needs M <= 16
    pb2 = lib.w4a8_packed_weight_bytes(512, 18944, 128)
    need = lib.w4a16_linear_workspace_bytes(1, 512, 18944, 128)
    assert need > 0
    assert f(FAKE, FAKE2, pb2, 1, 512, 18944, 128, y, None, 0, None) == -4    # split K: workspace
    assert lib.w4a16_select_path(4, 3584, 18944) == 2
    assert lib.w4a16_select_path(8, 3584, 18944) == 2                          # direct operand loads
    assert lib.w4a16_select_path(16, 3584, 18944) == 2
    assert lib.w4a16_select_path(17, 3584, 18944) == 3
    assert lib.w4a16_select_path(1, 18944, 3584) == 1                         # GEMV
    assert lib.w4a16_select_path(1, 3584, 18944) == 1
    assert lib.w4a16_select_path(1, 256, 65536) in (2, 3)                     # K past the GEMV's LDS


def test_prefill_workspace_plans(lib):
    """Host planning of the prefill grid, visible through the workspace sizes
    (no GPU here: the planner assumes 256 compute units, as on MI355X).
    - A partial last round of tiles runs as K slices whose float (int32 for
      W8A8) sums cover only the tail's channels: M = 512, K = 3584 -> N =
      18944 has 296 tiles (one round and 40), 6 slices of 512 x 2560.
    - W4A16 tiles hold 128 tokens: M = 2048 there has 2368 tiles (9 rounds
      and 64), 4 slices of 2048 x 512.
    - W4A8 at M = 2048 takes 256 x 256 tiles (592: two rounds and 80); the
      partial round's channels run as 160 half tiles of 256 x 128 over all of
      K, so nothing goes through the workspace; its 256 x 128 tiles (1184:
      four rounds and 160, too many to split) would need none either, and
      W8A8 keeps those.
    - Whole rounds need no workspace; nor do rows that run as several chunks
      (M * K >= 2^31).  The W4A8 size is the larger of the two tile widths'
      plans (the debug entry point can force either)."""
    slices = 6 * 512 * 2560 * 4
    assert lib.w4a8_gemm_workspace_bytes(512, 18944, 3584, 128) == slices
    assert lib.w8a8_gemm_workspace_bytes(512, 18944, 3584) == slices
    assert lib.w4a16_linear_workspace_bytes(2048, 18944, 3584, 128) == 4 * 2048 * 512 * 4
    assert lib.w4a8_gemm_workspace_bytes(2048, 18944, 3584, 128) == 0
    assert lib.w8a8_gemm_workspace_bytes(2048, 18944, 3584) == 0
    assert lib.w4a8_gemm_workspace_bytes(1024, 32768, 3584, 128) == 0      # 4 x 256 tiles
    assert lib.w4a8_gemm_workspace_bytes(1 << 24, 16, 128, 128) == 0       # row chunks


def test_peak_probe_rejections(lib):
    f = lib.w4a8_peak_stream_read
    assert f(None, 1 << 20, FAKE2, 64, None) == -1
    assert f(FAKE, 0, FAKE2, 64, None) == -1
    assert f(FAKE, 100, FAKE2, 64, None) == -1                           # not a 16-byte multiple
    assert f(FAKE, 1 << 20, FAKE2, 0, None) == -1
    assert f(FAKE, 1 << 20, FAKE2, 70000, None) == -1
    assert f(MIS, 1 << 20, FAKE2, 64, None) == -3
    assert f(FAKE, 1 << 20, ctypes.c_void_p((1 << 20) + 4096), 64, None) == -1  # sink in buf
    g = lib.w4a8_peak_mfma_i8
    assert g(0, FAKE, None, 256, None) == -1
    assert g(1 << 21, FAKE, None, 256, None) == -1
    assert g(16, None, None, 256, None) == -1
    assert g(16, FAKE, None, 0, None) == -1
    assert g(16, MIS, None, 256, None) == -3
    assert g(16, FAKE, FAKE, 256, None) == -1                            # clocks alias sink


def test_noalloc_rejections(lib):
    """The allocation-free entry point refuses bad shapes and shapes whose
    workspace exceeds its static scratch before touching the device."""
    f = lib.w4a8_linear_noalloc
    y = ctypes.c_void_p(1 << 28)
    pb = lib.w4a8_packed_weight_bytes(256, 8192, 128)
    assert f(FAKE, 0, FAKE2, pb, 8192, 256, 8192, 128, y, None) == -4   # 64 MiB of codes + more
    assert b"static scratch" in lib.w4a8_last_error()
    assert f(FAKE, 0, FAKE2, pb, 4, 250, 8192, 128, y, None) == -2      # N tail
    assert f(FAKE, 0, FAKE2, pb, 0, 256, 8192, 128, y, None) == -1      # M
    assert f(None, 0, FAKE2, pb, 4, 256, 8192, 128, y, None) == -1
