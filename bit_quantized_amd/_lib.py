"""ctypes binding of libw4a8.so (include/w4a8.h).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the layer runs in the library's HIP kernels.  If the
library is not built this module raises — there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# W4A8_LIB_PATH selects another build of the same library (the host
# AddressSanitizer build of the CPU-side checks); unset, the in-tree one.
LIB_PATH = os.environ.get("W4A8_LIB_PATH") or os.path.join(_PKG, "libw4a8.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED_SHAPE = -2
ERR_MISALIGNED = -3
ERR_BUFFER_TOO_SMALL = -4
ERR_DEVICE = -5

BF16 = 0
F32 = 1

PATH_AUTO = 0
PATH_GEMV = 1
PATH_SKINNY = 2
PATH_PREFILL = 3
PATH_PREFILL_N128 = 4      # w4a8_gemm_debug only: prefill with 256 x 128 tiles forced
PATH_PREFILL_N256 = 5      # w4a8_gemm_debug only: prefill with 256 x 256 tiles forced

GROUP = 128

# Every symbol include/w4a8.h declares, with its ctypes signature.
_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "w4a8_abi_version": (ctypes.c_int, []),
    "w4a8_layout_version": (ctypes.c_int, []),
    "w4a8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a8_last_error": (ctypes.c_char_p, []),
    "w4a8_packed_weight_bytes": (_sz, [_i64, _i64, _i32]),
    "w4a8_pack_weights": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _vp]),
    "w4a8_pack_weights_into": (ctypes.c_int,
                               [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _i64, _i64, _vp]),
    "w4a8_unpack_weights": (ctypes.c_int, [_vp, _sz, _i64, _i64, _i32, _vp, _vp, _vp, _vp]),
    "w4a8_quant_act": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "w4a8_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "w4a8_select_path": (ctypes.c_int, [_i64, _i64, _i64]),
    "w4a8_gemm": (ctypes.c_int, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32, _vp, _vp, _sz, _vp]),
    "w4a8_gemm_debug": (ctypes.c_int, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32, _i32, _i64,
                                       _i64, _vp, _vp, _vp, _sz, _vp]),
    "w4a8_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "w4a8_linear": (ctypes.c_int, [_vp, _i32, _vp, _sz, _i64, _i64, _i64, _i32, _vp, _vp, _sz,
                                   _vp]),
    "w4a8_quant_act_hadamard": (ctypes.c_int, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
    "w4a8_linear_hadamard_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "w4a8_linear_hadamard": (ctypes.c_int, [_vp, _i32, _vp, _sz, _i64, _i64, _i64, _i32, _vp, _vp,
                                            _sz, _vp]),
    "w4a16_linear_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "w4a16_select_path": (ctypes.c_int, [_i64, _i64, _i64]),
    "w4a16_linear": (ctypes.c_int, [_vp, _vp, _sz, _i64, _i64, _i64, _i32, _vp, _vp, _sz, _vp]),
    "w4a16_linear_path": (ctypes.c_int, [_vp, _vp, _sz, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _sz,
                                         _vp]),
    "w8a8_layout_version": (ctypes.c_int, []),
    "w8a8_packed_weight_bytes": (_sz, [_i64, _i64]),
    "w8a8_pack_weights": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _sz, _vp]),
    "w8a8_unpack_weights": (ctypes.c_int, [_vp, _sz, _i64, _i64, _vp, _vp, _vp]),
    "w8a8_select_path": (ctypes.c_int, [_i64, _i64, _i64]),
    "w8a8_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_gemm": (ctypes.c_int, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "w8a8_gemm_debug": (ctypes.c_int, [_vp, _vp, _vp, _sz, _i64, _i64, _i64, _i32, _i64, _i64,
                                       _vp, _vp, _vp, _sz, _vp]),
    "w8a8_linear_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "w8a8_linear": (ctypes.c_int, [_vp, _i32, _vp, _sz, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "w4a8_linear_noalloc": (ctypes.c_int, [_vp, _i32, _vp, _sz, _i64, _i64, _i64, _i32, _vp, _vp]),
    # include/w4a8_peaks.h
    "w4a8_peak_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "w4a8_peak_mfma_i8": (ctypes.c_int, [_i32, _vp, _vp, _i32, _vp]),
}

_lib = None


class W4A8Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"w4a8 status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_quantized_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != OK:
        lib = load()
        raise W4A8Error(rc, lib.w4a8_last_error().decode())


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


@dataclass
class PackedWeight:
    """A packed weight buffer with the identity that gives it meaning."""
    buf: torch.Tensor          # uint8, w4a8_packed_weight_bytes(N, K, group)
    N: int
    K: int
    group: int
    layout_version: int

    def check(self):
        v = load().w4a8_layout_version()
        if self.layout_version != v:
            raise ValueError(f"packed with layout {self.layout_version}, library has {v}")


def packed_weight_bytes(N: int, K: int, group: int = GROUP) -> int:
    return int(load().w4a8_packed_weight_bytes(N, K, group))


def pack_weights(q: torch.Tensor, z: torch.Tensor | None, s: torch.Tensor, group: int = GROUP,
                 out: torch.Tensor | None = None) -> PackedWeight:
    """q uint8 [N][K] codes 0..15, z uint8 [N][K/group] (None: the symmetric
    grid, every zero point 8), s float32 [N][K/group]."""
    lib = load()
    _need_cuda(q, z, s)
    if q.dtype != torch.uint8 or (z is not None and z.dtype != torch.uint8) or \
            s.dtype != torch.float32:
        raise TypeError("q, z must be uint8 and s float32")
    N, K = q.shape
    nbytes = lib.w4a8_packed_weight_bytes(N, K, group)
    if nbytes == 0:
        _check(lib.w4a8_pack_weights(None, None, None, N, K, group, None, 0, None))
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib.w4a8_pack_weights(_p(q), _p(z), _p(s), N, K, group, _p(out), out.numel(),
                                 _stream(q.device)))
    return PackedWeight(out, N, K, group, lib.w4a8_layout_version())


@dataclass
class SiblingWeight:
    """Sibling projections of one input (query/key/value, gate/up) packed
    side by side as one weight: one activation quantisation and one GEMM
    produce all of them, each a column range of the output."""
    packed: PackedWeight
    widths: tuple

    def split(self, y: torch.Tensor):
        """Per-sibling views of an output [M][sum(widths)] (no copy)."""
        return list(torch.split(y, list(self.widths), dim=1))


def pack_siblings(parts, group: int = GROUP) -> SiblingWeight:
    """parts: [(q, z, s), ...] sharing K; each packed straight into its
    output-channel range of one buffer (w4a8_pack_weights_into)."""
    lib = load()
    if not parts:
        raise ValueError("no parts")
    K = parts[0][0].shape[1]
    widths = tuple(int(q.shape[0]) for q, _, _ in parts)
    N = sum(widths)
    dev = parts[0][0].device
    nbytes = lib.w4a8_packed_weight_bytes(N, K, group)
    if nbytes == 0:
        _check(lib.w4a8_pack_weights(None, None, None, N, K, group, None, 0, None))
    out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    off = 0
    for (q, z, s), n in zip(parts, widths):
        _need_cuda(q, z, s)
        if q.dtype != torch.uint8 or z.dtype != torch.uint8 or s.dtype != torch.float32:
            raise TypeError("q, z must be uint8 and s float32")
        if q.shape[1] != K:
            raise ValueError("sibling projections must share K")
        _check(lib.w4a8_pack_weights_into(_p(q), _p(z), _p(s), n, K, group, _p(out), out.numel(),
                                          N, off, _stream(dev)))
        off += n
    return SiblingWeight(PackedWeight(out, N, K, group, lib.w4a8_layout_version()), widths)


def linear_siblings(x: torch.Tensor, w: SiblingWeight, out=None, workspace=None):
    """All siblings from one quantisation and one GEMM; returns their views."""
    return w.split(linear(x, w.packed, out=out, workspace=workspace))


def unpack_weights(w: PackedWeight):
    lib = load()
    w.check()
    G = w.K // w.group
    dev = w.buf.device
    q = torch.empty((w.N, w.K), dtype=torch.uint8, device=dev)
    z = torch.empty((w.N, G), dtype=torch.uint8, device=dev)
    s = torch.empty((w.N, G), dtype=torch.float32, device=dev)
    _check(lib.w4a8_unpack_weights(_p(w.buf), w.buf.numel(), w.N, w.K, w.group, _p(q), _p(z),
                                   _p(s), _stream(dev)))
    return q, z, s


def quant_act(x: torch.Tensor, qa: torch.Tensor | None = None, sa: torch.Tensor | None = None):
    """x bfloat16 or float32 [M][K] -> (qa int8 [M][K], sa float32 [M])."""
    lib = load()
    _need_cuda(x)
    M, K = x.shape
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(x.dtype)
    qa = torch.empty((M, K), dtype=torch.int8, device=x.device) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=x.device) if sa is None else sa
    _check(lib.w4a8_quant_act(_p(x), dt, M, K, _p(qa), _p(sa), _stream(x.device)))
    return qa, sa


def quant_act_hadamard(x: torch.Tensor, qa: torch.Tensor | None = None,
                       sa: torch.Tensor | None = None):
    """Online Hadamard rotation (each group of 128 by the unnormalised
    Walsh-Hadamard matrix) and the per-token quantisation."""
    lib = load()
    _need_cuda(x)
    M, K = x.shape
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(x.dtype)
    qa = torch.empty((M, K), dtype=torch.int8, device=x.device) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=x.device) if sa is None else sa
    _check(lib.w4a8_quant_act_hadamard(_p(x), dt, M, K, _p(qa), _p(sa), _stream(x.device)))
    return qa, sa


def linear_hadamard(x: torch.Tensor, w: PackedWeight, out=None, workspace=None) -> torch.Tensor:
    """The layer with the online rotation: rotated quantisation, then the GEMM
    against a weight packed from W H / 128."""
    lib = load()
    w.check()
    _need_cuda(x, out)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    dt = BF16 if x.dtype == torch.bfloat16 else F32 if x.dtype == torch.float32 else None
    if dt is None:
        raise TypeError(x.dtype)
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    need = int(lib.w4a8_linear_hadamard_workspace_bytes(M, w.N, w.K, w.group))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    wsb = workspace.numel() * workspace.element_size()
    _check(lib.w4a8_linear_hadamard(_p(x), dt, _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group,
                                    _p(out), _p(workspace), wsb, _stream(x.device)))
    return out


def workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    return int(load().w4a8_gemm_workspace_bytes(M, N, K, group))


def select_path(M: int, N: int, K: int) -> int:
    return int(load().w4a8_select_path(M, N, K))


def _workspace(M, w: PackedWeight, workspace):
    need = workspace_bytes(M, w.N, w.K, w.group)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.buf.device)
    return workspace, workspace.numel() * workspace.element_size()


def gemm(qa: torch.Tensor, sa: torch.Tensor, w: PackedWeight, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 y [M][N] from quantised activations and a packed weight."""
    lib = load()
    w.check()
    _need_cuda(qa, sa)
    M, K = qa.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=qa.device) if out is None else out
    ws, wsb = _workspace(M, w, workspace)
    _check(lib.w4a8_gemm(_p(qa), _p(sa), _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group, _p(out),
                         _p(ws), wsb, _stream(qa.device)))
    return out


def gemm_debug(qa, sa, w: PackedWeight, path: int = PATH_AUTO, rows=None, want_y: bool = True,
               workspace=None):
    """(partials int32 [rows][N][G], y bf16 [M][N] or None) from a forced path."""
    lib = load()
    w.check()
    M, K = qa.shape
    m0, m1 = rows if rows is not None else (0, M)
    G = w.K // w.group
    P = torch.empty((m1 - m0, w.N, G), dtype=torch.int32, device=qa.device)
    y = torch.empty((M, w.N), dtype=torch.bfloat16, device=qa.device) if want_y else None
    ws, wsb = _workspace(M, w, workspace)
    _check(lib.w4a8_gemm_debug(_p(qa), _p(sa), _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group,
                               path, m0, m1, _p(P) if P.numel() else None, _p(y), _p(ws), wsb,
                               _stream(qa.device)))
    return P, y


def linear_workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    return int(load().w4a8_linear_workspace_bytes(M, N, K, group))


def linear(x: torch.Tensor, w: PackedWeight, out=None, workspace=None) -> torch.Tensor:
    """The layer from raw bf16/f32 activations: per-token quantisation and the
    W4A8 GEMM (one launch at M == 1, where the GEMV quantises in-kernel)."""
    lib = load()
    w.check()
    _need_cuda(x, out)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(x.dtype)
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    need = linear_workspace_bytes(M, w.N, w.K, w.group)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w4a8_linear(_p(x), dt, _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group, _p(out),
                           _p(workspace), wsb, _stream(x.device)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_noalloc(x: torch.Tensor, w: PackedWeight, out: torch.Tensor) -> torch.Tensor:
    """w4a8_linear without a workspace (the library's static device scratch);
    `out` must be given, so nothing is allocated."""
    lib = load()
    w.check()
    _need_cuda(x, out)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    dt = BF16 if x.dtype == torch.bfloat16 else F32 if x.dtype == torch.float32 else None
    if dt is None:
        raise TypeError(x.dtype)
    _check(lib.w4a8_linear_noalloc(_p(x), dt, _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group,
                                   _p(out), _stream(x.device)))
    return out


# ------------------------------------------------------------------ W8A8

@dataclass
class PackedW8:
    """A packed W8A8 weight (int8 per channel) with its identity."""
    buf: torch.Tensor          # uint8, w8a8_packed_weight_bytes(N, K)
    N: int
    K: int
    layout_version: int

    def check(self):
        v = load().w8a8_layout_version()
        if self.layout_version != v:
            raise ValueError(f"packed with W8A8 layout {self.layout_version}, library has {v}")


def w8a8_pack_weights(qw: torch.Tensor, sw: torch.Tensor, out: torch.Tensor | None = None) -> PackedW8:
    """qw int8 [N][K], sw float32 [N] -> packed W8A8 weight."""
    lib = load()
    _need_cuda(qw, sw)
    if qw.dtype != torch.int8 or sw.dtype != torch.float32:
        raise TypeError("qw must be int8 and sw float32")
    N, K = qw.shape
    nbytes = lib.w8a8_packed_weight_bytes(N, K)
    if nbytes == 0:
        _check(lib.w8a8_pack_weights(None, None, N, K, None, 0, None))
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=qw.device)
    _check(lib.w8a8_pack_weights(_p(qw), _p(sw), N, K, _p(out), out.numel(), _stream(qw.device)))
    return PackedW8(out, N, K, lib.w8a8_layout_version())


def w8a8_unpack_weights(w: PackedW8):
    lib = load()
    w.check()
    dev = w.buf.device
    qw = torch.empty((w.N, w.K), dtype=torch.int8, device=dev)
    sw = torch.empty((w.N,), dtype=torch.float32, device=dev)
    _check(lib.w8a8_unpack_weights(_p(w.buf), w.buf.numel(), w.N, w.K, _p(qw), _p(sw), _stream(dev)))
    return qw, sw


def w8a8_select_path(M: int, N: int, K: int) -> int:
    return int(load().w8a8_select_path(M, N, K))


def w8a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().w8a8_gemm_workspace_bytes(M, N, K))


def _w8_workspace(M, w: PackedW8, workspace):
    need = w8a8_workspace_bytes(M, w.N, w.K)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.buf.device)
    return workspace, workspace.numel() * workspace.element_size()


def w8a8_gemm(qa: torch.Tensor, sa: torch.Tensor, w: PackedW8, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 y [M][N] from quantised activations and a packed W8A8 weight."""
    lib = load()
    w.check()
    _need_cuda(qa, sa)
    M, K = qa.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=qa.device) if out is None else out
    ws, wsb = _w8_workspace(M, w, workspace)
    _check(lib.w8a8_gemm(_p(qa), _p(sa), _p(w.buf), w.buf.numel(), M, w.N, w.K, _p(out), _p(ws),
                         wsb, _stream(qa.device)))
    return out


def w8a8_gemm_debug(qa, sa, w: PackedW8, path: int = PATH_AUTO, rows=None, want_y: bool = True,
                    workspace=None):
    """(totals int32 [rows][N], y bf16 [M][N] or None) from a forced path."""
    lib = load()
    w.check()
    M, K = qa.shape
    m0, m1 = rows if rows is not None else (0, M)
    P = torch.empty((m1 - m0, w.N), dtype=torch.int32, device=qa.device)
    y = torch.empty((M, w.N), dtype=torch.bfloat16, device=qa.device) if want_y else None
    ws, wsb = _w8_workspace(M, w, workspace)
    _check(lib.w8a8_gemm_debug(_p(qa), _p(sa), _p(w.buf), w.buf.numel(), M, w.N, w.K, path, m0, m1,
                               _p(P) if P.numel() else None, _p(y), _p(ws), wsb,
                               _stream(qa.device)))
    return P, y


def w8a8_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().w8a8_linear_workspace_bytes(M, N, K))


def w8a8_linear(x: torch.Tensor, w: PackedW8, out=None, workspace=None) -> torch.Tensor:
    """W8A8 from raw bf16/f32 activations: per-token quantisation and the
    int8 GEMM (one launch for M <= 16 when the rows fit in LDS)."""
    lib = load()
    w.check()
    _need_cuda(x, out)
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    if x.dtype == torch.bfloat16:
        dt = BF16
    elif x.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(x.dtype)
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    need = w8a8_linear_workspace_bytes(M, w.N, w.K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w8a8_linear(_p(x), dt, _p(w.buf), w.buf.numel(), M, w.N, w.K, _p(out),
                           _p(workspace), wsb, _stream(x.device)))
    return out


# ----------------------------------------------------------------- W4A16

def w4a16_workspace_bytes(M: int, N: int, K: int, group: int = GROUP) -> int:
    return int(load().w4a16_linear_workspace_bytes(M, N, K, group))


def w4a16_select_path(M: int, N: int, K: int) -> int:
    return int(load().w4a16_select_path(M, N, K))


def w4a16_linear(x: torch.Tensor, w: PackedWeight, out=None, workspace=None,
                 path: int = PATH_AUTO) -> torch.Tensor:
    """W4A16: bf16 activations times the packed int4 weights (no activation
    quantisation), bf16 out; `path` forces GEMV (M == 1), SKINNY or PREFILL."""
    lib = load()
    w.check()
    _need_cuda(x, out)
    if x.dtype != torch.bfloat16:
        raise TypeError("W4A16 takes bfloat16 activations")
    M, K = x.shape
    if K != w.K:
        raise ValueError(f"activations have K={K}, weight has K={w.K}")
    out = torch.empty((M, w.N), dtype=torch.bfloat16, device=x.device) if out is None else out
    need = w4a16_workspace_bytes(M, w.N, w.K, w.group)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.w4a16_linear_path(_p(x), _p(w.buf), w.buf.numel(), M, w.N, w.K, w.group, path,
                                 _p(out), _p(workspace), wsb, _stream(x.device)))
    return out


# ------------------------------------------------------------ peak probes

def peak_stream_read(buf: torch.Tensor, blocks: int, sink: torch.Tensor | None = None):
    """One read of `buf` (16-byte multiple) by the streaming probe."""
    _need_cuda(buf)
    if sink is None:
        sink = torch.empty(blocks, dtype=torch.int32, device=buf.device)
    _check(load().w4a8_peak_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                        blocks, _stream(buf.device)))
    return sink


def peak_mfma_i8(iters: int, blocks: int, sink: torch.Tensor | None = None,
                 clocks: torch.Tensor | None = None):
    """Chains of int8 matrix-core instructions; returns (sink, clocks) where
    clocks[b] = (shader cycles, 100 MHz ticks) of workgroup b."""
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    if clocks is None:
        clocks = torch.zeros((blocks, 2), dtype=torch.int64, device="cuda")
    _check(load().w4a8_peak_mfma_i8(iters, _p(sink), _p(clocks), blocks, _stream(sink.device)))
    return sink, clocks

