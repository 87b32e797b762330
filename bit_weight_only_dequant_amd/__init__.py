"""Python binding of libqgemm.so: weight-only low-bit matmul on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``csrc/``; PyTorch provides device memory and the stream.  There is
no CPU fallback: importing this package fails loudly when the library has not
been built (``python bit_weight_only_dequant_amd/build.py``), and device calls
reject tensors that are not on a GPU.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

INT4_ASYM = 0
INT2_ASYM = 1
Q4_0 = 2
Q8_0 = 3
Q4K = 4
BITS = {INT4_ASYM: 4, INT2_ASYM: 2, Q4_0: 4, Q8_0: 8, Q4K: 4}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python bit_weight_only_dequant_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")

# PyTorch-ROCm ships its own HIP runtime with the same soname as the system
# one.  Loading torch first makes libqgemm bind to that already-loaded copy, so
# the library and torch share one runtime (devices, streams, allocations).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_I64 = ctypes.c_int64

_SIGS = {
    "qg_version": ([], _I),
    "qg_status_str": ([_I], ctypes.c_char_p),
    "qg_last_error": ([], ctypes.c_char_p),
    "qg_packed_bytes": ([_I64, _I64, _I], _SZ),
    "qpack": ([_P, _P, _I, _I, _I, _P], _I),
    "qunpack": ([_P, _P, _I, _I, _I, _P], _I),
    "qpack_host": ([_P, _P, _I, _I, _I], _I),
    "qunpack_host": ([_P, _P, _I, _I, _I], _I),
    "qgemm": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P], _I),
    "qgemm_ex": ([_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _SZ, _P], _I),
    "qgemm_workspace_bytes": ([_I, _I, _I, _I, _I], _SZ),
    "qloop_block": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "qg_unpack_codes": ([_P, _P, _I, _I, _I, _P], _I),
    "qg_dequant": ([_P, _P, _P, _P, _I, _I, _I, _I, _P], _I),
    "qg_plan": ([_I, _I, _I, _I, _I, ctypes.POINTER(_I)], _I),
    "qg_classify_pointer": ([_I, _I, _I, _I], _I),
    "qgemm_noalloc": ([_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P], _I),
    "qloop_block_persistent": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P], _I),
    "qg_stream_read": ([_P, _SZ, _P, _I, _P], _I),
    "qg_empty_launch": ([_I, _I, _P], _I),
    "qg_mfma_probe": ([_P, _I, _I, _P], _I),
    "qg_device_info": ([_I] + [ctypes.POINTER(_I)] * 4, _I),
    "qg_clock_stamp": ([_P, _P], _I),
    "qg_clock_rate": ([_I, ctypes.POINTER(_I)], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class QGemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = int(status)
        msg = status_str(status)
        if self.status == 4:
            msg += f" ({_lib.qg_last_error().decode()})"
        super().__init__(f"{what}: {msg}" if what else msg)


def status_str(status: int) -> str:
    return _lib.qg_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QGemmError(status, what)


def version() -> int:
    return _lib.qg_version()


def cpw(fmt: int) -> int:
    return 32 // BITS[fmt]


def packed_bytes(N: int, K: int, fmt: int) -> int:
    return int(_lib.qg_packed_bytes(N, K, fmt))


def workspace_bytes(M: int, N: int, K: int, group: int, fmt: int) -> int:
    return int(_lib.qgemm_workspace_bytes(M, N, K, group, fmt))


def plan(M: int, N: int, K: int, group: int, fmt: int) -> dict:
    out = (_I * 5)()
    _check(_lib.qg_plan(M, N, K, group, fmt, out), "qg_plan")
    return dict(path={1: "gemv", 2: "gemm"}.get(out[0], "none"), splits=out[1],
                workgroups=out[2], tile_m=out[3], tile_n=out[4])


# ----------------------------------------------------------------------------
# host repack (numpy)
# ----------------------------------------------------------------------------

def qpack_host(canon: np.ndarray, N: int, K: int, fmt: int) -> np.ndarray:
    canon = np.ascontiguousarray(canon, dtype=np.uint32)
    out = np.zeros(packed_bytes(N, K, fmt) // 4, dtype=np.uint32)
    _check(_lib.qpack_host(canon.ctypes.data, out.ctypes.data, N, K, fmt), "qpack_host")
    return out


def qunpack_host(packed: np.ndarray, N: int, K: int, fmt: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint32)
    out = np.zeros((N, K // cpw(fmt)), dtype=np.uint32)
    _check(_lib.qunpack_host(packed.ctypes.data, out.ctypes.data, N, K, fmt), "qunpack_host")
    return out


# ----------------------------------------------------------------------------
# device calls (torch tensors on a GPU)
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev(t, what):
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what} must be a tensor on the GPU")
    return t


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device, stream=None) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _meta_shapes(N: int, K: int, group: int, fmt: int):
    """Element counts the kernels read: (scales, zeros or None)."""
    if fmt == Q4K:
        return N * (K // 256) * 2, N * (K // 32)
    if fmt in (Q4_0, Q8_0):
        return N * (K // group), None
    return N * (K // group), N * (K // group)


def _check_weights(packed, scales, zeros, N: int, K: int, group: int, fmt: int, device):
    """The packed codes and metadata hold at least what the kernels read, on
    x's device, with the element types the kernels take."""
    torch = _torch()
    if fmt not in BITS or group <= 0 or K % group or N < 0 or K < 0:
        return   # the library reports the bad argument itself
    for t, what in ((packed, "packed"), (scales, "scales"), (zeros, "zeros")):
        if t is not None and t.device != device:
            raise ValueError(f"{what} is on {t.device}, x on {device}")
    need = packed_bytes(N, K, fmt)
    if packed is not None and packed.numel() * packed.element_size() < need:
        raise ValueError(f"packed holds {packed.numel() * packed.element_size()} bytes, needs {need}")
    ns, nz = _meta_shapes(N, K, group, fmt)
    if scales is not None and (scales.dtype != torch.float16 or scales.numel() < ns):
        raise ValueError(f"scales must be fp16 with at least {ns} elements")
    if zeros is not None and nz is not None:
        zt = torch.int16 if fmt == Q4K else torch.float16
        if zeros.dtype != zt or zeros.numel() < nz:
            raise ValueError(f"zeros must be {zt} with at least {nz} elements")


def _check_out(t, M: int, N: int, what: str, device):
    """An fp16 [M, N] tensor with unit column stride on x's device."""
    torch = _torch()
    if t.dtype != torch.float16 or t.dim() != 2 or tuple(t.shape) != (M, N) or t.device != device:
        raise ValueError(f"{what} must be an fp16 [{M}, {N}] tensor on {device}")
    if N > 1 and M > 0 and t.stride(1) != 1:
        raise ValueError(f"{what} must have unit column stride")


def to_words_tensor(words: np.ndarray, device="cuda"):
    """uint32 numpy words -> int32 device tensor holding the same bits."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(words, dtype=np.uint32).view(np.int32)).to(device)


def to_half_tensor(a: Optional[np.ndarray], device="cuda"):
    if a is None:
        return None
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)


def to_bits16_tensor(a: Optional[np.ndarray], device="cuda"):
    """16-bit integer metadata (q4k's sc | m << 8) -> int16 device tensor
    holding the same bits."""
    if a is None:
        return None
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)


def qpack(canon, N: int, K: int, fmt: int, out=None, stream=None):
    """canonical words (int32 bits, [N, K/cpw], device) -> packed buffer (int32, device)."""
    torch = _torch()
    _dev(canon, "canon")
    n_words = packed_bytes(N, K, fmt) // 4
    if out is None:
        out = torch.empty(n_words, dtype=torch.int32, device=canon.device)
    _check(_lib.qpack(_ptr(canon), _ptr(out), N, K, fmt, _stream(canon.device, stream)), "qpack")
    return out


def qunpack(packed, N: int, K: int, fmt: int, stream=None):
    torch = _torch()
    _dev(packed, "packed")
    out = torch.empty((N, K // cpw(fmt)), dtype=torch.int32, device=packed.device)
    _check(_lib.qunpack(_ptr(packed), _ptr(out), N, K, fmt, _stream(packed.device, stream)), "qunpack")
    return out


def unpack_codes(packed, N: int, K: int, fmt: int, stream=None):
    torch = _torch()
    _dev(packed, "packed")
    out = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    _check(_lib.qg_unpack_codes(_ptr(packed), _ptr(out), N, K, fmt, _stream(packed.device, stream)),
           "qg_unpack_codes")
    return out


def dequant(packed, scales, zeros, N: int, K: int, group: int, fmt: int, stream=None):
    """fp16 [N, K] weights: fp16_rne(s * (q - z)), the GEMM's own dequant."""
    torch = _torch()
    out = torch.empty((N, K), dtype=torch.float16, device=packed.device)
    return dequant_into(packed, scales, zeros, N, K, group, fmt, out, stream=stream)


def dequant_into(packed, scales, zeros, N: int, K: int, group: int, fmt: int, out, stream=None):
    """As `dequant`, into a caller-owned contiguous fp16 [N, K] tensor."""
    torch = _torch()
    _dev(packed, "packed"); _dev(scales, "scales"); _dev(zeros, "zeros"); _dev(out, "out")
    if out.dtype != torch.float16 or tuple(out.shape) != (N, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 [N, K] tensor")
    _check_weights(packed, scales, zeros, N, K, group, fmt, out.device)
    _check(_lib.qg_dequant(_ptr(packed), _ptr(scales), _ptr(zeros), _ptr(out), N, K, group, fmt,
                           _stream(packed.device, stream)), "qg_dequant")
    return out


def qgemm(x, packed, scales, zeros, N: int, K: int, group: int, fmt: int, out=None,
          residual=None, workspace=None, stream=None):
    """y = x . dequant(W)^T (+ residual).  x: fp16 [M, K] with unit column
    stride (any row stride that is a multiple of 8); returns fp16 [M, N]."""
    torch = _torch()
    _dev(x, "x"); _dev(packed, "packed"); _dev(scales, "scales"); _dev(zeros, "zeros")
    _dev(residual, "residual"); _dev(out, "out"); _dev(workspace, "workspace")
    # unit column stride whatever M is: a one-row view with another stride
    # (x[:, ::2], buf.t()[0:1]) would otherwise be read as K contiguous halves
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != K or (K > 1 and x.stride(1) != 1):
        raise ValueError("x must be an fp16 [M, K] tensor with unit column stride")
    M = x.shape[0]
    _check_weights(packed, scales, zeros, N, K, group, fmt, x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check_out(out, M, N, "out", x.device)
    if residual is not None:
        _check_out(residual, M, N, "residual", x.device)
    ldx = x.stride(0) if M > 1 else K
    ldy = out.stride(0) if M > 1 else N
    ldr = (residual.stride(0) if M > 1 else N) if residual is not None else N
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = _lib.qgemm_ex(_ptr(x), ldx, _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(residual), ldr,
                       M, N, K, group, fmt, _ptr(out), ldy, ws_ptr, ws_bytes, _stream(x.device, stream))
    _check(st, "qgemm")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # QGEMM_NOALLOC_SCRATCH_BYTES of include/qgemm.h


def qgemm_noalloc(x, packed, scales, zeros, N: int, K: int, group: int, fmt: int, out,
                  residual=None, stream=None):
    """The `qgemm_noalloc` entry point: as `qgemm` into a caller-owned `out`,
    with split-K partials in the library's fixed per-GPU array (no device
    allocation anywhere in the call)."""
    torch = _torch()
    _dev(x, "x"); _dev(packed, "packed"); _dev(scales, "scales"); _dev(zeros, "zeros")
    _dev(residual, "residual"); _dev(out, "out")
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != K or (K > 1 and x.stride(1) != 1):
        raise ValueError("x must be an fp16 [M, K] tensor with unit column stride")
    M = x.shape[0]
    _check_weights(packed, scales, zeros, N, K, group, fmt, x.device)
    _check_out(out, M, N, "out", x.device)
    if residual is not None:
        _check_out(residual, M, N, "residual", x.device)
    ldx = x.stride(0) if M > 1 else K
    ldy = out.stride(0) if M > 1 else N
    ldr = (residual.stride(0) if M > 1 else N) if residual is not None else N
    st = _lib.qgemm_noalloc(_ptr(x), ldx, _ptr(packed), _ptr(scales), _ptr(zeros), _ptr(residual), ldr,
                            M, N, K, group, fmt, _ptr(out), ldy, _stream(x.device, stream))
    _check(st, "qgemm_noalloc")
    return out


def qgemm_plain(x, packed, scales, zeros, N: int, K: int, group: int, fmt: int, out, stream=None):
    """The plain `qgemm` entry point (contiguous x and y, library workspace)."""
    torch = _torch()
    _dev(x, "x"); _dev(out, "out")
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [M, K] tensor")
    _check_weights(packed, scales, zeros, N, K, group, fmt, x.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _check_out(out, x.shape[0], N, "out", x.device)
    st = _lib.qgemm(_ptr(x), _ptr(packed), _ptr(scales), _ptr(zeros), x.shape[0], N, K, group, fmt,
                    _ptr(out), _stream(x.device, stream))
    _check(st, "qgemm")
    return out


class QuantLinear:
    """One quantized weight matrix resident on the GPU in packed form."""

    def __init__(self, words: np.ndarray, scales: np.ndarray, zeros: Optional[np.ndarray],
                 N: int, K: int, group: int, fmt: int, device="cuda"):
        self.N, self.K, self.group, self.fmt = N, K, group, fmt
        canon = to_words_tensor(words, device)
        self.packed = qpack(canon, N, K, fmt)
        self.scales = to_half_tensor(scales, device)
        # q4k: zeros carries the (sc, m) bytes, not fp16 values
        self.zeros = to_bits16_tensor(zeros, device) if fmt == Q4K else to_half_tensor(zeros, device)
        self.weight_bytes = (self.packed.numel() * 4 + self.scales.numel() * 2 +
                             (0 if self.zeros is None else self.zeros.numel() * 2))

    @classmethod
    def from_case(cls, case, device="cuda"):
        return cls(case.words, case.scales, case.zeros, case.N, case.K, case.group, case.fmt, device)

    def __call__(self, x, out=None, residual=None, workspace=None, stream=None):
        return qgemm(x, self.packed, self.scales, self.zeros, self.N, self.K, self.group, self.fmt,
                     out=out, residual=residual, workspace=workspace, stream=stream)


def _loop_args(x, linears, L, scratch, events, stream):
    """Checked arguments of qloop_block / qloop_block_persistent."""
    torch = _torch()
    _dev(x, "x")
    qkv, o, up, down = linears
    if x.dtype != torch.float16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [M, D] tensor")
    M, D = x.shape
    F = up.N
    fmt, group = qkv.fmt, qkv.group
    shapes = [(l.N, l.K) for l in linears]
    if shapes != [(3 * D, D), (D, D), (F, D), (D, F)]:
        raise ValueError(f"linears must be QKV [3D, D], O [D, D], up [F, D], down [D, F] for D = {D}; got {shapes}")
    if any(l.fmt != fmt or l.group != group for l in linears):
        raise ValueError("the four linears must share one format and group")
    if L < 0:
        raise ValueError("L must be >= 0")
    need = M * (3 * D + D + F)
    if scratch is None:
        scratch = torch.empty(need, dtype=torch.float16, device=x.device)
    elif scratch.dtype != torch.float16 or scratch.numel() < need or scratch.device != x.device:
        raise ValueError(f"scratch must be fp16 with at least {need} elements on {x.device}")
    if events is not None and len(events) != L + 1:
        raise ValueError("events must hold L + 1 events")
    arr = lambda vals: (ctypes.c_void_p * 4)(*vals)
    packed4 = arr([l.packed.data_ptr() for l in linears])
    scales4 = arr([l.scales.data_ptr() for l in linears])
    zeros4 = arr([None if l.zeros is None else l.zeros.data_ptr() for l in linears])
    ev = None
    if events is not None:
        handles = []
        for e in events:
            if hasattr(e, "cuda_event"):
                if not e.cuda_event:      # torch creates the HIP event on first record
                    e.record(torch.cuda.current_stream(x.device))
                handles.append(e.cuda_event)
            else:
                handles.append(e)
        ev = (ctypes.c_void_p * (L + 1))(*handles)
    return (packed4, scales4, zeros4, M, D, F, group, fmt, scratch, ev, _stream(x.device, stream))


def loop_block(x, linears: Sequence[QuantLinear], L: int, scratch=None, events=None, stream=None):
    """Run the looped shared block in place on x (fp16 [M, D]); see qloop_block."""
    packed4, scales4, zeros4, M, D, F, group, fmt, scratch, ev, st_ = _loop_args(x, linears, L, scratch, events,
                                                                                  stream)
    st = _lib.qloop_block(_ptr(x), packed4, scales4, zeros4, M, D, F, group, fmt, L, _ptr(scratch), ev, st_)
    _check(st, "qloop_block")
    return x


def loop_block_persistent(x, linears: Sequence[QuantLinear], L: int, scratch=None, status=None, events=None,
                          stream=None, one_launch: bool = False):
    """The looped shared block at M = 1 with one launch per loop, or with one
    launch for all L loops (one_launch), grid barriers between the GEMVs; see
    qloop_block_persistent.  Returns (x, status): status is an int32 device
    tensor, 0 once the loops completed and 1 if a barrier stopped waiting
    (read it after synchronizing)."""
    torch = _torch()
    packed4, scales4, zeros4, M, D, F, group, fmt, scratch, ev, st_ = _loop_args(x, linears, L, scratch, events,
                                                                                  stream)
    if status is None:
        status = torch.zeros(4, dtype=torch.int32, device=x.device)
    elif status.dtype != torch.int32 or status.device != x.device:
        raise ValueError("status must be an int32 tensor on x's device")
    st = _lib.qloop_block_persistent(_ptr(x), packed4, scales4, zeros4, M, D, F, group, fmt, L, _ptr(scratch),
                                     1 if one_launch else 0, _ptr(status), ev, st_)
    _check(st, "qloop_block_persistent")
    return x, status


# ----------------------------------------------------------------------------
# Measurement helpers (not on the qGEMM path): the ceilings a kernel is read
# against, taken on the device it runs on.

MFMA_PROBE_FLOPS = 16 * 16 * 32 * 2 * 16   # per wave per qg_mfma_probe round


def stream_read(src, nbytes: int, sink, workgroups: int, stream=None):
    """Plain streaming read of the first `nbytes` bytes of device tensor `src`."""
    _dev(src, "src")
    _dev(sink, "sink")
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds src")
    if sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink must hold one uint32 per workgroup")
    _check(_lib.qg_stream_read(_ptr(src), nbytes, _ptr(sink), workgroups, _stream(src.device, stream)),
           "qg_stream_read")


def empty_launch(workgroups: int, threads: int, stream=None):
    """An empty kernel of workgroups x threads on the current device."""
    torch = _torch()
    _check(_lib.qg_empty_launch(workgroups, threads, _stream(torch.cuda.current_device(), stream)),
           "qg_empty_launch")


def mfma_probe(out, workgroups: int, iters: int, stream=None):
    """Back-to-back independent fp16 MFMAs: iters * MFMA_PROBE_FLOPS per wave,
    4 waves per workgroup; out: float32 device tensor of workgroups * 256."""
    _dev(out, "out")
    torch = _torch()
    if out.dtype != torch.float32 or out.numel() < workgroups * 256:
        raise ValueError("out must be float32 with workgroups * 256 elements")
    _check(_lib.qg_mfma_probe(_ptr(out), workgroups, iters, _stream(out.device, stream)), "qg_mfma_probe")


def clock_stamp(out, stream=None):
    """The device's constant-rate clock into out[0] (an int64 device tensor),
    in stream order: two stamps bracket exactly the launches between them."""
    _dev(out, "out")
    torch = _torch()
    if out.dtype != torch.int64 or out.numel() < 1:
        raise ValueError("out must be an int64 device tensor with at least one element")
    _check(_lib.qg_clock_stamp(_ptr(out), _stream(out.device, stream)), "qg_clock_stamp")


def clock_rate_khz(device: int = 0) -> int:
    """Rate of the clock clock_stamp reads, in kHz."""
    v = _I()
    _check(_lib.qg_clock_rate(device, ctypes.byref(v)), "qg_clock_rate")
    return v.value


def device_info(device: int = 0) -> dict:
    """Compute units and clocks of `device` as the HIP runtime reports them."""
    v = [_I() for _ in range(4)]
    _check(_lib.qg_device_info(device, *[ctypes.byref(x) for x in v]), "qg_device_info")
    return dict(compute_units=v[0].value, clock_khz=v[1].value, memory_clock_khz=v[2].value,
                memory_bus_bits=v[3].value)
