"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin."""
import numpy as np
import pytest

from oracle import qref
from tests import pins

_orig_unpack = qref.unpack_codes
_orig_pack = qref.pack_codes
_orig_deq = qref.dequant_f64
_orig_gemm = qref.qgemm_ref


def _unpack_msb_first(words, N, K, fmt):
    c = _orig_unpack(words, N, K, fmt)
    cpw = 32 // qref.BITS[fmt]
    return c.reshape(N, K // cpw, cpw)[:, :, ::-1].reshape(N, K).copy()


def _pack_msb_first(codes, fmt):
    cpw = 32 // qref.BITS[fmt]
    N, K = codes.shape
    return _orig_pack(np.asarray(codes).reshape(N, K // cpw, cpw)[:, :, ::-1].reshape(N, K), fmt)


def _deq_sign(words, scales, zeros, N, K, group, fmt):
    return -_orig_deq(words, scales, zeros, N, K, group, fmt)


def _deq_no_zero(words, scales, zeros, N, K, group, fmt):
    q = _orig_unpack(words, N, K, fmt).astype(np.float32)
    s = np.asarray(scales, np.float16).reshape(N, K // group).astype(np.float32)
    return s[:, np.arange(K) // group] * q


def _deq_group_mod(words, scales, zeros, N, K, group, fmt):
    q = _orig_unpack(words, N, K, fmt).astype(np.float32)
    s, z = qref._group_params(scales, zeros, N, K, group, fmt)
    g = np.arange(K) % (K // group)
    return s[:, g] * (q - z[:, g])


def _deq_q40_offset7(words, scales, zeros, N, K, group, fmt):
    if fmt == qref.Q4_0:
        q = _orig_unpack(words, N, K, fmt).astype(np.float32)
        s = np.asarray(scales, np.float16).reshape(N, K // group).astype(np.float32)
        return s[:, np.arange(K) // group] * (q - 7.0)
    return _orig_deq(words, scales, zeros, N, K, group, fmt)


def _deq_q80_offset127(words, scales, zeros, N, K, group, fmt):
    if fmt == qref.Q8_0:
        q = _orig_unpack(words, N, K, fmt).astype(np.float32)
        s = np.asarray(scales, np.float16).reshape(N, K // group).astype(np.float32)
        return s[:, np.arange(K) // group] * (q - 127.0)
    return _orig_deq(words, scales, zeros, N, K, group, fmt)


def _unpack_q80_low7(words, N, K, fmt):
    c = _orig_unpack(words, N, K, fmt)
    return c & 0x7F if fmt == qref.Q8_0 else c   # a 7-bit mask drops the top bit


def _deq_group_shift(words, scales, zeros, N, K, group, fmt):
    q = _orig_unpack(words, N, K, fmt).astype(np.float32)
    s, z = qref._group_params(scales, zeros, N, K, group, fmt)
    g = np.minimum((np.arange(K) + 1) // group, K // group - 1)
    return s[:, g] * (q - z[:, g])


def _gemm_transposed(x, words, scales, zeros, M, N, K, group, fmt, residual=None):
    x64 = np.asarray(x, np.float16).reshape(M, K).astype(np.float64)
    w = _orig_deq(words, scales, zeros, N, K, group, fmt).astype(np.float64)
    return x64 @ w.reshape(K, N)   # a transposed/reshaped operand


def _gemm_fp16_accumulate(x, words, scales, zeros, M, N, K, group, fmt, residual=None):
    x16 = np.asarray(x, np.float16).reshape(M, K)
    w16 = _orig_deq(words, scales, zeros, N, K, group, fmt).astype(np.float16)
    return (x16 @ w16.T).astype(np.float64)


def _keep_q4k(fn):
    """A mutant of the group formats that leaves q4k alone, so that only the
    pins of the formats it breaks can catch it."""
    def wrapped(words, scales, zeros, N, K, group, fmt):
        if fmt == qref.Q4K:
            return _orig_deq(words, scales, zeros, N, K, group, fmt)
        return fn(words, scales, zeros, N, K, group, fmt)
    return wrapped


def _q4k_params(words, scales, zeros, N, K):
    q = _orig_unpack(words, N, K, qref.Q4K).astype(np.float64)
    ds = np.asarray(scales, np.float16).reshape(N, K // 256, 2).astype(np.float64)
    sm = np.asarray(zeros, np.uint16).reshape(N, K // 32)
    return q, ds, (sm & 0xFF).astype(np.float64), (sm >> 8).astype(np.float64)


def _deq_q4k_no_offset(words, scales, zeros, N, K, group, fmt):
    if fmt != qref.Q4K:
        return _orig_deq(words, scales, zeros, N, K, group, fmt)
    q, ds, sc, m = _q4k_params(words, scales, zeros, N, K)
    sup = np.arange(K // 32) // 8
    return (ds[:, sup, 0] * sc)[:, np.arange(K) // 32] * q


def _deq_q4k_swapped_bytes(words, scales, zeros, N, K, group, fmt):
    if fmt != qref.Q4K:
        return _orig_deq(words, scales, zeros, N, K, group, fmt)
    q, ds, sc, m = _q4k_params(words, scales, zeros, N, K)
    sup = np.arange(K // 32) // 8
    s, b = ds[:, sup, 0] * m, ds[:, sup, 1] * sc      # sc and m read from the wrong bytes
    return s[:, np.arange(K) // 32] * q - b[:, np.arange(K) // 32]


def _deq_q4k_super_index(words, scales, zeros, N, K, group, fmt):
    if fmt != qref.Q4K:
        return _orig_deq(words, scales, zeros, N, K, group, fmt)
    q, ds, sc, m = _q4k_params(words, scales, zeros, N, K)
    sup = np.arange(K // 32) % (K // 256)               # sub-block -> wrong super-block
    s, b = ds[:, sup, 0] * sc, ds[:, sup, 1] * m
    return s[:, np.arange(K) // 32] * q - b[:, np.arange(K) // 32]


def _deq_q4k_dmin_for_d(words, scales, zeros, N, K, group, fmt):
    if fmt != qref.Q4K:
        return _orig_deq(words, scales, zeros, N, K, group, fmt)
    q, ds, sc, m = _q4k_params(words, scales, zeros, N, K)
    sup = np.arange(K // 32) // 8
    s, b = ds[:, sup, 1] * sc, ds[:, sup, 0] * m        # d and dmin exchanged
    return s[:, np.arange(K) // 32] * q - b[:, np.arange(K) // 32]


def _loop_wrong_slice(x0, lin, L, D=2048):
    # O consumes the K third instead of V
    x = np.asarray(x0, np.float16)
    M, outs = x.shape[0], []
    f = lambda a, l, r=None: _orig_gemm(a, l["words"], l["scales"], l["zeros"], M, l["N"], l["K"],
                                       l["group"], l.get("fmt", 0), residual=r).astype(np.float16)
    for _ in range(L):
        qkv, o, up, down = lin
        h = f(f(x, qkv)[:, D:2 * D], o, x)
        x = f(f(h, up), down, h)
        outs.append(x)
    return outs


def _loop_no_second_residual(x0, lin, L, D=2048):
    x = np.asarray(x0, np.float16)
    M, outs = x.shape[0], []
    f = lambda a, l, r=None: _orig_gemm(a, l["words"], l["scales"], l["zeros"], M, l["N"], l["K"],
                                       l["group"], l.get("fmt", 0), residual=r).astype(np.float16)
    for _ in range(L):
        qkv, o, up, down = lin
        h = f(f(x, qkv)[:, 2 * D:3 * D], o, x)
        x = f(f(h, up), down)
        outs.append(x)
    return outs


MUTANTS = {
    "unpack_msb_first": [("unpack_codes", _unpack_msb_first), ("pack_codes", _pack_msb_first)],
    "dequant_sign": [("dequant_f64", _keep_q4k(_deq_sign))],
    "dropped_zero_point": [("dequant_f64", _keep_q4k(_deq_no_zero))],
    "group_index_mod": [("dequant_f64", _keep_q4k(_deq_group_mod))],
    "group_index_shift": [("dequant_f64", _keep_q4k(_deq_group_shift))],
    "q4_0_offset_7": [("dequant_f64", _keep_q4k(_deq_q40_offset7))],
    "q8_0_offset_127": [("dequant_f64", _keep_q4k(_deq_q80_offset127))],
    "q8_0_seven_bit_mask": [("unpack_codes", _unpack_q80_low7)],
    "q4k_dropped_offset": [("dequant_f64", _deq_q4k_no_offset)],
    "loop_wrong_slice": [("loop_block_ref", _loop_wrong_slice)],
    "loop_no_second_residual": [("loop_block_ref", _loop_no_second_residual)],
    "q4k_swapped_bytes": [("dequant_f64", _deq_q4k_swapped_bytes)],
    "q4k_wrong_super_block": [("dequant_f64", _deq_q4k_super_index)],
    "q4k_d_dmin_exchanged": [("dequant_f64", _deq_q4k_dmin_for_d)],
    "transposed_operand": [("qgemm_ref", _gemm_transposed)],
    "fp16_accumulation": [("qgemm_ref", _gemm_fp16_accumulate)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(qref, attr, fn)
    with np.errstate(all="ignore"):   # some mutants overflow fp16 on purpose
        bad = pins.failing_pins(qref)
    assert bad, f"planted mistake {name} passed every pin"


def test_real_oracle_passes_all():
    assert pins.failing_pins(qref) == []
