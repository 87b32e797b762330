"""The C-ABI library on the CPU: it loads, exports every symbol include/qgemm.h
declares, validates arguments before any HIP call, and its host repack is the
documented bijection (checked against the oracle's unpack).  No compute call
reaches a GPU here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

qgm = pytest.importorskip("bit_weight_only_dequant_amd")
lib = qgm._lib
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_ARG, E_UNSUP, E_ALIGN, E_DEVICE, E_NOMEM, E_WS, E_NOT_DEVICE = range(8)
A = 0x10000  # a 16-byte aligned fake address: validation never dereferences it


def header_functions():
    text = open(os.path.join(ROOT, "include", "qgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(qgm.EXPORTED) == names


def gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def qgemm_status(x=A, packed=A, scales=A, zeros=A, M=1, N=16, K=128, group=32, fmt=0, y=A,
                 ldx=None, ldy=None, resid=None, ldr=None, ws=None, ws_bytes=0):
    return lib.qgemm_ex(x, K if ldx is None else ldx, packed, scales, zeros, resid,
                        N if ldr is None else ldr, M, N, K, group, fmt, y,
                        N if ldy is None else ldy, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(fmt=5), E_ARG),
    (dict(fmt=4, group=128), E_ARG),                 # q4k: super-blocks of 256
    (dict(fmt=4, group=256, K=384), E_ARG),          # K % 256
    (dict(fmt=4, group=256, K=256, zeros=None), E_ARG),   # q4k needs its (sc, m) bytes
    (dict(fmt=-1), E_ARG),
    (dict(group=48), E_ARG),
    (dict(group=256), E_ARG),
    (dict(fmt=2, zeros=None, group=64), E_ARG),      # q4_0 needs group 32
    (dict(fmt=2, zeros=A, group=32), E_ARG),         # q4_0 takes no zero points
    (dict(fmt=3, zeros=None, group=128), E_ARG),     # q8_0 needs group 32
    (dict(fmt=3, zeros=A, group=32), E_ARG),         # q8_0 takes no zero points
    (dict(fmt=0, zeros=None), E_ARG),                # asymmetric needs zero points
    (dict(K=100), E_ARG),                            # K % group
    (dict(M=-1), E_ARG),
    (dict(N=-5), E_ARG),
    (dict(K=-32), E_ARG),
    (dict(x=None), E_ARG),
    (dict(packed=None), E_ARG),
    (dict(scales=None), E_ARG),
    (dict(y=None), E_ARG),
    (dict(ldx=64), E_ARG),                           # ldx < K
    (dict(ldy=8), E_ARG),                            # ldy < N
    (dict(x=A + 2), E_ALIGN),
    (dict(packed=A + 4), E_ALIGN),
    (dict(y=A + 8), E_ALIGN),
    (dict(ldx=132), E_ALIGN),                        # row starts not 16-byte aligned
    (dict(resid=A, ldr=4), E_ARG),
    (dict(resid=A, ldr=32, ldy=16), E_ARG),          # residual aliases y with another stride
    (dict(M=128, N=1024, K=8192, ws=A, ws_bytes=16), E_WS),
])
def test_validation_before_any_hip_call(kw, expect):
    if kw.get("resid") == A and kw.get("ldr") == 32:
        kw = dict(kw, y=A)  # alias
    assert qgemm_status(**kw) == expect


def test_empty_calls_are_noops_without_hip():
    assert qgemm_status(M=0) == OK
    assert qgemm_status(N=0) == OK
    assert lib.qgemm(None, None, None, None, 0, 16, 128, 32, 0, None, None) == OK


@pytest.mark.skipif(gpu_present(), reason="checks the no-device status; a GPU is present")
def test_no_device_status():
    assert qgemm_status() == E_DEVICE
    assert lib.qpack(A, A, 16, 128, 0, None) == E_DEVICE


def test_status_strings():
    for s in range(8):
        assert qgm.status_str(s).startswith("QG_")
    assert "unknown" in qgm.status_str(99)


@pytest.mark.parametrize("N,K,fmt,expect", [
    (16, 128, 0, 1024), (17, 128, 0, 2048), (16, 136, 0, 2048), (6144, 2048, 0, 6291456),
    (8192, 2048, 1, 4194304), (8192, 2048, 2, 8388608), (0, 128, 0, 0), (16, 100, 0, 0),
    (16, 128, 5, 0), (8192, 2048, 3, 16777216), (16, 96, 3, 2048), (16, 98, 3, 0),
    (8192, 2048, 4, 8388608)])
def test_packed_bytes(N, K, fmt, expect):
    assert qgm.packed_bytes(N, K, fmt) == expect


def decode_packed_by_formula(packed, N, K, fmt):
    """The packed order as the header documents it, written out in Python."""
    b = oracle.BITS[fmt]
    cpw = 32 // b
    kw_n = K // cpw
    wt = -(-kw_n // 16)
    codes = np.zeros((N, K), dtype=np.uint8)
    for n in range(N):
        for kw in range(kw_n):
            rb, r, T, wi = n // 16, n % 16, kw // 16, kw % 16
            g, t = wi // 4, wi % 4
            word = int(packed[((rb * wt + T) * 64 + g * 16 + r) * 4 + t])
            for j in range(cpw):
                slot = (j & 1) * (cpw // 2) + (j >> 1)
                codes[n, kw * cpw + j] = (word >> (b * slot)) & ((1 << b) - 1)
    return codes


@pytest.mark.parametrize("fmt,N,K", [(0, 16, 128), (0, 37, 96), (1, 20, 256), (1, 33, 160),
                                     (2, 48, 64), (0, 5, 384), (3, 16, 64), (3, 37, 96), (3, 20, 160),
                                     (4, 21, 512)])
def test_host_qpack_layout_and_roundtrip(fmt, N, K):
    c = synth.random_codes_case(N * 7 + K + fmt, fmt, 256 if fmt == 4 else 32, N, K, 1)
    packed = qgm.qpack_host(c.words, N, K, fmt)
    assert packed.nbytes == qgm.packed_bytes(N, K, fmt)
    assert np.array_equal(decode_packed_by_formula(packed, N, K, fmt),
                          oracle.unpack_codes(c.words, N, K, fmt))
    assert np.array_equal(qgm.qunpack_host(packed, N, K, fmt), c.words)
    # padding is zero: the codes of every slot of every packed word (padding
    # included) add up to the canonical codes' sum
    b = oracle.BITS[fmt]
    allcodes = sum(int(((packed >> (b * i)) & ((1 << b) - 1)).sum()) for i in range(32 // b))
    assert allcodes == int(oracle.unpack_codes(c.words, N, K, fmt).astype(np.int64).sum())


def test_host_repack_is_a_permutation_of_codes():
    c = synth.random_codes_case(3, 0, 32, 64, 512, 1)
    packed = qgm.qpack_host(c.words, 64, 512, 0)
    a = np.sort(oracle.unpack_codes(c.words, 64, 512, 0).ravel())
    b = np.sort(decode_packed_by_formula(packed, 64, 512, 0).ravel())
    assert np.array_equal(a, b)


def test_gemv_rows_override(monkeypatch):
    monkeypatch.setenv("QGEMM_GEMV_ROWS", "16")
    assert qgm.plan(1, 6144, 2048, 128, 0)["tile_n"] == 16
    monkeypatch.setenv("QGEMM_GEMV_ROWS", "8")
    assert qgm.plan(1, 8192, 2048, 128, 0)["tile_n"] == 8
    assert (qgm.plan(2, 8192, 2048, 128, 0)["tile_m"], qgm.plan(2, 8192, 2048, 128, 0)["tile_n"]) == (2, 8)
    assert (qgm.plan(4, 8192, 2048, 128, 0)["tile_m"], qgm.plan(4, 8192, 2048, 128, 0)["tile_n"]) == (4, 8)
    assert qgm.plan(5, 8192, 2048, 128, 0)["tile_n"] == 16      # M > 4: MFMA GEMV only
    assert qgm.plan(1, 8192, 2048, 256, 4)["tile_n"] == 8
    # 128 word tiles: past 8 waves x 8 tiles, so 8-row workgroups need K splits
    p = qgm.plan(1, 8192, 16384, 128, 0)
    assert p["tile_n"] == 8 and p["splits"] == 2


@pytest.mark.parametrize("rows", [8, 16])
@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 5, 16])
def test_gemv_rows_override_holds_with_any_split(monkeypatch, rows, M, splits):
    # the plan honours a forced row count for M <= 4 under every forced K
    # split, including counts that equal tile shares round to another count
    monkeypatch.setenv("QGEMM_GEMV_ROWS", str(rows))
    if splits:
        monkeypatch.setenv("QGEMM_SPLITK", str(splits))
    for fmt, group, N, K in [(0, 128, 384, 2048), (1, 64, 272, 4096), (3, 32, 72, 1056), (4, 256, 300, 2048),
                             (0, 64, 48, 6016), (2, 32, 33, 224)]:
        p = qgm.plan(M, N, K, group, fmt)
        assert p["path"] == "gemv" and p["tile_n"] == rows, (fmt, N, K, M, p)


def test_gemv_split_policy():
    # no K split unless the per-workgroup tile cap forces one, or few row blocks
    # carry long K: one launch beats a split plus its reduce launch
    assert qgm.plan(1, 2048, 2048, 128, 0)["splits"] == 1
    assert qgm.plan(1, 512, 4096, 128, 0)["splits"] == 1
    assert qgm.plan(8, 2048, 2048, 128, 0)["splits"] == 1
    assert qgm.plan(2, 512, 4096, 128, 0)["splits"] == 1       # 8-row kernel: 32 tiles per workgroup
    assert qgm.plan(1, 256, 8192, 128, 0)["splits"] > 1        # 16 row blocks x 64 tiles
    assert qgm.plan(8, 1024, 4096, 128, 0)["splits"] == 1      # the MFMA GEMV streams K in chunks
    assert qgm.plan(8, 4096, 14336, 128, 0)["splits"] == 1
    p = qgm.plan(1, 16, 1 << 20, 128, 0)                         # 8192 tiles on one row block
    assert p["splits"] * 64 >= 8192 and p["splits"] <= 256
    # the M <= 2 cost model: 4096 x 14336 stays unsplit on 16-row workgroups (one
    # round of 256), 6144 x 16384 splits in two rather than run 1.5 rounds
    p = qgm.plan(1, 4096, 14336, 128, 0)
    assert (p["tile_n"], p["splits"]) == (16, 1)
    assert qgm.plan(1, 6144, 16384, 128, 0)["splits"] == 2
    assert qgm.plan(1, 6144, 8192, 128, 0)["tile_n"] == 8
    assert qgm.workspace_bytes(1, 2048, 2048, 128, 0) == 0


def test_plans_for_the_workloads():
    assert qgm.plan(1, 6144, 2048, 128, 0)["path"] == "gemv"
    assert qgm.plan(8, 6144, 2048, 128, 0)["path"] == "gemv"
    p = qgm.plan(128, 8192, 2048, 128, 0)
    assert p["path"] == "gemm" and p["workgroups"] >= 128
    assert qgm.plan(16, 64, 128, 32, 0)["path"] == "gemv"
    assert qgm.plan(17, 64, 128, 32, 0)["path"] == "gemm"
    # 17..32 rows: 32 x 32 tiles; 33..64: 64 x 32; above: 64 x 64
    assert (qgm.plan(32, 8192, 2048, 128, 0)["tile_m"], qgm.plan(32, 8192, 2048, 128, 0)["tile_n"]) == (32, 32)
    assert (qgm.plan(33, 8192, 2048, 128, 0)["tile_m"], qgm.plan(33, 8192, 2048, 128, 0)["tile_n"]) == (64, 32)
    assert (qgm.plan(65, 8192, 2048, 128, 0)["tile_m"], qgm.plan(65, 8192, 2048, 128, 0)["tile_n"]) == (64, 64)
    assert qgm.plan(32, 8192, 2048, 128, 0)["workgroups"] == 256
    # 64 x 64 tiles would split K 4 ways at 128 x 2048 x 2048; 32 x 32 tiles fill the CUs unsplit
    p = qgm.plan(128, 2048, 2048, 128, 0)
    assert (p["tile_m"], p["tile_n"], p["splits"]) == (32, 32, 1)
    # K = 8192: 64 x 64 tiles would split 4 ways; 32 x 32 tiles take 8 word tiles per wave, unsplit
    p = qgm.plan(128, 2048, 8192, 128, 0)
    assert (p["tile_m"], p["tile_n"], p["splits"]) == (32, 32, 1)
    assert qgm.workspace_bytes(1, 16, 128, 32, 0) == 0
    assert qgm.workspace_bytes(128, 1024, 8192, 128, 0) > 0   # split-K for small N
    # q8_0: 64-wide word tiles, 4 per GEMM wave, so K = 2048 needs no split
    q = qgm.plan(128, 8192, 2048, 32, 3)
    assert q["path"] == "gemm" and q["splits"] == 1
    assert qgm.plan(1, 6144, 2048, 32, 3)["path"] == "gemv"
    # q4k: 4-bit tiles; its metadata comes per 32-weight sub-block
    k = qgm.plan(128, 8192, 2048, 256, 4)
    assert k["path"] == "gemm" and k["splits"] == 1
    assert qgm.plan(1, 8192, 2048, 256, 4)["path"] == "gemv"
    # M = 1: 8-row workgroups when 16-row ones leave the CUs unevenly loaded
    # (384 row blocks on 256 CUs), 16-row ones when they already fill them
    assert (qgm.plan(1, 6144, 2048, 128, 0)["tile_n"], qgm.plan(1, 6144, 2048, 128, 0)["workgroups"]) == (8, 768)
    assert (qgm.plan(1, 8192, 2048, 128, 0)["tile_n"], qgm.plan(1, 8192, 2048, 128, 0)["workgroups"]) == (16, 512)
    assert qgm.plan(1, 6144, 2048, 32, 3)["tile_n"] == 8
    assert qgm.plan(1, 6144, 2048, 256, 4)["tile_n"] == 8    # q4k too
    assert qgm.plan(8, 6144, 2048, 128, 0)["tile_n"] == 16
    # M = 2: the v_dot2 kernel on 8-row workgroups where they balance, else the MFMA GEMV
    assert (qgm.plan(2, 6144, 2048, 128, 0)["tile_m"], qgm.plan(2, 6144, 2048, 128, 0)["tile_n"]) == (2, 8)
    assert (qgm.plan(2, 8192, 2048, 128, 0)["tile_m"], qgm.plan(2, 8192, 2048, 128, 0)["tile_n"]) == (4, 16)
    assert qgm.plan(3, 6144, 2048, 128, 0)["tile_n"] == 16
    # M = 3, 4: the MFMA GEMV, which streams K unsplit (8-row v_dot2 only when forced)
    p = qgm.plan(4, 2048, 8192, 128, 0)
    assert (p["tile_m"], p["tile_n"], p["splits"]) == (4, 16, 1)
    assert qgm.plan(4, 6144, 8192, 128, 0)["tile_n"] == 16


# hipMemoryType: 0 unregistered, 1 host, 2 device, 3 managed, 10 array, 11 unified
@pytest.mark.parametrize("rc,mtype,pdev,cdev,expect", [
    (0, 2, 0, 0, OK),            # device memory of the current device
    (0, 2, 1, 0, E_NOT_DEVICE),  # another GPU's memory
    (0, 3, 1, 0, OK),            # managed memory is reachable from any device
    (0, 11, 0, 0, OK),           # unified address space
    (0, 1, 0, 0, E_NOT_DEVICE),  # pinned / registered host memory
    (0, 0, 0, 0, E_NOT_DEVICE),  # unregistered
    (0, 10, 0, 0, E_NOT_DEVICE), # arrays
    (1, 2, 0, 0, E_NOT_DEVICE),  # hipPointerGetAttributes failed (plain malloc memory)
])
def test_pointer_classification(rc, mtype, pdev, cdev, expect):
    assert lib.qg_classify_pointer(rc, mtype, pdev, cdev) == expect


def test_dequant_checks_metadata_alignment():
    # q4k reads its (d, dmin) pairs as 32-bit words: scales and zeros must be
    # 16-byte aligned like every other buffer, checked before any HIP call
    assert lib.qg_dequant(A, A + 2, A, A, 16, 256, 256, 4, None) == E_ALIGN
    assert lib.qg_dequant(A, A, A + 8, A, 16, 256, 128, 0, None) == E_ALIGN
    assert lib.qg_dequant(A, A + 4, None, A, 16, 256, 32, 2, None) == E_ALIGN


def test_dequant_empty_is_a_noop():
    assert lib.qg_dequant(None, None, None, None, 0, 256, 128, 0, None) == OK


def _loop_status(D=64, F=128, group=32, fmt=0, M=4, L=2, scales=(A, A, A, A), events=None):
    arr = lambda vals: (ctypes.c_void_p * 4)(*vals)
    zeros = (None,) * 4 if fmt in (2, 3) else (A,) * 4
    ev = None if events is None else (ctypes.c_void_p * (L + 1))(*events)
    return lib.qloop_block(A, arr((A,) * 4), arr(scales), arr(zeros), M, D, F, group, fmt, L, A, ev, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(F=100), E_ARG),                       # F % group: the down projection's K
    (dict(F=96, group=64), E_ARG),
    (dict(D=64, group=32, F=128), OK if gpu_present() else E_DEVICE),   # valid
    (dict(scales=(A, A, A, A + 2)), E_ALIGN),   # the down projection's scales
    (dict(fmt=7), E_ARG),
    (dict(L=-1), E_ARG),
])
def test_loop_block_validates_every_linear_first(kw, expect):
    # on error nothing is launched: the four calls are checked before the first
    # event record or launch, so a bad down projection fails without a GPU
    if expect == OK:
        pytest.skip("valid arguments launch work; covered by the GPU tests")
    assert _loop_status(**kw) == expect


def test_loop_block_records_no_event_on_error():
    # a bad last linear with events given: the status comes back before any
    # HIP call (the events are fake handles that a record would reject)
    assert _loop_status(F=100, events=[A] * 3) == E_ARG


def _persistent_status(M=1, D=64, F=128, group=32, fmt=0, L=2, status=A, mode=0):
    arr = lambda vals: (ctypes.c_void_p * 4)(*vals)
    zeros = (None,) * 4 if fmt in (2, 3) else (A,) * 4
    return lib.qloop_block_persistent(A, arr((A,) * 4), arr((A,) * 4), arr(zeros), M, D, F, group, fmt, L, A,
                                      mode, status, None, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(M=2), E_UNSUP),                  # M = 1 only
    (dict(M=1, fmt=3), E_UNSUP),           # q8_0 is not among its formats
    (dict(D=64, F=128 * 128), E_UNSUP),    # K of down: 2048 word tiles, beyond 8 waves x 8
    (dict(status=None), E_ARG),
    (dict(mode=2), E_ARG),
    (dict(mode=-1), E_ARG),
    (dict(status=A + 4), E_ALIGN),
    (dict(F=100), E_ARG),                        # the same validation as qloop_block
])
def test_persistent_loop_rejects_before_any_hip_call(kw, expect):
    assert _persistent_status(**kw) == expect


def test_noalloc_refuses_oversized_plans_before_any_hip_call():
    # 56 MiB of split-K partials is beyond the fixed per-GPU array (8 MiB):
    # refused during validation, so this holds without a GPU too
    assert qgm.workspace_bytes(512, 4096, 14336, 32, 2) > qgm.NOALLOC_SCRATCH_BYTES
    assert lib.qgemm_noalloc(A, 14336, A, A, None, None, 4096, 512, 4096, 14336, 32, 2, A, 4096, None) == E_WS
    assert lib.qgemm_noalloc(A, 128, A, A, A, None, 16, 0, 16, 128, 32, 0, A, 16, None) == OK   # M = 0: no-op
    assert lib.qgemm_noalloc(A + 2, 128, A, A, A, None, 16, 1, 16, 128, 32, 0, A, 16, None) == E_ALIGN


def test_clock_helpers_validate_before_any_hip_call():
    # the in-graph timing stamps of bench.py: NULL and misaligned outputs are
    # refused on the host
    assert lib.qg_clock_stamp(None, None) == E_ARG
    assert lib.qg_clock_stamp(A + 4, None) == E_ALIGN
    assert lib.qg_clock_rate(0, None) == E_ARG
