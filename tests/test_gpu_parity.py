"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work (repack, code unpack) is compared bit for bit; the dequantized
fp16 weight bit for bit against fp16_rne(s*(q-z)); y within
max|y - y_ref| <= 2e-3 * max|y_ref|, and bit for bit where the arithmetic is
exact (one-hot x; x in {-1,0,1} with power-of-two scales).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from tests import pins

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)
import bit_weight_only_dequant_amd as qgm  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def dev_half(a):
    return qgm.to_half_tensor(a, DEV)


def ref_y(case, x, residual=None):
    return oracle.qgemm_ref(x, case.words, case.scales, case.zeros, x.shape[0], case.N, case.K,
                            case.group, case.fmt, residual=residual)


def run_gemm(lin, x_np, residual=None, **kw):
    x = dev_half(x_np)
    r = dev_half(residual) if residual is not None else None
    y = lin(x, residual=r, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_close(y, yr, what):
    err = oracle.rel_error(y, yr)
    say(f"  {what}: rel err {err:.3e}")
    assert np.all(np.isfinite(y)), what
    assert oracle.within_tolerance(y, yr), f"{what}: rel err {err}"


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    monkeypatch.delenv("QGEMM_FORCE", raising=False)
    monkeypatch.delenv("QGEMM_SPLITK", raising=False)
    monkeypatch.delenv("QGEMM_GEMV_ROWS", raising=False)
    monkeypatch.delenv("QGEMM_GEMM_TILE", raising=False)
    yield


# ----------------------------------------------------------------------------
# integer work: repack and unpack, bit-exact
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,group,N,K", [(0, 32, 256, 256), (0, 128, 6144, 2048), (1, 64, 8192, 2048),
                                           (2, 32, 8192, 2048), (0, 32, 37, 96), (1, 32, 50, 160),
                                           (2, 32, 3, 32), (3, 32, 8192, 2048), (3, 32, 37, 96),
                                           (3, 32, 5, 32), (4, 256, 512, 2048), (4, 256, 17, 256)])
def test_repack_and_codes_bit_exact(fmt, group, N, K):
    say(f"repack fmt={fmt} N={N} K={K}")
    c = synth.random_codes_case(N + K + fmt, fmt, group, N, K, 1)
    canon = qgm.to_words_tensor(c.words, DEV)
    packed = qgm.qpack(canon, N, K, fmt)
    host = qgm.qpack_host(c.words, N, K, fmt)
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), host)
    back = qgm.qunpack(packed, N, K, fmt)
    assert np.array_equal(back.cpu().numpy().view(np.uint32), c.words)
    codes = qgm.unpack_codes(packed, N, K, fmt)
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack_codes(c.words, N, K, fmt))


@pytest.mark.parametrize("fmt,group,N,K", [(0, 32, 256, 256), (0, 128, 512, 2048), (1, 64, 256, 2048),
                                           (1, 32, 64, 512), (2, 32, 256, 2048), (0, 64, 40, 192),
                                           (3, 32, 256, 2048), (3, 32, 40, 96)])
def test_dequant_bit_exact(fmt, group, N, K):
    say(f"dequant fmt={fmt} g={group} N={N} K={K}")
    c = synth.random_codes_case(7 * N + K + fmt, fmt, group, N, K, 1)
    lin = qgm.QuantLinear.from_case(c, DEV)
    w = qgm.dequant(lin.packed, lin.scales, lin.zeros, N, K, group, fmt)
    expect = oracle.dequant_f16(c.words, c.scales, c.zeros, N, K, group, fmt)
    got = w.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), expect.view(np.uint16))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

WL = [("tiny_int4_g32", 1), ("tiny_int4_g32", 4), ("decode_int4_g128", 1), ("decode_int4_g128", 8),
      ("prefill_int4_g128", 128), ("int2_g64", 1), ("int2_g64", 128), ("q4_0_b32", 1), ("q4_0_b32", 128),
      ("q8_0_b32", 1), ("q8_0_b32", 8), ("q8_0_b32", 128), ("q4k_s256", 1), ("q4k_s256", 8),
      ("q4k_s256", 128)]

_cases = {}


def get_case(name):
    if name not in _cases:
        c = synth.workload(name)
        _cases[name] = (c, qgm.QuantLinear.from_case(c, DEV))
    return _cases[name]


@pytest.mark.parametrize("name,M", WL, ids=[f"{n}-M{m}" for n, m in WL])
def test_workload_parity(name, M):
    c, lin = get_case(name)
    say(f"workload {name} M={M} plan={qgm.plan(M, c.N, c.K, c.group, c.fmt)}")
    x = c.x[:M]
    y = run_gemm(lin, x)
    check_close(y, ref_y(c, x), f"{name} M={M}")
    # codes of the packed buffer are the oracle's codes
    codes = qgm.unpack_codes(lin.packed, c.N, c.K, c.fmt).cpu().numpy()
    assert np.array_equal(codes, c.codes)


def test_row0_consistency():
    c, lin = get_case("decode_int4_g128")
    y1 = run_gemm(lin, c.x[:1])
    y8 = run_gemm(lin, c.x[:8])
    check_close(y8[:1], ref_y(c, c.x[:1]), "row 0 of M=8")
    assert oracle.rel_error(y8[:1], y1) <= 2e-3


# ----------------------------------------------------------------------------
# ragged shapes, forced paths, split-K variants
# ----------------------------------------------------------------------------

RAGGED = [
    # fmt, group, N, K, M
    (0, 32, 16, 32, 1), (0, 32, 100, 96, 3), (0, 64, 130, 192, 5), (0, 128, 1000, 384, 7),
    (0, 128, 48, 2048, 8), (1, 32, 40, 160, 2), (1, 64, 272, 320, 6), (2, 32, 33, 224, 4),
    (0, 32, 100, 96, 9), (0, 64, 130, 192, 17), (0, 128, 1000, 384, 100), (0, 128, 300, 2048, 129),
    (1, 32, 40, 160, 33), (1, 64, 272, 320, 127), (2, 32, 33, 224, 200), (2, 32, 520, 1056, 257),
    (0, 128, 2048, 8192, 130),
    (0, 128, 300, 2048, 16), (1, 32, 72, 512, 12), (2, 32, 48, 1024, 16), (0, 64, 520, 4352, 11),
    # q8_0: a word tile is 64 wide, so K = 32 mod 64 leaves half a tile
    (3, 32, 16, 32, 1), (3, 32, 100, 96, 3), (3, 32, 33, 224, 4), (3, 32, 130, 160, 12),
    (3, 32, 72, 544, 17), (3, 32, 300, 2048, 129), (3, 32, 520, 1056, 257), (3, 32, 1000, 4096, 64),
    (3, 32, 48, 8192, 8), (3, 32, 40, 8224, 1), (3, 32, 64, 96, 100),
    # q4k: K a multiple of 256
    (4, 256, 16, 256, 1), (4, 256, 100, 512, 3), (4, 256, 33, 768, 12), (4, 256, 130, 1280, 17),
    (4, 256, 300, 2048, 129), (4, 256, 520, 4352, 257), (4, 256, 48, 8192, 8), (4, 256, 40, 8192, 1),
    (4, 256, 64, 256, 100), (4, 256, 1000, 4096, 64),
    # 17 <= M <= 32: 32 x 32 GEMM tiles (with and without split-K)
    (0, 128, 300, 2048, 32), (1, 64, 272, 320, 24), (2, 32, 520, 1056, 20), (3, 32, 100, 96, 32),
    (4, 256, 64, 512, 30), (0, 128, 2048, 8192, 32), (0, 32, 33, 96, 31), (3, 32, 2048, 2048, 18),
    # 33 <= M <= 64: 64 x 32 tiles
    (0, 128, 300, 2048, 48), (4, 256, 130, 1280, 40), (2, 32, 520, 1056, 64), (1, 64, 2048, 8192, 60),
    (3, 32, 72, 544, 33),
]


@pytest.mark.parametrize("fmt,group,N,K,M", RAGGED)
def test_ragged_parity(fmt, group, N, K, M):
    say(f"ragged fmt={fmt} g={group} N={N} K={K} M={M} plan={qgm.plan(M, N, K, group, fmt)}")
    c = synth.random_codes_case(N * 31 + K * 7 + M + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), "ragged")


@pytest.mark.parametrize("force,M", [("gemm", 1), ("gemm", 3), ("gemm", 4), ("gemm", 8), ("gemm", 16)])
@pytest.mark.parametrize("fmt,group", [(0, 128), (1, 64), (2, 32), (3, 32), (4, 256)])
def test_forced_path(monkeypatch, force, M, fmt, group):
    monkeypatch.setenv("QGEMM_FORCE", force)
    N, K = 272, 1024
    say(f"forced {force} fmt={fmt} M={M} plan={qgm.plan(M, N, K, group, fmt)}")
    c = synth.random_codes_case(11 + M + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), f"forced {force}")


@pytest.mark.parametrize("fmt,group,N,K,M", [(0, 128, 16, 1 << 20, 1), (3, 32, 32, 1 << 19, 1),
                                             (0, 32, 64, 1 << 18, 40), (4, 256, 16, 1 << 18, 8)])
def test_very_long_k(fmt, group, N, K, M):
    # hundreds of K splits (a single row block or column tile), through every path
    say(f"long K fmt={fmt} N={N} K={K} M={M} plan={qgm.plan(M, N, K, group, fmt)}")
    c = synth.random_codes_case(K + M + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), "long K")


@pytest.mark.parametrize("fmt,group,N,K,M", [(0, 128, 131080, 256, 1), (3, 32, 65544, 128, 2),
                                             (0, 32, 65544, 256, 8), (4, 256, 40968, 256, 40),
                                             (1, 64, 98312, 256, 130)])
def test_very_wide_n(fmt, group, N, K, M):
    # tens of thousands of row blocks (large grid x, ragged last block) through every path
    say(f"wide N fmt={fmt} N={N} K={K} M={M} plan={qgm.plan(M, N, K, group, fmt)}")
    c = synth.random_codes_case(N + K + M + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), "wide N")


def test_offset_guards_reject_oversized_shapes():
    # shapes whose byte offsets would not fit the kernels' 32-bit arithmetic are
    # refused before any launch (the pointers are never dereferenced)
    import ctypes
    lib = qgm._lib
    buf = torch.zeros(1 << 16, dtype=torch.int32, device=DEV)
    p = buf.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    E_UNSUP = 2
    # M * ldx * 2 >= 2^32: GEMV (M = 2) and GEMM (M = 17)
    for M in (2, 17):
        ldx = (1 << 32) // (2 * M) + 8
        ldx -= ldx % 8
        assert lib.qgemm_ex(p, ldx, p, p, p, None, 16, M, 16, 128, 128, 0, p, 16, None, 0, st) == E_UNSUP
    # one row block's codes past 4 GiB: K = 2^29 INT4
    K = 1 << 29
    assert lib.qgemm_ex(p, K, p, p, p, None, 16, 1, 16, K, 128, 0, p, 16, None, 0, st) == E_UNSUP
    torch.cuda.synchronize()


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 16])
@pytest.mark.parametrize("M", [2, 24, 64, 100])
def test_split_k_variants(monkeypatch, splits, M):
    monkeypatch.setenv("QGEMM_SPLITK", str(splits))
    N, K, group, fmt = 384, 2048, 128, 0
    say(f"splitk={splits} M={M} plan={qgm.plan(M, N, K, group, fmt)}")
    c = synth.random_codes_case(splits * 100 + M, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), f"splitk {splits}")


# M = 1, 2, 4 through 16-row workgroups (v_dot2 kernel for M = 1, MFMA GEMV
# above) and 8-row (half row block) v_dot2 workgroups of 4 x 2, 8 x 2, 8 x 4
# and 8 x 8 word tiles, with and without split-K, ragged N and K, and a fused
# residual
HALF_CASES = [
    # fmt, group, N, K, splits (0: the plan's own)
    (0, 128, 6144, 2048, 0), (0, 32, 100, 96, 0), (0, 64, 1000, 1024, 0), (0, 128, 4100, 4096, 0),
    (0, 128, 384, 2048, 3), (1, 64, 272, 2048, 0), (1, 32, 40, 8192, 0), (1, 64, 272, 4096, 5),
    (2, 32, 33, 224, 0), (2, 32, 6144, 2048, 0), (2, 32, 520, 1056, 2), (3, 32, 6144, 2048, 0),
    (3, 32, 130, 160, 0), (3, 32, 72, 1056, 3), (3, 32, 300, 2080, 0),
    # 33..64 word tiles per workgroup: 8 waves of 8 tiles on 8-row workgroups
    (0, 128, 520, 8192, 0), (3, 32, 520, 4096, 0), (0, 64, 48, 6016, 1),
    # q4k: (d*sc, dmin*m) per sub-block and per-run x sums on either row count
    (4, 256, 6144, 2048, 0), (4, 256, 130, 1280, 0), (4, 256, 520, 8192, 0), (4, 256, 300, 2048, 3),
]


@pytest.mark.parametrize("M", [1, 2, 4])
@pytest.mark.parametrize("rows", [8, 16])
@pytest.mark.parametrize("fmt,group,N,K,splits", HALF_CASES)
def test_gemv_row_variants(monkeypatch, M, rows, fmt, group, N, K, splits):
    monkeypatch.setenv("QGEMM_GEMV_ROWS", str(rows))
    if splits:
        monkeypatch.setenv("QGEMM_SPLITK", str(splits))
    p = qgm.plan(M, N, K, group, fmt)
    say(f"gemv M={M} rows={rows} fmt={fmt} g={group} N={N} K={K} plan={p}")
    assert p["path"] == "gemv" and p["tile_n"] == rows
    c = synth.random_codes_case(N + 3 * K + fmt + rows + 7 * M, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    res = synth.draw_x(np.random.default_rng(N + K), M, N) if N % 2 else None
    check_close(run_gemm(lin, c.x, residual=res), ref_y(c, c.x, residual=res), f"M {M} rows {rows}")


# GEMM tiles forced to each shape (32 x 32, 64 x 32, 64 x 64) on ragged M, N, K
@pytest.mark.parametrize("tile", [3232, 6432, 6464])
@pytest.mark.parametrize("fmt,group,N,K,M", [(0, 128, 300, 2048, 129), (3, 32, 100, 96, 100),
                                             (1, 64, 272, 320, 127), (4, 256, 130, 1280, 70),
                                             (2, 32, 520, 1056, 40)])
def test_gemm_tile_variants(monkeypatch, tile, fmt, group, N, K, M):
    monkeypatch.setenv("QGEMM_GEMM_TILE", str(tile))
    p = qgm.plan(M, N, K, group, fmt)
    say(f"gemm tile {tile} fmt={fmt} g={group} N={N} K={K} M={M} plan={p}")
    assert (p["tile_m"], p["tile_n"]) == (tile // 100, tile % 100)
    c = synth.random_codes_case(tile + N + K + M + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), f"tile {tile}")


# GEMM stage issue: word tiles per wave (TPW) follow the split, and every wave
# issues all TPW x stages (those past its share clamped, not computed) when at
# most an eighth would be wasted, else only its own.  Each case names the TPW
# and mode it reaches; ragged K and short waves on both modes and both depths.
def gemm_issue_mode(fmt, K, splits, small=False):
    cpw = {0: 8, 1: 16, 2: 8, 3: 4, 4: 8}[fmt]
    wordtiles = -(-(K // cpw) // 16)
    tps = -(-wordtiles // splits)
    per = -(-tps // 8)
    tmax = 8 if small else 4 if fmt == 3 else 2
    tpw = 1 if per <= 1 else 2 if per <= 2 or tmax == 2 else 4 if per <= 4 or tmax == 4 else 8
    return tpw, 8 * (8 * tpw - tps) <= 8 * tpw


@pytest.mark.parametrize("tile", [3232, 6464])
@pytest.mark.parametrize("fmt,group,K,splits,tpw,all_", [
    (0, 128, 1024, 1, 1, True), (0, 128, 2048, 1, 2, True), (0, 128, 2048, 4, 1, False),
    (0, 128, 1920, 1, 2, True), (0, 128, 1664, 1, 2, False),
    (3, 32, 2048, 1, 4, True), (3, 32, 1344, 1, 4, False), (3, 32, 1984, 1, 4, True),
    (1, 64, 2048, 1, 1, True), (1, 64, 2048, 2, 1, False),
    (4, 256, 2048, 1, 2, True), (4, 256, 1792, 1, 2, True), (2, 32, 1056, 1, 2, False)])
def test_gemm_stage_issue_modes(monkeypatch, tile, fmt, group, K, splits, tpw, all_):
    monkeypatch.setenv("QGEMM_GEMM_TILE", str(tile))
    monkeypatch.setenv("QGEMM_SPLITK", str(splits))
    N, M = 200, 72
    p = qgm.plan(M, N, K, group, fmt)
    say(f"gemm issue tile {tile} fmt={fmt} g={group} K={K} splits={splits} plan={p}")
    assert p["path"] == "gemm" and p["splits"] == splits
    assert gemm_issue_mode(fmt, K, splits, tile == 3232) == (tpw, all_)
    c = synth.random_codes_case(tile + K + 31 * splits + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    res = synth.draw_x(np.random.default_rng(K + fmt), M, N) if splits == 1 else None
    check_close(run_gemm(lin, c.x, residual=res), ref_y(c, c.x, residual=res),
                f"issue tile {tile} K {K} splits {splits}")


# 32 x 32 tiles take up to 8 word tiles per wave (two stages in flight), so
# long K runs unsplit; issue-all and own-stage modes, ragged K
@pytest.mark.parametrize("fmt,group,K,tpw,all_", [(0, 128, 8192, 8, True), (0, 128, 6144, 8, False),
                                                  (0, 128, 4224, 8, False), (2, 32, 2048, 2, True),
                                                  (0, 128, 7936, 8, True)])
def test_gemm_long_k_small_tiles(monkeypatch, fmt, group, K, tpw, all_):
    monkeypatch.setenv("QGEMM_GEMM_TILE", "3232")
    monkeypatch.setenv("QGEMM_SPLITK", "1")
    N, M = 200, 40
    p = qgm.plan(M, N, K, group, fmt)
    say(f"long K 32x32 fmt={fmt} g={group} K={K} plan={p}")
    assert p["path"] == "gemm" and p["splits"] == 1 and (p["tile_m"], p["tile_n"]) == (32, 32)
    assert gemm_issue_mode(fmt, K, 1, True) == (tpw, all_)
    c = synth.random_codes_case(K + fmt + group, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    res = synth.draw_x(np.random.default_rng(K), M, N)
    check_close(run_gemm(lin, c.x, residual=res), ref_y(c, c.x, residual=res), f"long K {K}")


# Seeded sweep over random shapes, formats and M: every plan branch the
# shapes reach (GEMV rows, MFMA GEMV chunks, GEMM tiles, word tiles per wave,
# issue modes, splits) against the oracle, half of the cases with a residual.
# QGEMM_TEST_RANDOM_CASES / QGEMM_TEST_RANDOM_SEED widen it for a longer run.
def _random_shape_cases(n=int(os.environ.get("QGEMM_TEST_RANDOM_CASES", "40")),
                        seed=int(os.environ.get("QGEMM_TEST_RANDOM_SEED", "20261203"))):
    rng = np.random.default_rng(seed)
    groups = {0: (32, 64, 128), 1: (32, 64, 128), 2: (32,), 3: (32,), 4: (256,)}
    out = []
    while len(out) < n:
        fmt = int(rng.integers(0, 5))
        g = int(rng.choice(groups[fmt]))
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 9, 16, 17, 31, 33, 64, 65, 100, 128, 129, 200]))
        N = int(rng.integers(1, 700))
        K = g * int(rng.integers(1, max(2, 8192 // g)))
        if M * N * K > 2e8:
            continue
        out.append((fmt, g, M, N, K, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("fmt,group,M,N,K,with_res", _random_shape_cases())
def test_random_shapes(fmt, group, M, N, K, with_res):
    p = qgm.plan(M, N, K, group, fmt)
    say(f"random fmt={fmt} g={group} M={M} N={N} K={K} res={with_res} plan={p}")
    c = synth.random_codes_case(M * 7919 + N * 31 + K + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    res = synth.draw_x(np.random.default_rng(M + N + K), M, N) if with_res else None
    check_close(run_gemm(lin, c.x, residual=res), ref_y(c, c.x, residual=res), "random shape")


def test_gemm_small_tiles_without_split():
    # 128 x 2048 x 2048 (the looped block's O projection): 32 x 32 tiles fill
    # the CUs with no K split where 64 x 64 tiles would split 4 ways
    p = qgm.plan(128, 2048, 2048, 128, 0)
    assert (p["tile_m"], p["tile_n"], p["splits"]) == (32, 32, 1)
    c = synth.random_codes_case(777, 0, 128, 2048, 2048, 128)
    lin = qgm.QuantLinear.from_case(c, DEV)
    check_close(run_gemm(lin, c.x), ref_y(c, c.x), "32x32 no split")


# ----------------------------------------------------------------------------
# q4k: the fp16 weight of the matrix-core paths, bit for bit and against the
# oracle's exact weight
# ----------------------------------------------------------------------------

def q4k_fp16_weight(c):
    """fp16(fp16(d*sc) * q - fp16(dmin*m)) with one rounding of the fused
    multiply-add: the documented dequant of the matrix-core paths, restated
    here in NumPy (fp32 products are exact, fp64 holds the fma exactly)."""
    N, K = c.N, c.K
    ds = c.scales.reshape(N, K // 256, 2).astype(np.float32)
    sc = (c.zeros & 0xFF).astype(np.float32)
    m = (c.zeros >> 8).astype(np.float32)
    sup = np.arange(K // 32) // 8
    dsc = (ds[:, sup, 0] * sc).astype(np.float16).astype(np.float64)
    nb = (-(ds[:, sup, 1] * m)).astype(np.float16).astype(np.float64)
    idx = np.arange(K) // 32
    return (dsc[:, idx] * c.codes.astype(np.float64) + nb[:, idx]).astype(np.float16)


@pytest.mark.parametrize("N,K", [(256, 2048), (40, 512)])
def test_q4k_dequant(N, K):
    say(f"q4k dequant N={N} K={K}")
    c = synth.random_codes_case(N + K, 4, 256, N, K, 1)
    lin = qgm.QuantLinear.from_case(c, DEV)
    got = qgm.dequant(lin.packed, lin.scales, lin.zeros, N, K, 256, 4).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), q4k_fp16_weight(c).view(np.uint16))
    # against the exact weight: one fp16 rounding of the result, of fp16(d*sc)
    # (times q <= 15) and of fp16(dmin*m)
    w = oracle.dequant_f64(c.words, c.scales, c.zeros, N, K, 256, 4)
    s, b = oracle.q4k_subblock_params(c.scales, c.zeros, N, K)
    idx = np.arange(K) // 32
    ulp = lambda v: np.spacing(np.abs(v).astype(np.float16)).astype(np.float64)
    bound = 0.5 * ulp(got) + 0.5 * 15 * ulp(s[:, idx]) + 0.5 * ulp(b[:, idx])
    assert np.all(np.abs(got.astype(np.float64) - w) <= bound * (1 + 1e-9))


@pytest.mark.parametrize("M", [1, 5, 64])
def test_q4k_one_hot_bit_exact(M):
    # x = e_k picks column k: M = 1 (fp32 terms) gives fp16(fp32(w)); the
    # matrix-core paths give the fp16 weight above
    N, K = 144, 512
    say(f"q4k one-hot M={M}")
    c = synth.random_codes_case(M * 5 + 3, 4, 256, N, K, 1)
    ks = np.random.default_rng(M).integers(0, K, size=M)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    y = run_gemm(qgm.QuantLinear.from_case(c, DEV), x)
    if M == 1:
        w = oracle.dequant_f64(c.words, c.scales, c.zeros, N, K, 256, 4)
        expect = w[:, ks].T.astype(np.float32).astype(np.float16)
    else:
        expect = q4k_fp16_weight(c)[:, ks].T
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))


# ----------------------------------------------------------------------------
# exact-arithmetic cases: bit-exact outputs whatever the order
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("M", [1, 5, 24, 64, 130])
@pytest.mark.parametrize("fmt,group", [(0, 32), (0, 128), (1, 64), (2, 32), (3, 32)])
def test_one_hot_bit_exact(M, fmt, group):
    N, K = 144, 512
    say(f"one-hot fmt={fmt} g={group} M={M}")
    c = synth.random_codes_case(M * 3 + fmt + group, fmt, group, N, K, 1)
    rng = np.random.default_rng(M)
    ks = rng.integers(0, K, size=M)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    lin = qgm.QuantLinear.from_case(c, DEV)
    y = run_gemm(lin, x)
    w16 = oracle.dequant_f16(c.words, c.scales, c.zeros, N, K, group, fmt)
    expect = w16[:, ks].T
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("M", [1, 8, 32, 128])
@pytest.mark.parametrize("fmt,group", [(0, 128), (1, 64), (2, 32), (3, 32)])
def test_exact_regime_bit_exact(M, fmt, group):
    # x in {-1, 0, 1}, power-of-two scales, integer zero points: every partial
    # sum is an integer multiple of the smallest scale and exact in fp32
    # (q8_0 at K = 512, so that |y| <= 512 * 128 / 2 stays inside fp16)
    N, K = 256, 512 if fmt == 3 else 2048
    say(f"exact regime fmt={fmt} M={M}")
    rng = np.random.default_rng(fmt * 10 + M)
    b = oracle.BITS[fmt]
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    s = (2.0 ** rng.integers(-4, 0, size=(N, K // group))).astype(np.float16)
    z = None if fmt in (2, 3) else rng.integers(0, 1 << b, size=(N, K // group)).astype(np.float16)
    x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    c = synth.QCase(fmt=fmt, group=group, N=N, K=K, codes=codes, words=synth.pack_words(codes, b),
                    scales=s, zeros=z, x=x)
    lin = qgm.QuantLinear.from_case(c, DEV)
    y = run_gemm(lin, x)
    yr = ref_y(c, x)
    assert np.all(np.abs(yr) < (2048 if b <= 4 else 32768))
    assert np.array_equal(y.astype(np.float64), yr.astype(np.float16).astype(np.float64))


def test_closed_form_zero_codes():
    N, K, group = 128, 1024, 128
    codes = np.zeros((N, K), np.uint8)
    s = np.full((N, K // group), 0.125, np.float16)
    z = np.full((N, K // group), 7.0, np.float16)
    for M in (1, 128):
        x = np.random.default_rng(M).uniform(-1, 1, size=(M, K)).astype(np.float16)
        c = synth.QCase(fmt=0, group=group, N=N, K=K, codes=codes, words=synth.pack_words(codes, 4),
                        scales=s, zeros=z, x=x)
        y = run_gemm(qgm.QuantLinear.from_case(c, DEV), x)
        expect = -0.125 * 7.0 * x.astype(np.float64).sum(axis=1, keepdims=True) * np.ones((1, N))
        check_close(y, expect, f"zero codes M={M}")


@pytest.mark.parametrize("fmt,u,bits", [(2, 8, 4), (3, 128, 8)])
def test_block_format_zero_code_is_zero(fmt, u, bits):
    # q4_0 byte 8 and q8_0 byte 128 are the signed code 0: y is exactly 0
    N, K = 64, 512
    codes = np.full((N, K), u, np.uint8)
    s = np.random.default_rng(0).uniform(0.1, 2, size=(N, K // 32)).astype(np.float16)
    for M in (1, 8, 32):
        x = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
        c = synth.QCase(fmt=fmt, group=32, N=N, K=K, codes=codes, words=synth.pack_words(codes, bits),
                        scales=s, zeros=None, x=x)
        y = run_gemm(qgm.QuantLinear.from_case(c, DEV), x)
        assert np.array_equal(y, np.zeros_like(y))


# ----------------------------------------------------------------------------
# determinism, no stray writes, residual / strides / caller workspace
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name,M", [("prefill_int4_g128", 128), ("decode_int4_g128", 1),
                                    ("int2_g64", 128), ("q4k_s256", 8)])
def test_deterministic(name, M):
    c, lin = get_case(name)
    x = dev_half(c.x[:M])
    a = lin(x).clone()
    b = lin(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("M", [1, 7, 100])
def test_no_writes_outside_output(M):
    N, K, group = 200, 640, 64
    c = synth.random_codes_case(M + 5, 0, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    x = dev_half(c.x)
    big = torch.full((M + 2, 256), float("nan"), dtype=torch.float16, device=DEV)
    out = big[1:M + 1, :N]  # strided view, NaN guard rows and columns around it
    lin(x, out=out)
    torch.cuda.synchronize()
    h = big.cpu().numpy()
    assert np.all(np.isnan(h[0])) and np.all(np.isnan(h[M + 1])) and np.all(np.isnan(h[1:M + 1, N:]))
    check_close(h[1:M + 1, :N], ref_y(c, c.x), "strided out")


@pytest.mark.parametrize("M", [1, 8, 64])
@pytest.mark.parametrize("fmt,group", [(0, 128), (3, 32), (4, 256)])
def test_residual_and_strided_input(M, fmt, group):
    N, K = 256, 1024
    c = synth.random_codes_case(M + 77 + fmt, fmt, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    wide = np.random.default_rng(1).standard_normal((M, K + 64)).astype(np.float16)
    wide[:, 32:32 + K] = c.x
    xw = dev_half(wide)
    x_view = xw[:, 32:32 + K]
    res = np.random.default_rng(2).standard_normal((M, N)).astype(np.float16)
    y = lin(x_view, residual=dev_half(res))
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), ref_y(c, c.x, residual=res), "residual+strided")


def test_caller_workspace():
    M, N, K, group = 128, 1024, 2048, 128
    c = synth.random_codes_case(5, 0, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    nbytes = qgm.workspace_bytes(M, N, K, group, 0)
    assert nbytes > 0
    ws = torch.zeros(nbytes // 4 + 64, dtype=torch.int32, device=DEV)
    x = dev_half(c.x)
    y1 = lin(x, workspace=ws).clone()
    y2 = lin(x, workspace=ws).clone()   # counters were left at zero
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    check_close(y1.cpu().numpy(), ref_y(c, c.x), "caller workspace")
    with pytest.raises(qgm.QGemmError):
        lin(x, workspace=torch.zeros(4, dtype=torch.int32, device=DEV))


def test_plain_entry_point_and_empty():
    c, lin = get_case("tiny_int4_g32")
    x = dev_half(c.x)
    y = torch.empty((4, c.N), dtype=torch.float16, device=DEV)
    qgm.qgemm_plain(x, lin.packed, lin.scales, lin.zeros, c.N, c.K, c.group, c.fmt, y)
    torch.cuda.synchronize()
    check_close(y.cpu().numpy(), ref_y(c, c.x), "plain qgemm")
    empty = lin(torch.empty((0, c.K), dtype=torch.float16, device=DEV))
    assert empty.shape == (0, c.N)


def test_binding_rejects_mismatched_tensors():
    # the binding checks what the C ABI cannot see (tensor sizes, dtypes,
    # devices) before any launch
    c, lin = get_case("tiny_int4_g32")
    x = dev_half(c.x)
    M, N, K = x.shape[0], c.N, c.K
    bad_out = [torch.empty((M - 1, N), dtype=torch.float16, device=DEV),       # too few rows
               torch.empty((M, N), dtype=torch.float32, device=DEV),           # wrong dtype
               torch.empty((N, M), dtype=torch.float16, device=DEV).t()]       # column stride != 1
    for out in bad_out:
        with pytest.raises(ValueError):
            lin(x, out=out)
    with pytest.raises(ValueError):
        lin(x, residual=torch.zeros((M, N - 1), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):   # packed codes too short for [N, K]
        qgm.qgemm(x, lin.packed[:-1], lin.scales, lin.zeros, N, K, c.group, c.fmt)
    with pytest.raises(ValueError):   # scales for a smaller N
        qgm.qgemm(x, lin.packed, lin.scales[:-1], lin.zeros, N, K, c.group, c.fmt)
    with pytest.raises(ValueError):   # fp16 zero points given as int16 bits
        qgm.qgemm(x, lin.packed, lin.scales, lin.zeros.view(torch.int16), N, K, c.group, c.fmt)
    with pytest.raises(ValueError):
        qgm.dequant(lin.packed[:10], lin.scales, lin.zeros, N, K, c.group, c.fmt)
    # x with a column stride other than 1 is refused for every M, M = 1 included
    wide = dev_half(np.zeros((4, 2 * K), np.float16))
    for xs in (wide[:1, ::2], wide[:, ::2], torch.zeros((K, 1), dtype=torch.float16, device=DEV).t()[:, :]):
        if xs.stride(1) == 1:
            continue
        with pytest.raises(ValueError):
            lin(xs)
    # the looped block checks its four shapes and the scratch size
    D, F = 64, 128
    cases = [synth.random_codes_case(70 + i, 0, 32, n, k, 1)
             for i, (n, k) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    lins = [qgm.QuantLinear.from_case(cc, DEV) for cc in cases]
    xl = dev_half(np.zeros((4, D), np.float16))
    with pytest.raises(ValueError):
        qgm.loop_block(xl, [lins[0], lins[1], lins[3], lins[2]], 1)   # up and down swapped
    with pytest.raises(ValueError):
        qgm.loop_block(xl, lins, 1, scratch=torch.empty(10, dtype=torch.float16, device=DEV))
    qgm.loop_block(xl, lins, 1)   # the right shapes run
    torch.cuda.synchronize()


def test_loop_block_bad_down_projection_launches_nothing():
    # F % group != 0 makes only the down projection invalid; the C ABI checks
    # all four linears before launching, so x and the scratch stay untouched
    import ctypes
    D, F, g = 64, 96, 64
    lins = []
    for i, (n, k) in enumerate(((3 * D, D), (D, D), (F, D), (D, F))):
        cc = synth.random_codes_case(90 + i, 0, 32, n, k, 1)
        lins.append(qgm.QuantLinear.from_case(cc, DEV))
    x = dev_half(np.random.default_rng(5).standard_normal((4, D)).astype(np.float16))
    x0 = x.clone()
    scratch = torch.full((4 * (3 * D + D + F),), 7.0, dtype=torch.float16, device=DEV)
    arr = lambda vals: (ctypes.c_void_p * 4)(*vals)
    st = qgm._lib.qloop_block(x.data_ptr(), arr([l.packed.data_ptr() for l in lins]),
                              arr([l.scales.data_ptr() for l in lins]),
                              arr([l.zeros.data_ptr() for l in lins]), 4, D, F, g, 0, 2,
                              scratch.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 1   # QG_E_ARG
    assert torch.equal(x, x0)
    assert bool((scratch == 7.0).all())


def test_k_zero_writes_zeros():
    packed = torch.zeros(64, dtype=torch.int32, device=DEV)
    s = torch.ones((16, 1), dtype=torch.float16, device=DEV)
    x = torch.empty((3, 0), dtype=torch.float16, device=DEV)
    y = torch.full((3, 16), 5.0, dtype=torch.float16, device=DEV)
    qgm.qgemm(x, packed, s, s, 16, 0, 32, 0, out=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("name,M", [("decode_int4_g128", 1), ("prefill_int4_g128", 128), ("int2_g64", 8),
                                    ("q8_0_b32", 1), ("q4k_s256", 1), ("q4k_s256", 128)])
def test_graph_replays_match_eager(name, M):
    # the benchmark captures calls in a HIP graph: every replay, with eager
    # work and synchronisation in between, must equal the eager result
    c, lin = get_case(name)
    x = dev_half(c.x[:M])
    eager = lin(x).clone()
    torch.cuda.synchronize()
    y = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lin(x, out=y)
        lin(x, out=y)
    for rep in range(4):
        y.fill_(float("nan"))
        other = lin(x)            # eager call between replays (same workspace)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(other.view(torch.int16), eager.view(torch.int16))


def test_graph_survives_workspace_growth(monkeypatch):
    # a graph captured with the library-owned split-K workspace must still
    # replay correctly after a later, larger call has grown that workspace
    # (the outgrown buffer is kept, never freed)
    ca = synth.random_codes_case(5150, 0, 128, 512, 2048, 32)     # 32 x 32 tiles, 16-way split
    assert qgm.workspace_bytes(32, 512, 2048, 128, 0) > 0
    la = qgm.QuantLinear.from_case(ca, DEV)
    xa = dev_half(ca.x)
    eager = la(xa).clone()
    torch.cuda.synchronize()
    ya = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        la(xa, out=ya)
    # 128 tiles x 8 forced splits of 64 x 64 fp32 partials: 16 MiB, more than
    # any earlier call in this process asked for, so the workspace grows
    Mb, Nb, Kb = 256, 2048, 16384
    monkeypatch.setenv("QGEMM_SPLITK", "8")
    assert qgm.workspace_bytes(Mb, Nb, Kb, 128, 0) >= 16 << 20
    cb = synth.random_codes_case(5151, 0, 128, Nb, Kb, 1)
    lb = qgm.QuantLinear.from_case(cb, DEV)
    xb = torch.randn((Mb, Kb), device=DEV).to(torch.float16)
    yb0 = lb(xb).clone()
    torch.cuda.synchronize()
    say(f"workspace growth: graph plan {qgm.plan(32, 512, 2048, 128, 0)}, big plan {qgm.plan(Mb, Nb, Kb, 128, 0)}")
    for rep in range(3):
        ya.fill_(float("nan"))
        g.replay()
        yb = lb(xb)               # eager call on the grown workspace between replays
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(yb.view(torch.int16), yb0.view(torch.int16))


# ----------------------------------------------------------------------------
# looped shared block: qloop_block against the oracle's chain
# ----------------------------------------------------------------------------

def _loop_lin_dicts(cases):
    return [dict(words=c.words, scales=c.scales, zeros=c.zeros, N=c.N, K=c.K, group=c.group, fmt=c.fmt)
            for c in cases]


@pytest.mark.parametrize("fmt,group,M", [(0, 128, 1), (0, 128, 8), (0, 128, 40), (1, 64, 1), (2, 32, 40),
                                         (3, 32, 8), (4, 256, 40), (4, 256, 1)])
def test_loop_block_parity(fmt, group, M):
    D, F, L = 256, 512, 3
    say(f"loop fmt={fmt} g={group} M={M} D={D} F={F} L={L}")
    cases = [synth.random_case(4000 + 10 * fmt + i, fmt, group, N, K, 1)
             for i, (N, K) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    x0 = synth.draw_x(np.random.default_rng(4100 + M), M, D)
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in cases]
    x = dev_half(x0)
    qgm.loop_block(x, lins, L)
    torch.cuda.synchronize()
    ref = oracle.loop_block_ref(x0, _loop_lin_dicts(cases), L, D=D)
    check_close(x.cpu().numpy(), ref[-1], f"loop x_{L}")


@pytest.mark.parametrize("M", [1, 8, 40])
def test_loop_block_exact_chain(M):
    # exact weights (see tests/pins.exact_loop_linears): every loop is x -> 4x
    D, L = 64, 3
    x0 = (np.random.default_rng(M).integers(-8, 9, size=(M, D)) / 8.0).astype(np.float16)
    lins = [qgm.QuantLinear(l["words"], l["scales"], l["zeros"], l["N"], l["K"], l["group"], l["fmt"], DEV)
            for l in pins.exact_loop_linears(D)]
    x = dev_half(x0)
    qgm.loop_block(x, lins, L)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy().astype(np.float64), x0.astype(np.float64) * 4.0 ** L)


@pytest.mark.parametrize("M", [1, 128])
def test_loop_block_full_size(M):
    # the benchmark's block: D = 2048, F = 8192, INT4 g128, all 8 loops; M = 128
    # runs the GEMM path, M = 1 (decode) the GEMV kernels with fused residuals
    lc = synth.loop_workload(M=M, L=8)
    say(f"loop full size M={M} D=2048 F=8192 L=8")
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in lc.linears()]
    x = dev_half(lc.x0)
    qgm.loop_block(x, lins, lc.L)
    torch.cuda.synchronize()
    ref = oracle.loop_block_ref(lc.x0, _loop_lin_dicts(lc.linears()), lc.L)
    check_close(x.cpu().numpy(), ref[-1], "loop x_8 full size")


@pytest.mark.parametrize("M", [1, 128])
def test_loop_block_graph_replays_match_eager(M):
    # the benchmark times the looped block as loops captured in a HIP graph:
    # every replay (x reset outside the graph, eager work in between) must give
    # the eager block's bits
    D, F, L = 256, 512, 3
    say(f"loop graph replay M={M} D={D} F={F} L={L}")
    cases = [synth.random_case(4200 + i, 0, 128, N, K, 1)
             for i, (N, K) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in cases]
    x0 = dev_half(synth.draw_x(np.random.default_rng(4300 + M), M, D))
    scratch = torch.empty(M * (3 * D + D + F), dtype=torch.float16, device=DEV)
    x = x0.clone()
    qgm.loop_block(x, lins, L, scratch=scratch)
    torch.cuda.synchronize()
    eager = x.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qgm.loop_block(x, lins, L, scratch=scratch)
    for rep in range(4):
        x.copy_(x0)
        other = x0.clone()
        qgm.loop_block(other, lins, 1)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_dequant_into_caller_buffer_feeds_an_fp16_gemm():
    # the dequantize-at-load comparison path: qg_dequant into a caller-owned
    # fp16 [N, K] buffer (same bits as `dequant`), then a plain fp32 product
    N, K, group, M = 200, 640, 64, 16
    say("dequant_into + fp16 product")
    c = synth.random_case(4242, 0, group, N, K, M)
    lin = qgm.QuantLinear.from_case(c, DEV)
    w = torch.full((N, K), float("nan"), dtype=torch.float16, device=DEV)
    qgm.dequant_into(lin.packed, lin.scales, lin.zeros, N, K, group, 0, w)
    ref_w = qgm.dequant(lin.packed, lin.scales, lin.zeros, N, K, group, 0)
    assert torch.equal(w.view(torch.int16), ref_w.view(torch.int16))
    y = (torch.from_numpy(c.x.astype(np.float32)) @ w.cpu().float().t()).numpy()
    check_close(y, ref_y(c, c.x), "dequant then product")
    with pytest.raises(ValueError):
        qgm.dequant_into(lin.packed, lin.scales, lin.zeros, N, K, group, 0, w[:, :K - 8])
