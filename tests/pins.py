"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes the oracle module ``O`` and raises AssertionError (or any
exception) when the oracle disagrees with a hand-worked value, a closed form,
exact rational arithmetic or a literal-loop brute force.  The pins are run on
the real oracle (all must pass) and on planted mistakes (each must be caught).
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FMT = {"int4": 0, "int2": 1, "q4_0": 2, "q8_0": 3}
BITS = {0: 4, 1: 2, 2: 4, 3: 8, 4: 4}
Q4K = 4
# implicit zero points of the block formats: q4_0 stores q + 8, q8_0 q + 128
ZIMPL = {2: 8, 3: 128}


# -- independent helpers (no oracle code) ------------------------------------

def pack_literal(codes, bits):
    """Literal bit loop: canonical LSB-first packing, one code at a time."""
    codes = [[int(c) for c in row] for row in np.asarray(codes)]
    cpw = 32 // bits
    out = []
    for row in codes:
        words = []
        for w0 in range(0, len(row), cpw):
            v = 0
            for j in range(cpw):
                v |= (row[w0 + j] & ((1 << bits) - 1)) << (bits * j)
            words.append(v)
        out.append(words)
    return np.array(out, dtype=np.uint32)


def half_rne(v: float) -> float:
    """Round a double to fp16, nearest-even, via the struct 'e' codec."""
    return struct.unpack("<e", struct.pack("<e", v))[0]


def brute_y(x, codes, scales, zeros, group, fmt):
    """Literal triple loop over unpacked integer codes, Python floats (fp64)."""
    x = np.asarray(x, dtype=np.float16).astype(float)
    M, K = x.shape
    N = len(codes)
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                g = k // group
                s = float(scales[n][g])
                z = float(ZIMPL[fmt]) if fmt in ZIMPL else float(zeros[n][g])
                acc += float(x[m][k]) * (s * (float(codes[n][k]) - z))
            y[m][n] = acc
    return np.array(y)


def exact_y(x, codes, scales, zeros, group, fmt):
    """Exact rational result."""
    x = np.asarray(x, dtype=np.float16)
    M, K = x.shape
    N = len(codes)
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // group
                s = Fraction(float(np.float16(scales[n][g])))
                z = Fraction(ZIMPL[fmt]) if fmt in ZIMPL else Fraction(float(np.float16(zeros[n][g])))
                acc += Fraction(float(x[m][k])) * s * (int(codes[n][k]) - z)
            row.append(acc)
        out.append(row)
    return out


def _rand_inputs(seed, fmt, N, K, M, group):
    rng = np.random.default_rng(seed)
    b = BITS[fmt]
    codes = rng.integers(0, 1 << b, size=(N, K), dtype=np.uint8)
    s = (rng.uniform(0.01, 0.2, size=(N, K // group))).astype(np.float16)
    z = None if fmt in ZIMPL else rng.integers(0, 1 << b, size=(N, K // group)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    return codes, s, z, x


def q4k_meta(d, dmin, sc, m):
    """Metadata arrays of one q4k row set: scales fp16 [N, S, 2], zeros uint16
    [N, 8S] with sc in the low byte and m in the high byte."""
    d, dmin = np.asarray(d, np.float16), np.asarray(dmin, np.float16)
    scales = np.stack([d, dmin], axis=-1)
    zeros = (np.asarray(sc, np.uint16) | (np.asarray(m, np.uint16) << 8)).astype(np.uint16)
    return scales, zeros


def brute_y_q4k(x, codes, d, dmin, sc, m):
    """Literal loops: w = d[S] * sc[j] * q - dmin[S] * m[j], S = k // 256, j = k // 32."""
    x = np.asarray(x, dtype=np.float16).astype(float)
    M, K = x.shape
    N = len(codes)
    y = np.zeros((M, N))
    for mm in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                S, j = k // 256, k // 32
                w = float(d[n][S]) * int(sc[n][j]) * int(codes[n][k]) - float(dmin[n][S]) * int(m[n][j])
                acc += float(x[mm][k]) * w
            y[mm, n] = acc
    return y


def exact_w_q4k(codes, d, dmin, sc, m, n, k):
    S, j = k // 256, k // 32
    return (Fraction(float(d[n][S])) * int(sc[n][j]) * int(codes[n][k])
            - Fraction(float(dmin[n][S])) * int(m[n][j]))


def _rand_q4k(seed, N, K, M):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    d = rng.uniform(1e-4, 2e-3, size=(N, K // 256)).astype(np.float16)
    dmin = rng.uniform(1e-4, 2e-3, size=(N, K // 256)).astype(np.float16)
    sc = rng.integers(0, 64, size=(N, K // 32))
    m = rng.integers(0, 64, size=(N, K // 32))
    x = rng.standard_normal((M, K)).astype(np.float16)
    return codes, d, dmin, sc, m, x


# -- pins ---------------------------------------------------------------------

def pin_worked_words(O):
    for line in open(os.path.join(GOLDEN, "canonical_words.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt_s, codes_s, word_s = line.split()
        fmt = FMT[fmt_s]
        codes = np.array([[int(c) for c in codes_s.split(",")]], dtype=np.uint8)
        word = int(word_s, 16)
        got = O.pack_codes(codes, fmt)
        assert got.shape == (1, 1) and int(got[0, 0]) == word, (line, hex(int(got[0, 0])))
        back = O.unpack_codes(np.array([[word]], dtype=np.uint32), 1, codes.shape[1], fmt)
        assert np.array_equal(back, codes), line


def pin_handcases(O):
    for line in open(os.path.join(GOLDEN, "handcases.jsonl")):
        c = json.loads(line)
        if "name" not in c:
            continue
        fmt = FMT[c["fmt"]]
        K, g = c["K"], c["group"]
        rule = c["codes"]
        def code(k):
            if rule == "k%16":
                return k % 16
            if rule == "k%4":
                return k % 4
            if rule == "8k":
                return 8 * k
            if rule == "0/255":
                return 255 * (k % 2)
            return rule
        codes = np.array([[code(k) for k in range(K)]], dtype=np.uint8)
        x = np.array([[1.0 if c["x"] == "ones" else (-1.0) ** k for k in range(K)]], dtype=np.float16)
        s = np.array([c["scales"]], dtype=np.float16)
        z = None if c["zeros"] is None else np.array([c["zeros"]], dtype=np.float16)
        words = pack_literal(codes, BITS[fmt])
        y = O.qgemm_ref(x, words, s, z, 1, 1, K, g, fmt)
        assert float(y[0, 0]) == c["y"], (c["name"], float(y[0, 0]), c["y"])


def pin_zero_codes_closed_form(O):
    # all-zero codes: y[m,n] = -sum_g s[n,g] z[n,g] sum_{k in g} x[m,k]
    for fmt, group in ((0, 32), (0, 128), (1, 64)):
        N, K, M = 8, 256, 3
        _, s, z, x = _rand_inputs(7 + fmt + group, fmt, N, K, M, group)
        codes = np.zeros((N, K), dtype=np.uint8)
        y = O.qgemm_ref(x, pack_literal(codes, BITS[fmt]), s, z, M, N, K, group, fmt)
        xs = x.astype(float)
        for m in range(M):
            for n in range(N):
                exp = Fraction(0)
                for gi in range(K // group):
                    sx = sum(Fraction(float(v)) for v in xs[m, gi * group:(gi + 1) * group])
                    exp -= Fraction(float(s[n, gi])) * Fraction(float(z[n, gi])) * sx
                assert abs(float(y[m, n]) - float(exp)) <= 1e-12 * max(1.0, abs(float(exp))), (fmt, m, n)
    # uniform s, z: -s * z * sum(x)
    N, K = 4, 128
    x = np.random.default_rng(3).standard_normal((2, K)).astype(np.float16)
    s = np.full((N, K // 32), 0.125, dtype=np.float16)
    z = np.full((N, K // 32), 5.0, dtype=np.float16)
    y = O.qgemm_ref(x, np.zeros((N, K // 8), dtype=np.uint32), s, z, 2, N, K, 32, 0)
    for m in range(2):
        exp = -0.125 * 5.0 * sum(float(v) for v in x[m].astype(float))
        assert np.allclose(y[m], exp, rtol=1e-12, atol=1e-12)


def pin_one_hot(O):
    # x = e_k selects column k of the dequantized matrix: y[m, n] = s(q[n,k] - z)
    for fmt, group in ((0, 32), (0, 128), (1, 32), (1, 64), (2, 32), (3, 32)):
        N, K = 24, 256     # N != K: a transposed operand cannot pass
        codes, s, z, _ = _rand_inputs(11 + fmt * 10 + group, fmt, N, K, 1, group)
        ks = [0, 1, 7, 8, 31, 32, 33, 100, 127, 128, 200, 255]
        x = np.zeros((len(ks), K), dtype=np.float16)
        for i, k in enumerate(ks):
            x[i, k] = 1.0
        y = O.qgemm_ref(x, pack_literal(codes, BITS[fmt]), s, z, len(ks), N, K, group, fmt)
        for i, k in enumerate(ks):
            for n in range(N):
                zz = float(ZIMPL[fmt]) if fmt in ZIMPL else float(z[n, k // group])
                exp = float(s[n, k // group]) * (int(codes[n, k]) - zz)
                assert float(y[i, n]) == exp, (fmt, group, k, n, float(y[i, n]), exp)


def pin_format_identity(O):
    # q4_0 (u, s) equals INT4-asym with every zero point 8 and group 32
    N, K, M = 16, 128, 3
    codes, s, _, x = _rand_inputs(5, 2, N, K, M, 32)
    words = pack_literal(codes, 4)
    a = O.qgemm_ref(x, words, s, None, M, N, K, 32, 2)
    b = O.qgemm_ref(x, words, s, np.full(s.shape, 8.0, dtype=np.float16), M, N, K, 32, 0)
    assert np.array_equal(a, b)
    uz = pack_literal(np.full((N, K), 8, dtype=np.uint8), 4)
    assert np.array_equal(O.qgemm_ref(x, uz, s, None, M, N, K, 32, 2), np.zeros((M, N)))
    # q8_0 whose bytes are 120 + c for 4-bit c is q4_0 on the nibbles c
    # (both decode to s * (c - 8)): one identity across the two block formats
    u8 = codes.astype(np.uint8) + 120
    c8 = O.qgemm_ref(x, pack_literal(u8, 8), s, None, M, N, K, 32, 3)
    assert np.array_equal(a, c8)
    u128 = pack_literal(np.full((N, K), 128, dtype=np.uint8), 8)
    assert np.array_equal(O.qgemm_ref(x, u128, s, None, M, N, K, 32, 3), np.zeros((M, N)))


def pin_bruteforce(O):
    for fmt, group, N, K, M in ((0, 32, 8, 64, 3), (0, 64, 16, 128, 2), (1, 32, 8, 64, 3),
                                (1, 64, 16, 128, 1), (2, 32, 8, 64, 3), (2, 32, 16, 32, 2),
                                (3, 32, 8, 64, 3), (3, 32, 16, 96, 2)):
        codes, s, z, x = _rand_inputs(100 + N + K + fmt, fmt, N, K, M, group)
        y = O.qgemm_ref(x, pack_literal(codes, BITS[fmt]), s, z, M, N, K, group, fmt)
        yb = brute_y(x, codes, s, z, group, fmt)
        assert y.shape == (M, N)
        assert np.max(np.abs(y - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb))), (fmt, group, N, K, M)


def pin_exact_rational(O):
    for fmt, group in ((0, 32), (1, 64), (2, 32), (3, 32)):
        N, K, M = 6, 64, 2
        codes, s, z, x = _rand_inputs(300 + fmt, fmt, N, K, M, group)
        y = O.qgemm_ref(x, pack_literal(codes, BITS[fmt]), s, z, M, N, K, group, fmt)
        ex = exact_y(x, codes, s, z, group, fmt)
        for m in range(M):
            for n in range(N):
                e = float(ex[m][n])
                assert abs(float(y[m, n]) - e) <= 1e-13 * max(1.0, abs(e)), (fmt, m, n)


def pin_dequant_exact(O):
    # the fp32 dequantized weight is exact, and its fp16 rounding is nearest-even
    for fmt, group in ((0, 32), (1, 64), (2, 32), (3, 32)):
        N, K = 8, 128
        codes, s, z, _ = _rand_inputs(400 + fmt, fmt, N, K, 1, group)
        words = pack_literal(codes, BITS[fmt])
        w32 = O.dequant_f32(words, s, z, N, K, group, fmt)
        w16 = O.dequant_f16(words, s, z, N, K, group, fmt)
        assert w32.dtype == np.float32 and w16.dtype == np.float16
        for n in range(N):
            for k in range(K):
                zz = Fraction(ZIMPL[fmt]) if fmt in ZIMPL else Fraction(float(z[n, k // group]))
                e = Fraction(float(s[n, k // group])) * (int(codes[n, k]) - zz)
                assert Fraction(float(w32[n, k])) == e, (fmt, n, k)
                assert float(w16[n, k]) == half_rne(float(e)), (fmt, n, k)


def pin_fold_identity(O):
    N, K, M, group = 16, 256, 3, 64
    codes, s, z, x = _rand_inputs(500, 0, N, K, M, group)
    words = pack_literal(codes, 4)
    sym, corr = O.fold_zero_point_ref(x, words, s, z, M, N, K, group)
    y = O.qgemm_ref(x, words, s, z, M, N, K, group, 0)
    yb = brute_y(x, codes, s, z, group, 0)
    assert np.max(np.abs((sym - corr) - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb)))
    assert np.max(np.abs(y - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb)))


def pin_q4k_handcases(O):
    for line in open(os.path.join(GOLDEN, "q4k_handcases.jsonl")):
        c = json.loads(line)
        if "name" not in c:
            continue
        K, rule = c["K"], c["codes"]
        codes = np.array([[(k % 16 if rule == "k%16" else rule) for k in range(K)]], dtype=np.uint8)
        x = np.array([[1.0 if c["x"] == "ones" else (-1.0) ** k for k in range(K)]], dtype=np.float16)
        scales, zeros = q4k_meta([c["d"]], [c["dmin"]], [c["sc"]], [c["m"]])
        y = O.qgemm_ref(x, pack_literal(codes, 4), scales, zeros, 1, 1, K, 256, Q4K)
        assert float(y[0, 0]) == c["y"], (c["name"], float(y[0, 0]), c["y"])


def pin_q4k_bruteforce_and_exact(O):
    for N, K, M in ((5, 256, 3), (3, 768, 2)):
        codes, d, dmin, sc, m, x = _rand_q4k(600 + K, N, K, M)
        scales, zeros = q4k_meta(d, dmin, sc, m)
        words = pack_literal(codes, 4)
        y = O.qgemm_ref(x, words, scales, zeros, M, N, K, 256, Q4K)
        yb = brute_y_q4k(x, codes, d, dmin, sc, m)
        assert y.shape == (M, N)
        assert np.max(np.abs(y - yb)) <= 1e-12 * max(1.0, np.max(np.abs(yb))), (N, K, M)
        w16 = O.dequant_f16(words, scales, zeros, N, K, 256, Q4K)
        for n in range(N):
            for k in range(0, K, 7):
                e = exact_w_q4k(codes, d, dmin, sc, m, n, k)
                assert float(w16[n, k]) == half_rne(float(e)), (n, k)
        for mm in range(M):
            for n in range(N):
                ex = sum(Fraction(float(x[mm, k])) * exact_w_q4k(codes, d, dmin, sc, m, n, k) for k in range(K))
                assert abs(float(y[mm, n]) - float(ex)) <= 1e-13 * max(1.0, abs(float(ex))), (mm, n)


def pin_q4k_one_hot_and_zero_codes(O):
    N, K = 24, 512       # N != K
    codes, d, dmin, sc, m, _ = _rand_q4k(700, N, K, 1)
    scales, zeros = q4k_meta(d, dmin, sc, m)
    ks = [0, 1, 31, 32, 255, 256, 300, 511]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = O.qgemm_ref(x, pack_literal(codes, 4), scales, zeros, len(ks), N, K, 256, Q4K)
    for i, k in enumerate(ks):
        for n in range(N):
            assert Fraction(float(y[i, n])) == exact_w_q4k(codes, d, dmin, sc, m, n, k), (k, n)
    # all codes 0: y = -sum_j dmin[S] m[j] sum_{k in j} x
    xr = np.random.default_rng(5).standard_normal((2, K)).astype(np.float16)
    y0 = O.qgemm_ref(xr, np.zeros((N, K // 8), np.uint32), scales, zeros, 2, N, K, 256, Q4K)
    for mm in range(2):
        for n in range(N):
            ex = Fraction(0)
            for j in range(K // 32):
                sx = sum(Fraction(float(v)) for v in xr[mm, 32 * j:32 * j + 32])
                ex -= Fraction(float(dmin[n, j // 8])) * int(m[n, j]) * sx
            assert abs(float(y0[mm, n]) - float(ex)) <= 1e-12 * max(1.0, abs(float(ex))), (mm, n)


def pin_q4k_matches_int4_g32(O):
    # d a power of two, m = sc * z with integer z: w = d sc (q - z), i.e. INT4
    # with group 32, scale d * sc (exact in fp16) and zero point z
    rng = np.random.default_rng(800)
    N, K, M = 8, 512, 3
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    sc = rng.integers(1, 5, size=(N, K // 32))
    z = np.array([[rng.integers(0, min(15, 63 // int(v)) + 1) for v in row] for row in sc])
    d = (2.0 ** rng.integers(-10, -4, size=(N, K // 256))).astype(np.float16)
    scales, zeros = q4k_meta(d, d, sc, sc * z)
    x = rng.standard_normal((M, K)).astype(np.float16)
    words = pack_literal(codes, 4)
    a = O.qgemm_ref(x, words, scales, zeros, M, N, K, 256, Q4K)
    s32 = (d.astype(np.float64)[:, np.arange(K // 32) // 8] * sc).astype(np.float16)
    b = O.qgemm_ref(x, words, s32, z.astype(np.float16), M, N, K, 32, 0)
    assert np.array_equal(a, b)


def exact_loop_linears(D):
    """INT4 g32 weights with s = 1, z = 1, so w = q - 1 in {-1, 0, 1} exactly:
    QKV = [0; -I; +I] (Q zero, K = -x, V = x), O = I, up = [I; -I] (F = 2D),
    down = [I, 0].  One loop maps x to h = x + V = 2x and then to
    h + down(up(h)) = 2h = 4x; any other slice of QKV, a missing residual or a
    transposed operand gives something else."""
    I = np.eye(D, dtype=np.int64)
    Z = np.zeros((D, D), dtype=np.int64)
    mats = [np.vstack([Z, -I, I]), I, np.vstack([I, -I]), np.hstack([I, Z])]
    lins = []
    for w in mats:
        N, K = w.shape
        codes = (w + 1).astype(np.uint8)
        lins.append(dict(words=pack_literal(codes, 4), scales=np.ones((N, K // 32), np.float16),
                         zeros=np.ones((N, K // 32), np.float16), N=N, K=K, group=32, fmt=0))
    return lins


def pin_loop_block_closed_form(O):
    D, M, L = 64, 3, 3
    x0 = (np.random.default_rng(9).integers(-8, 9, size=(M, D)) / 8.0).astype(np.float16)
    outs = O.loop_block_ref(x0, exact_loop_linears(D), L, D=D)
    assert len(outs) == L
    for l, xl in enumerate(outs):
        assert xl.dtype == np.float16 and xl.shape == (M, D)
        assert np.array_equal(xl.astype(np.float64), x0.astype(np.float64) * 4.0 ** (l + 1)), l


def pin_tolerance_rule(O):
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    tol = O.TOLERANCE
    assert tol == 2e-3
    ok = ref.copy()
    ok[0, 0] += 0.999 * tol * 4.0
    assert O.within_tolerance(ok, ref)
    bad = ref.copy()
    bad[1, 1] -= 1.01 * tol * 4.0
    assert not O.within_tolerance(bad, ref)
    nan = ref.copy()
    nan[0, 1] = np.nan
    assert not O.within_tolerance(nan, ref)
    assert O.rel_error(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


ALL_PINS = [pin_worked_words, pin_handcases, pin_zero_codes_closed_form, pin_one_hot,
            pin_format_identity, pin_bruteforce, pin_exact_rational, pin_dequant_exact,
            pin_fold_identity, pin_tolerance_rule, pin_q4k_handcases, pin_q4k_bruteforce_and_exact,
            pin_q4k_one_hot_and_zero_codes, pin_q4k_matches_int4_g32, pin_loop_block_closed_form]


def failing_pins(O):
    bad = []
    for p in ALL_PINS:
        try:
            p(O)
        except Exception:
            bad.append(p.__name__)
    return bad
