"""Plain, slow, obviously-correct CPU oracle (NumPy) for y = x . dequant(W)^T.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Nothing here is used by the library.

What is computed, and where it comes from:

* The operation itself is the "dequantizing matmul" of the skyzh/tiny-llm
  feature list (items "Dequantizing Runtimes", "Quantized Matrix
  Multiplication" and "Dequantization Matrix Multiplications"): low-bit
  weights are turned back into full-precision values and then multiplied.
  Written out:  y[m, n] = sum_k x[m, k] * w[n, k]  with
  w[n, k] = s[n, k // g] * (q[n, k] - z[n, k // g]).
* The weight formats are the INT4 group weights with GPTQ zero points and the
  INT2 body weights of the TinyLoop README (sections "Status" and "Current
  Runtime Snapshot") and q4_0 and q8_0 from the torchnative guide "Inference
  with real transformers" (section "Quantise while loading").  The pages give
  names, not layouts; the readings used are:
    - canonical words hold cpw = 32 / b codes, least significant bits first
      along K (code k of a row lives in word k // cpw at bit b * (k % cpw));
    - q4_0 stores u = q + 8 in a nibble, so w = s * (u - 8): the same formula
      with an implicit zero point of 8 and group 32;
    - q8_0 stores u = q + 128 in a byte (signed 8-bit codes, offset binary),
      so w = s * (u - 128): implicit zero point 128, group 32.  The guide says
      this format loses nothing when the operands are integers; read here as:
      a weight that already is a block scale times an integer in [-127, 127]
      comes back exactly, and every code and every s * q is exact in fp32;
    - q4k, the k-quant of the same guide, is only named there, with the
      remark that layer widths must be multiples of 256.  Read as the
      published k-quant scheme: super-blocks of 256 weights along K, each with
      fp16 factors d and dmin, split into 8 sub-blocks of 32 whose 6-bit
      integers sc and m (0..63) give the sub-block scale d * sc and the
      sub-block offset dmin * m; 4-bit codes q in 0..15 (canonical INT4
      words), w = d * sc * q - dmin * m.  The metadata layout is this
      library's own: scales fp16 [N, K/256, 2] holding (d, dmin), zeros
      uint16 [N, K/32] holding sc in the low byte and m in the high byte;
      the group argument is the super-block, 256;
    - zero points are fp16 values holding integers in [0, 2^b - 1].
* Precision: the dequantized weight is formed in fp32, which is exact (an
  11-bit fp16 significand times an integer of at most 8 bits needs at most 19
  significant bits); the product is taken in fp64.  A q4k weight is the
  difference of two such exact products (d * sc * q has at most 21
  significant bits), formed in fp64, where it is exact whenever d and dmin
  are within a factor 2^31 of each other; its fp32 copy is rounded once.  The torchnative guide
  (section "float32 or bfloat16") notes that a change of accumulation order
  alone changes low-precision results, so parity is judged by a tolerance on
  y, and bit-exactly only on integer codes.

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, hand-worked values (tests/golden/), exact rational arithmetic and a
literal-loop brute force.  No function is left "parity unpinned".
"""
from __future__ import annotations

import numpy as np

INT4_ASYM = 0
INT2_ASYM = 1
Q4_0 = 2
Q8_0 = 3
Q4K = 4
BITS = {INT4_ASYM: 4, INT2_ASYM: 2, Q4_0: 4, Q8_0: 8, Q4K: 4}
Q4K_SUPER = 256   # weights per q4k super-block (one (d, dmin) pair)
Q4K_SUB = 32      # weights per q4k sub-block (one (sc, m) pair)
# implicit zero points of the symmetric block formats (offset-binary codes)
IMPLICIT_ZERO = {Q4_0: 8.0, Q8_0: 128.0}

# max |y - y_ref| <= TOLERANCE * max |y_ref| over one call's output
TOLERANCE = 2e-3


def _cpw(fmt: int) -> int:
    return 32 // BITS[fmt]


def unpack_codes(words: np.ndarray, N: int, K: int, fmt: int) -> np.ndarray:
    """Canonical words uint32 [N, K/cpw] -> integer codes uint8 [N, K]."""
    b = BITS[fmt]
    cpw = _cpw(fmt)
    words = np.asarray(words, dtype=np.uint32).reshape(N, K // cpw)
    mask = np.uint32((1 << b) - 1)
    codes = np.empty((N, K), dtype=np.uint8)
    for j in range(cpw):
        codes[:, j::cpw] = ((words >> np.uint32(b * j)) & mask).astype(np.uint8)
    return codes


def pack_codes(codes: np.ndarray, fmt: int) -> np.ndarray:
    """Inverse of unpack_codes (used by the round-trip pins)."""
    b = BITS[fmt]
    cpw = _cpw(fmt)
    codes = np.asarray(codes, dtype=np.uint32)
    N, K = codes.shape
    out = np.zeros((N, K // cpw), dtype=np.uint32)
    for j in range(cpw):
        out |= codes[:, j::cpw] << np.uint32(b * j)
    return out


def _group_params(scales, zeros, N, K, group, fmt):
    ng = K // group
    s = np.asarray(scales, dtype=np.float16).reshape(N, ng).astype(np.float32)
    if fmt in IMPLICIT_ZERO:
        if group != 32:
            raise ValueError("q4_0 and q8_0 use blocks of 32")
        z = np.full((N, ng), IMPLICIT_ZERO[fmt], dtype=np.float32)
    else:
        z = np.asarray(zeros, dtype=np.float16).reshape(N, ng).astype(np.float32)
    return s, z


def q4k_subblock_params(scales, zeros, N: int, K: int):
    """q4k: per sub-block scale d * sc and offset dmin * m, fp64 [N, K/32]
    each (both exact: an fp16 value times a 6-bit integer)."""
    if K % Q4K_SUPER != 0:
        raise ValueError("q4k needs K divisible by 256")
    ds = np.asarray(scales, dtype=np.float16).reshape(N, K // Q4K_SUPER, 2).astype(np.float64)
    sm = np.asarray(zeros, dtype=np.uint16).reshape(N, K // Q4K_SUB)
    sc = (sm & 0xFF).astype(np.float64)
    m = (sm >> 8).astype(np.float64)
    if sc.size and (sc.max() > 63 or m.max() > 63):
        raise ValueError("q4k sub-block scales and offsets are 6-bit")
    sup = np.arange(K // Q4K_SUB) // (Q4K_SUPER // Q4K_SUB)   # super-block of each sub-block
    return ds[:, sup, 0] * sc, ds[:, sup, 1] * m


def dequant_f64(words, scales, zeros, N: int, K: int, group: int, fmt: int) -> np.ndarray:
    """The dequantized weight in fp64 (exact for every format)."""
    if fmt == Q4K:
        if group != Q4K_SUPER:
            raise ValueError("q4k uses super-blocks of 256")
        q = unpack_codes(words, N, K, fmt).astype(np.float64)
        s, b = q4k_subblock_params(scales, zeros, N, K)
        sidx = np.arange(K) // Q4K_SUB
        return s[:, sidx] * q - b[:, sidx]
    q = unpack_codes(words, N, K, fmt).astype(np.float32)
    s, z = _group_params(scales, zeros, N, K, group, fmt)
    gidx = np.arange(K) // group
    return (s[:, gidx] * (q - z[:, gidx])).astype(np.float64)


def dequant_f32(words, scales, zeros, N: int, K: int, group: int, fmt: int) -> np.ndarray:
    """w[n, k] = s[n, k // g] * (q[n, k] - z[n, k // g]) in fp32 (exact; for
    q4k, d * sc * q - dmin * m rounded once to fp32)."""
    return dequant_f64(words, scales, zeros, N, K, group, fmt).astype(np.float32)


def dequant_f16(words, scales, zeros, N: int, K: int, group: int, fmt: int) -> np.ndarray:
    """The exact dequantized weight rounded once to fp16 (nearest-even)."""
    return dequant_f64(words, scales, zeros, N, K, group, fmt).astype(np.float16)


def qgemm_ref(x, words, scales, zeros, M: int, N: int, K: int, group: int, fmt: int,
              residual=None) -> np.ndarray:
    """y_ref = x . dequant(W)^T in fp64 (+ residual, when given)."""
    x64 = np.asarray(x, dtype=np.float16).reshape(M, K).astype(np.float64)
    w64 = dequant_f64(words, scales, zeros, N, K, group, fmt)
    y = x64 @ w64.T
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float16).reshape(M, N).astype(np.float64)
    return y


def rel_error(y, y_ref) -> float:
    """max |y - y_ref| / max |y_ref| over the whole output (0 for empty)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(y_ref)))
    err = float(np.max(np.abs(y - y_ref)))
    if den == 0.0:
        return 0.0 if err == 0.0 else float("inf")
    return err / den


def within_tolerance(y, y_ref, tol: float = TOLERANCE) -> bool:
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return False
    return rel_error(y, y_ref) <= tol


def fold_zero_point_ref(x, words, scales, zeros, M, N, K, group):
    """Zero-point fold used by symmetric-only kernels: for INT4 codes,
    x.(s(q-z))^T = x.(s(q-8))^T - sum_g (sum_{k in g} x) s (z - 8).
    Returned as the two fp64 terms; their difference equals qgemm_ref."""
    x64 = np.asarray(x, dtype=np.float16).reshape(M, K).astype(np.float64)
    q = unpack_codes(words, N, K, INT4_ASYM).astype(np.float64)
    s, z = _group_params(scales, zeros, N, K, group, INT4_ASYM)
    gidx = np.arange(K) // group
    sym = x64 @ (s[:, gidx].astype(np.float64) * (q - 8.0)).T
    xg = x64.reshape(M, K // group, group).sum(axis=2)            # [M, G]
    corr = xg @ (s.astype(np.float64) * (z.astype(np.float64) - 8.0)).T  # [M, N]
    return sym, corr


# ----------------------------------------------------------------------------
# looped shared block (TinyLoop README, "Why TinyLoop Exists": one block applied
# L times with the same weights).  Readings: QKV output columns are [Q|K|V];
# O consumes the V third (what attention returns when each token sees only
# itself); no norm, no activation; residual adds rounded to fp16.
# ----------------------------------------------------------------------------

def loop_block_ref(x0, lin, L: int, D: int = 2048):
    """Run the oracle's own chain.  ``lin`` is a list of 4 dicts with keys
    words, scales, zeros, N, K, group and optionally fmt (default INT4_ASYM)
    for QKV, O, up, down.  Returns the list of fp16 block outputs x_1..x_L."""
    x = np.asarray(x0, dtype=np.float16)
    M = x.shape[0]
    outs = []

    def lin_ref(a, l, residual=None):
        return qgemm_ref(a, l["words"], l["scales"], l["zeros"], M, l["N"], l["K"], l["group"],
                         l.get("fmt", INT4_ASYM), residual=residual).astype(np.float16)

    for _ in range(L):
        qkv, o, up, down = lin
        y_qkv = lin_ref(x, qkv)
        v = y_qkv[:, 2 * D:3 * D]
        h = lin_ref(v, o, residual=x)
        u = lin_ref(h, up)
        x = lin_ref(u, down, residual=h)
        outs.append(x)
    return outs
