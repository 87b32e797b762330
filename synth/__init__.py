"""Seeded synthetic inputs for the weight-only low-bit matmul y = x . dequant(W)^T.

This module is shared by the tests, the benchmark and the smoke check.  It draws
the dense weights and activations, turns the weights into integer codes plus
fp16 scales (and zero points) and packs the codes into 32-bit words in the
canonical order.  It holds no dequantization and no matrix product: those live
in the CPU oracle (``oracle/``) and in the HIP library, which share no code.

Where the sources are silent the readings below are used:

* W is [N, K]; groups run along K inside one output row n.
* Asymmetric b-bit groups (INT4 with GPTQ-style zero points, and the INT2 body
  weights of the TinyLoop README, sections "Status" and "Current Runtime
  Snapshot"): scale = (max - min) / (2^b - 1) rounded to fp16 (nearest-even);
  zero = clip(rint(-min / scale), 0, 2^b - 1) computed from the stored fp16
  scale; code = clip(rint(w / scale) + zero, 0, 2^b - 1).  A constant group
  uses scale 1.
* q4_0 (named in the torchnative guide "Inference with real transformers",
  section "Quantise while loading"): blocks of 32, one fp16 scale, no zero
  point, signed codes in [-8, 7].  d = m / -8 where m is the signed element of
  largest magnitude; code = clip(rint(w / fp16(d)), -8, 7); stored as the
  offset-binary nibble u = code + 8.  An all-zero block has scale 0, u = 8.
* q8_0 (same guide and section): blocks of 32, one fp16 scale, signed codes
  in [-127, 127].  d = max|w| / 127; code = clip(rint(w / fp16(d)), -127, 127);
  stored as the offset-binary byte u = code + 128.  An all-zero block has
  scale 0, u = 128.  A block that already is d times integers in [-127, 127]
  with one of magnitude 127 (d an fp16 value) is reproduced exactly.
* q4k (same guide and section, named only, with widths divisible by 256):
  the k-quant reading -- super-blocks of 256 with fp16 (d, dmin), sub-blocks
  of 32 with 6-bit (sc, m), w = d * sc * q - dmin * m, q in 0..15.  Quantizer:
  per sub-block, offset o = max(0, -min) and scale t = (max + o) / 15; per
  super-block d = max t / 63 and dmin = max o / 63 in fp16; sc = rint(t / d),
  m = rint(o / dmin), both clipped to 0..63; q = clip(rint((w + dmin m) /
  (d sc)), 0, 15) with the stored values.  Metadata: scales fp16 [N, K/256, 2]
  = (d, dmin), zeros uint16 [N, K/32] = sc | m << 8.
* Canonical packing: code (n, k) sits in word [n, k // cpw] at bits
  [b*(k % cpw), b*(k % cpw) + b), i.e. least significant bits first along K,
  cpw = 32 / b codes per uint32.
* "N(0, 0.02)" is a standard deviation of 0.02; x is drawn in fp32 and rounded
  to fp16 (nearest-even).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

INT4_ASYM = 0
INT2_ASYM = 1
Q4_0 = 2
Q8_0 = 3
Q4K = 4

FORMAT_NAMES = {INT4_ASYM: "int4_asym", INT2_ASYM: "int2_asym", Q4_0: "q4_0", Q8_0: "q8_0", Q4K: "q4k"}
FORMAT_BITS = {INT4_ASYM: 4, INT2_ASYM: 2, Q4_0: 4, Q8_0: 8, Q4K: 4}
SYMMETRIC = (Q4_0, Q8_0)   # block formats with no stored zero point


def codes_per_word(fmt: int) -> int:
    return 32 // FORMAT_BITS[fmt]


# ----------------------------------------------------------------------------
# quantizers (input generation only)
# ----------------------------------------------------------------------------

def quantize_asym(w: np.ndarray, bits: int, group: int):
    """Asymmetric per-group quantizer.  Returns (codes uint8 [N,K], scale fp16
    [N,K/g], zero fp16 [N,K/g])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % group == 0
    qmax = (1 << bits) - 1
    wg = w.reshape(n, k // group, group)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    s32 = ((hi - lo) / np.float32(qmax)).astype(np.float32)
    s16 = s32.astype(np.float16)
    flat = (hi == lo) | (s16 == 0)
    s16 = np.where(flat, np.float16(1.0), s16)
    sf = s16.astype(np.float32)
    z = np.clip(np.rint(-lo / sf), 0, qmax).astype(np.float32)
    q = np.clip(np.rint(wg / sf[:, :, None]) + z[:, :, None], 0, qmax)
    codes = q.astype(np.uint8).reshape(n, k)
    return codes, s16, z.astype(np.float16)


def quantize_q4_0(w: np.ndarray, block: int = 32):
    """Symmetric block quantizer.  Returns (offset-binary codes uint8 [N,K] in
    [0, 15], scale fp16 [N,K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % block == 0
    wb = w.reshape(n, k // block, block)
    idx = np.abs(wb).argmax(axis=2)
    m = np.take_along_axis(wb, idx[:, :, None], axis=2)[:, :, 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    s16 = d.astype(np.float16)
    sf = s16.astype(np.float32)
    safe = np.where(sf == 0, np.float32(1.0), sf)
    q = np.clip(np.rint(wb / safe[:, :, None]), -8, 7)
    q = np.where((sf == 0)[:, :, None], 0, q)
    u = (q + 8).astype(np.uint8).reshape(n, k)
    return u, s16


def quantize_q8_0(w: np.ndarray, block: int = 32):
    """Symmetric 8-bit block quantizer.  Returns (offset-binary codes uint8
    [N,K] in [1, 255], scale fp16 [N,K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % block == 0
    wb = w.reshape(n, k // block, block)
    amax = np.abs(wb).max(axis=2)
    s16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    sf = s16.astype(np.float32)
    safe = np.where(sf == 0, np.float32(1.0), sf)
    q = np.clip(np.rint(wb / safe[:, :, None]), -127, 127)
    q = np.where((sf == 0)[:, :, None], 0, q)
    u = (q + 128).astype(np.uint8).reshape(n, k)
    return u, s16


def quantize_q4k(w: np.ndarray):
    """k-quant 4-bit quantizer.  Returns (codes uint8 [N,K] in [0, 15],
    scales fp16 [N,K/256,2] = (d, dmin), zeros uint16 [N,K/32] = sc | m << 8)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % 256 == 0
    ns = k // 32
    wb = w.reshape(n, ns, 32)
    off = np.maximum(0.0, -wb.min(axis=2)).astype(np.float32)          # [n, ns]
    t = ((wb.max(axis=2) + off) / np.float32(15.0)).astype(np.float32)
    tS = t.reshape(n, k // 256, 8)
    oS = off.reshape(n, k // 256, 8)
    d = (tS.max(axis=2) / np.float32(63.0)).astype(np.float16)
    dmin = (oS.max(axis=2) / np.float32(63.0)).astype(np.float16)
    df = d.astype(np.float32)[:, :, None]
    mf = dmin.astype(np.float32)[:, :, None]
    sc = np.where(df > 0, np.clip(np.rint(tS / np.where(df > 0, df, 1)), 0, 63), 0).reshape(n, ns)
    m = np.where(mf > 0, np.clip(np.rint(oS / np.where(mf > 0, mf, 1)), 0, 63), 0).reshape(n, ns)
    sup = np.arange(ns) // 8
    s_eff = d.astype(np.float32)[:, sup] * sc.astype(np.float32)      # [n, ns]
    b_eff = dmin.astype(np.float32)[:, sup] * m.astype(np.float32)
    safe = np.where(s_eff > 0, s_eff, 1.0)
    q = np.clip(np.rint((wb + b_eff[:, :, None]) / safe[:, :, None]), 0, 15)
    q = np.where((s_eff > 0)[:, :, None], q, 0)
    codes = q.astype(np.uint8).reshape(n, k)
    scales = np.stack([d, dmin], axis=-1)
    zeros = (sc.astype(np.uint16) | (m.astype(np.uint16) << 8)).astype(np.uint16)
    return codes, scales, zeros


def pack_words(codes: np.ndarray, bits: int) -> np.ndarray:
    """Canonical packing: least significant bits first along K."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, k = codes.shape
    cpw = 32 // bits
    assert k % cpw == 0
    c = codes.reshape(n, k // cpw, cpw)
    words = np.zeros((n, k // cpw), dtype=np.uint32)
    for j in range(cpw):
        words |= (c[:, :, j] & np.uint32((1 << bits) - 1)) << np.uint32(bits * j)
    return words


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------

@dataclass
class QCase:
    """One quantized weight matrix plus activations."""
    fmt: int
    group: int
    N: int
    K: int
    codes: np.ndarray            # uint8 [N, K]
    words: np.ndarray            # uint32 [N, K / cpw], canonical order
    scales: np.ndarray           # fp16 [N, K / group]
    zeros: Optional[np.ndarray]  # fp16 [N, K / group] or None for q4_0 / q8_0
    #                              (q4k: scales fp16 [N, K/256, 2], zeros uint16 [N, K/32])
    x: Optional[np.ndarray] = None  # fp16 [M, K]

    @property
    def M(self) -> int:
        return 0 if self.x is None else self.x.shape[0]

    @property
    def weight_bytes(self) -> int:
        b = self.words.nbytes + self.scales.nbytes
        if self.zeros is not None:
            b += self.zeros.nbytes
        return b


def quantize(w: np.ndarray, fmt: int, group: int) -> QCase:
    n, k = w.shape
    if fmt == Q4_0:
        assert group == 32
        codes, s = quantize_q4_0(w, 32)
        z = None
    elif fmt == Q8_0:
        assert group == 32
        codes, s = quantize_q8_0(w, 32)
        z = None
    elif fmt == Q4K:
        assert group == 256
        codes, s, z = quantize_q4k(w)
    else:
        codes, s, z = quantize_asym(w, FORMAT_BITS[fmt], group)
    return QCase(fmt=fmt, group=group, N=n, K=k, codes=codes,
                 words=pack_words(codes, FORMAT_BITS[fmt]), scales=s, zeros=z)


def draw_weights(rng: np.random.Generator, n: int, k: int, std: float = 0.02) -> np.ndarray:
    return (rng.standard_normal((n, k)) * std).astype(np.float32)


def draw_x(rng: np.random.Generator, m: int, k: int, dist: str = "normal") -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal((m, k)).astype(np.float32)
    elif dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=(m, k)).astype(np.float32)
    else:
        raise ValueError(dist)
    return x.astype(np.float16)


def random_case(seed: int, fmt: int, group: int, N: int, K: int, M: int,
                xdist: str = "normal") -> QCase:
    """A generic seeded case: W ~ N(0, 0.02) [N, K] then x [M, K]."""
    rng = np.random.default_rng(seed)
    w = draw_weights(rng, N, K)
    c = quantize(w, fmt, group)
    c.x = draw_x(rng, M, K, xdist)
    return c


def random_codes_case(seed: int, fmt: int, group: int, N: int, K: int, M: int) -> QCase:
    """Uniformly random codes / scales / zeros (stress case: every code value
    and every zero point appear).  Scales ~ 0.005 * U(0.5, 1.5) in fp16."""
    rng = np.random.default_rng(seed)
    bits = FORMAT_BITS[fmt]
    codes = rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)
    if fmt == Q4K:
        # d, dmin ~ 3e-4 * U(0.5, 1.5); sc, m uniform over 0..63
        ds = (3e-4 * rng.uniform(0.5, 1.5, size=(N, K // 256, 2))).astype(np.float16)
        sc = rng.integers(0, 64, size=(N, K // 32))
        m = rng.integers(0, 64, size=(N, K // 32))
        z = (sc | (m << 8)).astype(np.uint16)
        x = draw_x(rng, M, K, "normal")
        return QCase(fmt=fmt, group=group, N=N, K=K, codes=codes,
                     words=pack_words(codes, bits), scales=ds, zeros=z, x=x)
    s = (0.005 * rng.uniform(0.5, 1.5, size=(N, K // group))).astype(np.float16)
    z = None
    if fmt not in SYMMETRIC:
        z = rng.integers(0, 1 << bits, size=(N, K // group)).astype(np.float16)
    x = draw_x(rng, M, K, "normal")
    return QCase(fmt=fmt, group=group, N=N, K=K, codes=codes,
                 words=pack_words(codes, bits), scales=s, zeros=z, x=x)


# Named workloads.  Seeds and draw order: W (then each further W), then x.
WORKLOADS: Dict[str, dict] = {
    "tiny_int4_g32":   dict(seed=1001, fmt=INT4_ASYM, group=32,  N=256,  K=256,  M=4, xdist="uniform", Ms=(1, 4)),
    "decode_int4_g128": dict(seed=1002, fmt=INT4_ASYM, group=128, N=6144, K=2048, M=8, xdist="normal", Ms=(1, 8)),
    "prefill_int4_g128": dict(seed=1003, fmt=INT4_ASYM, group=128, N=8192, K=2048, M=128, xdist="normal", Ms=(128,)),
    "int2_g64":        dict(seed=1004, fmt=INT2_ASYM, group=64,  N=8192, K=2048, M=128, xdist="normal", Ms=(1, 128)),
    "q4_0_b32":        dict(seed=1004, fmt=Q4_0,      group=32,  N=8192, K=2048, M=128, xdist="normal", Ms=(1, 128)),
    "q8_0_b32":        dict(seed=1004, fmt=Q8_0,      group=32,  N=8192, K=2048, M=128, xdist="normal", Ms=(1, 128)),
    "q4k_s256":        dict(seed=1004, fmt=Q4K,       group=256, N=8192, K=2048, M=128, xdist="normal", Ms=(1, 128)),
}


def workload(name: str) -> QCase:
    p = WORKLOADS[name]
    rng = np.random.default_rng(p["seed"])
    w = draw_weights(rng, p["N"], p["K"])
    c = quantize(w, p["fmt"], p["group"])
    c.x = draw_x(rng, p["M"], p["K"], p["xdist"])
    return c


# Looped shared block: QKV 2048->6144, O 2048->2048, up 2048->8192, down 8192->2048.
LOOP_DIMS = dict(D=2048, QKV=6144, MLP=8192)
LOOP_SEED = 1005


@dataclass
class LoopCase:
    qkv: QCase
    o: QCase
    up: QCase
    down: QCase
    x0: np.ndarray   # fp16 [M, D]
    L: int = 8

    def linears(self) -> List[QCase]:
        return [self.qkv, self.o, self.up, self.down]


def loop_workload(M: int = 128, D: int = 2048, qkv: int = 6144, mlp: int = 8192,
                  group: int = 128, L: int = 8, seed: int = LOOP_SEED) -> LoopCase:
    rng = np.random.default_rng(seed)
    ws = [draw_weights(rng, qkv, D), draw_weights(rng, D, D),
          draw_weights(rng, mlp, D), draw_weights(rng, D, mlp)]
    qs = [quantize(w, INT4_ASYM, group) for w in ws]
    x0 = draw_x(rng, M, D, "normal")
    return LoopCase(qkv=qs[0], o=qs[1], up=qs[2], down=qs[3], x0=x0, L=L)
