"""The seeded input generator: quantizer bounds, the q4_0 worked block, and
agreement of its canonical packing with the oracle's unpack."""
import numpy as np
import pytest

import oracle
import synth


def test_q4_0_worked_block():
    # block [0.03, -0.05, 0.01, 0.049] (padded with zeros to 32): the extreme
    # -0.05 maps to -8, so d = 0.00625 and the codes are [5, -8, 2, 7] (0.049
    # would be 8 and clips to 7).
    w = np.zeros((1, 32), np.float32)
    w[0, :4] = [0.03, -0.05, 0.01, 0.049]
    u, s = synth.quantize_q4_0(w)
    assert float(s[0, 0]) == float(np.float16(0.00625))
    assert list(u[0, :4].astype(int) - 8) == [5, -8, 2, 7]
    assert np.all(u[0, 4:] == 8)


def test_q8_0_worked_block():
    # block [0.5, -1.27, 0.004, 1.0] (padded with zeros to 32): max |w| = 1.27,
    # d = 0.01 (fp16 0.010002136...), codes rint(w / d) = [50, -127, 0, 100]
    w = np.zeros((1, 32), np.float32)
    w[0, :4] = [0.5, -1.27, 0.004, 1.0]
    u, s = synth.quantize_q8_0(w)
    assert float(s[0, 0]) == float(np.float16(0.01))
    assert list(u[0, :4].astype(int) - 128) == [50, -127, 0, 100]
    assert np.all(u[0, 4:] == 128)
    z, sz = synth.quantize_q8_0(np.zeros((2, 64), np.float32))
    assert np.all(z == 128) and np.all(sz == 0)


def test_q8_0_integer_operands_round_trip():
    # a block that already is an fp16 scale times integers in [-127, 127] with
    # one of magnitude 127 comes back exactly through quantizer and oracle
    rng = np.random.default_rng(77)
    N, K = 16, 256
    q = rng.integers(-127, 128, size=(N, K // 32, 32))
    q[:, :, 5] = np.where(rng.integers(0, 2, size=(N, K // 32)) == 1, 127, -127)
    d = rng.uniform(1e-4, 0.1, size=(N, K // 32)).astype(np.float16).astype(np.float32)
    w = (q * d[:, :, None]).astype(np.float32).reshape(N, K)
    c = synth.quantize(w, synth.Q8_0, 32)
    assert np.array_equal(c.scales.astype(np.float32), d)
    assert np.array_equal(c.codes.astype(int) - 128, q.reshape(N, K))
    back = oracle.dequant_f32(c.words, c.scales, None, N, K, 32, oracle.Q8_0)
    assert np.array_equal(back, w)


def test_q4k_quantizer_bounds_and_error():
    rng = np.random.default_rng(31)
    w = synth.draw_weights(rng, 32, 1024)
    codes, scales, zeros = synth.quantize_q4k(w)
    assert codes.max() <= 15 and scales.shape == (32, 4, 2) and zeros.shape == (32, 32)
    assert (zeros & 0xFF).max() <= 63 and (zeros >> 8).max() <= 63
    deq = oracle.dequant_f64(synth.pack_words(codes, 4), scales, zeros, 32, 1024, 256, oracle.Q4K)
    # every weight within one sub-block step (d * sc) of its dequantized value
    step = (scales[:, :, 0].astype(np.float64)[:, np.arange(32) // 8] * (zeros & 0xFF))[:, np.arange(1024) // 32]
    assert np.all(np.abs(deq - w) <= step * 1.0 + 1e-7)
    assert np.sqrt(np.mean((deq - w) ** 2)) < 0.1 * np.sqrt(np.mean(w.astype(np.float64) ** 2))


def test_q4k_worked_sub_block():
    # one super-block; sub-block 0 = [-0.3, 0.6, 0, ...], every other weight 0:
    # offset 0.3, scale t0 = 0.9 / 15 = 0.06; all other sub-blocks t = o = 0.
    # d = 0.06 / 63, dmin = 0.3 / 63 (fp16), so sc0 = m0 = 63 and the codes are
    # rint((w + dmin*63) / (d*63)) = [0, 15, 5, 5, ...] in sub-block 0
    w = np.zeros((1, 256), np.float32)
    w[0, :2] = [-0.3, 0.6]
    codes, scales, zeros = synth.quantize_q4k(w)
    assert int(zeros[0, 0]) == 63 | (63 << 8)
    assert np.all(zeros[0, 1:] == 0)
    assert float(scales[0, 0, 0]) == float(np.float16(0.06 / 63))
    assert float(scales[0, 0, 1]) == float(np.float16(0.3 / 63))
    assert list(codes[0, :4]) == [0, 15, 5, 5]
    assert np.all(codes[0, 32:] == 0)


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (2, 64), (2, 32)])
def test_asym_quantizer_bounds(bits, group):
    rng = np.random.default_rng(bits * 1000 + group)
    w = synth.draw_weights(rng, 64, 512)
    codes, s, z = synth.quantize_asym(w, bits, group)
    qmax = (1 << bits) - 1
    assert codes.max() <= qmax and z.max() <= qmax and z.min() >= 0
    assert np.all(np.floor(z.astype(np.float32)) == z.astype(np.float32))
    sf = s.astype(np.float32)[:, np.arange(512) // group]
    zf = z.astype(np.float32)[:, np.arange(512) // group]
    deq = sf * (codes.astype(np.float32) - zf)
    unclipped = (codes > 0) & (codes < qmax)
    # unclipped elements are within half a step of the dense weight
    assert np.all(np.abs(w - deq)[unclipped] <= 0.5 * sf[unclipped] * (1 + 1e-3))
    # the group extremes land at (or next to) the ends of the code range
    wg = w.reshape(64, -1, group)
    cg = codes.reshape(64, -1, group)
    lo_code = np.take_along_axis(cg, wg.argmin(axis=2)[:, :, None], 2)
    hi_code = np.take_along_axis(cg, wg.argmax(axis=2)[:, :, None], 2)
    assert lo_code.max() <= 1 and hi_code.min() >= qmax - 1


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_generator_words_match_oracle_unpack(fmt):
    c = synth.random_codes_case(9, fmt, {1: 64, 4: 256}.get(fmt, 32), 48, 512, 2)
    assert np.array_equal(oracle.unpack_codes(c.words, c.N, c.K, fmt), c.codes)


def test_workloads_shapes_and_seeds():
    c = synth.workload("tiny_int4_g32")
    assert (c.N, c.K, c.M, c.group) == (256, 256, 4, 32)
    assert c.words.shape == (256, 32) and c.scales.shape == (256, 8)
    assert np.abs(c.x.astype(np.float32)).max() <= 1.0
    c2 = synth.workload("tiny_int4_g32")
    assert np.array_equal(c.words, c2.words) and np.array_equal(c.x, c2.x)
    p = synth.WORKLOADS["int2_g64"]
    q = synth.WORKLOADS["q4_0_b32"]
    assert p["seed"] == q["seed"]     # the same W feeds both formats
