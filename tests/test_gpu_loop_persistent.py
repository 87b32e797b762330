"""qloop_block_persistent (one launch per loop, grid barriers between the
four GEMVs) on the GPU: the oracle's looped block at small and full size,
the exact x -> 4x chain, and a barrier that is made to give up from the host
(a spin cap of 0), after which the kernel still ends and reports it."""
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


def lin_dicts(cases):
    return [dict(words=c.words, scales=c.scales, zeros=c.zeros, N=c.N, K=c.K, group=c.group, fmt=c.fmt)
            for c in cases]


def check_close(y, yr, what):
    err = oracle.rel_error(y, yr)
    say(f"  {what}: rel err {err:.3e}")
    assert np.all(np.isfinite(y)), what
    assert oracle.within_tolerance(y, yr), f"{what}: rel err {err}"


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    monkeypatch.delenv("QGEMM_LOOP_SPIN_CAP", raising=False)
    monkeypatch.delenv("QGEMM_LOOP_GRID", raising=False)


@pytest.mark.parametrize("one_launch", [False, True])
@pytest.mark.parametrize("fmt,group", [(0, 128), (0, 32), (1, 64), (2, 32), (4, 256)])
def test_persistent_loop_parity(fmt, group, one_launch):
    D, F, L = 256, 512, 3
    say(f"persistent loop fmt={fmt} g={group} D={D} F={F} L={L} one_launch={one_launch}")
    cases = [synth.random_case(5000 + 10 * fmt + i, fmt, group, N, K, 1)
             for i, (N, K) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    x0 = synth.draw_x(np.random.default_rng(5100 + fmt), 1, D)
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in cases]
    x = qgm.to_half_tensor(x0, DEV)
    _, status = qgm.loop_block_persistent(x, lins, L, one_launch=one_launch)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    ref = oracle.loop_block_ref(x0, lin_dicts(cases), L, D=D)
    check_close(x.cpu().numpy(), ref[-1], f"persistent loop x_{L}")


@pytest.mark.parametrize("grid,one_launch", [(0, False), (7, False), (0, True), (7, True)])
def test_persistent_loop_full_size(monkeypatch, grid, one_launch):
    # the benchmark's decode block: D = 2048, F = 8192, INT4 g128, 8 loops; a
    # grid of 7 workgroups makes every phase loop over many blocks per workgroup
    if grid:
        monkeypatch.setenv("QGEMM_LOOP_GRID", str(grid))
    lc = synth.loop_workload(M=1, L=8)
    say(f"persistent loop full size M=1 D=2048 F=8192 L=8 grid={grid or 'default'} one_launch={one_launch}")
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in lc.linears()]
    x = qgm.to_half_tensor(lc.x0, DEV)
    _, status = qgm.loop_block_persistent(x, lins, lc.L, one_launch=one_launch)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    ref = oracle.loop_block_ref(lc.x0, lin_dicts(lc.linears()), lc.L)
    check_close(x.cpu().numpy(), ref[-1], "persistent loop x_8 full size")


@pytest.mark.parametrize("one_launch", [False, True])
def test_persistent_loop_exact_chain(one_launch):
    # exact weights: every loop is x -> 4x, bit for bit
    D, L = 64, 3
    say(f"persistent loop exact chain one_launch={one_launch}")
    x0 = (np.random.default_rng(3).integers(-8, 9, size=(1, D)) / 8.0).astype(np.float16)
    lins = [qgm.QuantLinear(l["words"], l["scales"], l["zeros"], l["N"], l["K"], l["group"], l["fmt"], DEV)
            for l in pins.exact_loop_linears(D)]
    x = qgm.to_half_tensor(x0, DEV)
    _, status = qgm.loop_block_persistent(x, lins, L, one_launch=one_launch)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    assert np.array_equal(x.cpu().numpy().astype(np.float64), x0.astype(np.float64) * 4.0 ** L)


def test_persistent_loop_records_one_event_per_loop():
    D, F, L = 256, 512, 4
    cases = [synth.random_case(5300 + i, 0, 128, N, K, 1)
             for i, (N, K) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in cases]
    x = qgm.to_half_tensor(synth.draw_x(np.random.default_rng(1), 1, D), DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
    qgm.loop_block_persistent(x, lins, L, events=ev)
    ev[-1].synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(L)]
    assert all(t > 0 for t in per)


@pytest.mark.parametrize("one_launch", [False, True])
def test_persistent_loop_barrier_gives_up_when_told(monkeypatch, one_launch):
    # a spin cap of 0 polls: the first workgroups to arrive give up at once,
    # the kernel ends, status says so; the next call (default cap) is whole
    D, F, L = 256, 512, 2
    say(f"persistent loop with spin cap 0, one_launch={one_launch}")
    cases = [synth.random_case(5200 + i, 0, 128, N, K, 1)
             for i, (N, K) in enumerate(((3 * D, D), (D, D), (F, D), (D, F)))]
    lins = [qgm.QuantLinear.from_case(c, DEV) for c in cases]
    x0 = synth.draw_x(np.random.default_rng(2), 1, D)
    monkeypatch.setenv("QGEMM_LOOP_SPIN_CAP", "0")
    x = qgm.to_half_tensor(x0, DEV)
    _, status = qgm.loop_block_persistent(x, lins, L, one_launch=one_launch)
    torch.cuda.synchronize()
    assert int(status[0]) == 1
    monkeypatch.delenv("QGEMM_LOOP_SPIN_CAP")
    x = qgm.to_half_tensor(x0, DEV)
    _, status = qgm.loop_block_persistent(x, lins, L, status=status, one_launch=one_launch)
    torch.cuda.synchronize()
    assert int(status[0]) == 0
    ref = oracle.loop_block_ref(x0, lin_dicts(cases), L, D=D)
    check_close(x.cpu().numpy(), ref[-1], "persistent loop after a failed call")
