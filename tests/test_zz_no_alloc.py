"""qgemm_noalloc (split-K partials in the library's fixed per-GPU array, no
device allocation) against qgemm_ex on the same inputs: bit for bit, since
both run the same kernels with the same deterministic split-K order.  Two
calls in a row, the second on a smaller problem, so the second reads an
array that still holds the first call's partials."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU visible", allow_module_level=True)
import bit_weight_only_dequant_amd as qgm  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def _run_both(c, M, residual):
    lin = qgm.QuantLinear.from_case(c, DEV)
    x = qgm.to_half_tensor(c.x[:M], DEV)
    r = qgm.to_half_tensor(residual, DEV) if residual is not None else None
    # reference: qgemm_ex with a caller workspace full of NaN (its contents
    # must not matter) and with the library's own workspace
    need = qgm.workspace_bytes(M, c.N, c.K, c.group, c.fmt)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    y_ex = lin(x, residual=r, workspace=ws)
    y_lib = lin(x, residual=r)
    y_na = torch.full((M, c.N), 3.0, dtype=torch.float16, device=DEV)
    qgm.qgemm_noalloc(x, lin.packed, lin.scales, lin.zeros, c.N, c.K, c.group, c.fmt, y_na, residual=r)
    torch.cuda.synchronize()
    return y_ex.cpu().numpy(), y_lib.cpu().numpy(), y_na.cpu().numpy()


# (fmt, group, N, K, M): every pair's first case needs more split-K partials
# than its second, and each plan splits K, so the array is really used
PAIRS = [
    ((2, 32, 2048, 8192, 128), (0, 32, 64, 16384, 40)),    # GEMM split 4 (4 MiB), then GEMM split
    ((0, 128, 256, 8192, 1), (3, 32, 32, 4096, 1)),        # GEMV split 8, then a smaller GEMV split
    ((3, 32, 1024, 16384, 128), (4, 256, 16, 8192, 8)),    # GEMM split 8, then the MFMA GEMV split
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_qgemm_ex_twice(first, second):
    for i, (fmt, group, N, K, M) in enumerate((first, second)):
        plan = qgm.plan(M, N, K, group, fmt)
        need = qgm.workspace_bytes(M, N, K, group, fmt)
        say(f"noalloc call {i}: fmt={fmt} g={group} N={N} K={K} M={M} plan={plan} partials={need}")
        assert plan["splits"] > 1 and 0 < need <= qgm.NOALLOC_SCRATCH_BYTES
        c = synth.random_codes_case(101 + 7 * i + fmt, fmt, group, N, K, M)
        res = np.random.default_rng(5 + i).standard_normal((M, N)).astype(np.float16) if i else None
        y_ex, y_lib, y_na = _run_both(c, M, res)
        assert np.array_equal(y_na.view(np.uint16), y_ex.view(np.uint16)), "noalloc != qgemm_ex (caller workspace)"
        assert np.array_equal(y_na.view(np.uint16), y_lib.view(np.uint16)), "noalloc != qgemm_ex (library workspace)"
        y_ref = oracle.qgemm_ref(c.x[:M], c.words, c.scales, c.zeros, M, N, K, group, fmt, residual=res)
        assert oracle.within_tolerance(y_na, y_ref), oracle.rel_error(y_na, y_ref)


def test_noalloc_refuses_plans_beyond_its_array():
    # 56 MiB of partials: refused before any launch, y untouched
    M, N, K, group, fmt = 512, 4096, 14336, 32, 2
    assert qgm.workspace_bytes(M, N, K, group, fmt) > qgm.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    packed = torch.zeros(qgm.packed_bytes(N, K, fmt) // 4, dtype=torch.int32, device=DEV)
    scales = torch.zeros((N, K // group), dtype=torch.float16, device=DEV)
    y = torch.full((M, N), 2.0, dtype=torch.float16, device=DEV)
    with pytest.raises(qgm.QGemmError) as e:
        qgm.qgemm_noalloc(x, packed, scales, None, N, K, group, fmt, y)
    assert e.value.status == 6   # QG_E_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 2.0).all())
