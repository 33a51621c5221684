"""The entry point that allocates nothing (mul_mat_q4_0_q8_0_noalloc), through
the C ABI, against the operator it varies (mul_mat_q4_0_q8_0): two calls in a
row on each kernel family, the second with a smaller input (the fixed scratch
keeps the first call's contents), every output within the operator's bar of
both the operator and the oracle, and bit for bit equal to the caller-
workspace form, which runs the same kernels.  Sizes past the fixed scratch are
refused before anything is launched."""
import numpy as np
import pytest
import torch

from q4_block_quantized_amd import inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-5


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device")
    from q4_block_quantized_amd import binding
    return binding.lib()


def _abi(L, name, Wq, rows, K, X, N, Y, *extra):
    stream = torch.cuda.current_stream().cuda_stream
    return getattr(L, name)(Wq.data_ptr(), rows, K, X.data_ptr(), N, Y.data_ptr(), *extra, stream)


def _within(Y, Yref):
    Y = Y.astype(np.float64)
    return np.all(np.abs(Y - Yref) <= RTOL * np.abs(Yref) + ATOL)


# (first call, second call with a smaller input): matrix-core kernel (scratch
# holds the prefill records), row kernel with the quantizer's buffer in the
# scratch (N * K above 16384), task kernel, and one token (no scratch used)
SEQUENCES = [((1000, 4096, 512), (300, 4096, 130)),
             ((700, 14336, 8), (700, 4096, 3)),
             ((513, 768, 6), (129, 768, 2)),
             ((2304, 768, 1), (64, 768, 1))]


@pytest.mark.parametrize("first,second", SEQUENCES)
def test_noalloc_twice_against_the_operator(L, orc, first, second):
    from q4_block_quantized_amd import binding as hip
    for rows, K, N in (first, second):
        print("noalloc rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W = inputs.random_matrix(71000 + rows + K, rows, K, 0.02)
        X = inputs.random_matrix(72000 + N + K, N, K)
        Wq = hip.q4_0_quantize(torch.from_numpy(W).cuda())
        Xt = torch.from_numpy(X).cuda()
        Y_na = torch.full((N, rows), float("nan"), dtype=torch.float32, device="cuda")
        Y_op = torch.empty((N, rows), dtype=torch.float32, device="cuda")
        Y_ex = torch.empty((N, rows), dtype=torch.float32, device="cuda")
        ws = hip.workspace(rows, K, N)
        torch.cuda.synchronize()
        assert _abi(L, "mul_mat_q4_0_q8_0_noalloc", Wq, rows, K, Xt, N, Y_na) == 0
        assert _abi(L, "mul_mat_q4_0_q8_0", Wq, rows, K, Xt, N, Y_op) == 0
        assert _abi(L, "mul_mat_q4_0_q8_0_ex", Wq, rows, K, Xt, N, Y_ex, ws.data_ptr(), ws.numel()) == 0
        torch.cuda.synchronize()
        y_na, y_op = Y_na.cpu().numpy(), Y_op.cpu().numpy()
        assert np.array_equal(y_na, Y_ex.cpu().numpy()), (rows, K, N)
        assert _within(y_na, y_op.astype(np.float64)), (rows, K, N)
        Yref = orc.mul_mat_ref(orc.q4_0_quantize(W), orc.q8_0_quantize(X), K)
        assert _within(y_na, Yref), (rows, K, N)


def test_noalloc_refuses_sizes_past_its_scratch(L):
    from q4_block_quantized_amd import binding as hip
    rows, K, N = 64, 32768, 512          # prefill records: 512 * 1024 * 64 B = 32 MiB > 16 MiB
    assert hip.q4bq_workspace_size(rows, K, N) > hip.NOALLOC_SCRATCH_BYTES
    Wq = torch.zeros((rows, K // 32 * 18), dtype=torch.uint8, device="cuda")
    X = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    Y = torch.full((N, rows), 7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    assert _abi(L, "mul_mat_q4_0_q8_0_noalloc", Wq, rows, K, X, N, Y) == hip.Q4BQ_ESCRATCH
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))     # nothing was launched
