"""Parity of the HIP path with the CPU oracle, through the C ABI.

Bars (fixed before any kernel existed):
  * Q4_0 / Q8_0 bytes and per-block int32 dots: bit-exact;
  * fp32 outputs: |Y - Y_ref| <= 1e-4 * |Y_ref| + 1e-5 element-wise, Y_ref the
    oracle's fp64 accumulation of exact per-block terms.

Every input is seeded and synthetic (q4_block_quantized_amd.inputs); the oracle
quantizes its own copy of each fp32 input, nothing it sees comes from the GPU.
"""
import numpy as np
import pytest
import torch

from conftest import hexbytes, read_golden
from q4_block_quantized_amd import inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-5


@pytest.fixture(scope="module")
def hip():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device: the parity tests need an MI355X")
    from q4_block_quantized_amd import binding
    binding.lib()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(Y, Yref, what):
    Y = Y.astype(np.float64)
    err = np.abs(Y - Yref)
    lim = RTOL * np.abs(Yref) + ATOL
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outside tolerance; first at %s: got %r want %r"
                             % (what, int(bad.sum()), Y.size, tuple(i), Y[tuple(i)], Yref[tuple(i)]))


def edge_blocks():
    rng = np.random.default_rng(5)
    parts = [inputs.random_matrix(51, 64, 32, 0.02), inputs.random_matrix(52, 64, 32, 1.0),
             inputs.random_matrix(53, 16, 32, 1e-6), inputs.random_matrix(54, 16, 32, 1e-9),
             inputs.random_matrix(55, 16, 32, 3000.0), np.zeros((2, 32), np.float32)]
    spiky = inputs.random_matrix(56, 32, 32, 0.02)
    spiky[np.arange(32), rng.integers(0, 32, 32)] *= 10.0
    parts.append(spiky)
    ties = np.zeros((2, 32), np.float32)
    ties[0, :6] = [-1.0, 0.0625, -0.0625, 0.1875, 0.3125, 1.0]
    ties[1, :5] = [0.9921875, 2.0 ** -8, -1.5 * 2.0 ** -7, 2.5 * 2.0 ** -7, -0.5 * 2.0 ** -7]
    parts.append(ties)
    ramp = np.array([((k % 16) - 8) / 8 for k in range(32)], np.float32)[None]
    parts += [ramp, np.ones((1, 32), np.float32), -np.zeros((1, 32), np.float32)]
    return np.concatenate(parts, axis=0)


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def test_quantizers_golden_blocks(hip, orc):
    ramp = np.array([((k % 16) - 8) / 8 for k in range(32)], np.float32)[None]
    got = host(hip.q4_0_quantize(dev(ramp)))[0]
    assert np.array_equal(got, hexbytes(read_golden("q4_0_ramp_block.txt")["bytes"][0]))
    w = np.zeros((1, 32), np.float32)
    w[0, :6] = [-1.0, 0.0625, -0.0625, 0.1875, 0.3125, 1.0]
    assert np.array_equal(host(hip.q4_0_quantize(dev(w)))[0],
                          hexbytes(read_golden("q4_0_tie_clip_block.txt")["bytes"][0]))
    assert np.array_equal(host(hip.q8_0_quantize(dev(np.ones((1, 32), np.float32))))[0],
                          hexbytes(read_golden("q8_0_ones_block.txt")["bytes"][0]))
    z = np.zeros((1, 32), np.float32)
    g = read_golden("zero_blocks.txt")
    assert np.array_equal(host(hip.q4_0_quantize(dev(z)))[0], hexbytes(g["q4_0_bytes"][0]))
    assert np.array_equal(host(hip.q8_0_quantize(dev(z)))[0], hexbytes(g["q8_0_bytes"][0]))


def test_quantizers_edge_blocks(hip, orc):
    E = edge_blocks()
    assert np.array_equal(host(hip.q4_0_quantize(dev(E))), orc.q4_0_quantize(E))
    assert np.array_equal(host(hip.q8_0_quantize(dev(E))), orc.q8_0_quantize(E))


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (37, 160), (1000, 768), (257, 4096)])
def test_quantizers_random(hip, orc, rows, K):
    W = inputs.random_matrix(1000 + rows + K, rows, K, 0.02)
    W[inputs.random_matrix(2000 + rows + K, rows, K) > 2.33] *= 10.0
    assert np.array_equal(host(hip.q4_0_quantize(dev(W))), orc.q4_0_quantize(W))
    X = inputs.random_matrix(3000 + rows + K, rows, K)
    assert np.array_equal(host(hip.q8_0_quantize(dev(X))), orc.q8_0_quantize(X))


def test_quantizers_fp16_scale_sweep(hip, orc):
    """Blocks whose largest magnitude sweeps many binade positions, so the
    binary16 rounding of amax/8 and amax/127 meets ties and subnormals."""
    rng = np.random.default_rng(77)
    amax = np.float32(2.0) ** rng.uniform(-27, 15, 4096).astype(np.float32)
    amax = np.concatenate([amax, (np.arange(1, 2049, dtype=np.float32) * np.float32(2.0 ** -24)) * 8,
                           (np.arange(1, 2049, dtype=np.float32) * np.float32(2.0 ** -24)) * 127])
    B = rng.uniform(-1, 1, (amax.size, 32)).astype(np.float32) * amax[:, None]
    B[np.arange(amax.size), rng.integers(0, 32, amax.size)] = amax * np.where(rng.random(amax.size) < 0.5, -1, 1)
    B = B.astype(np.float32)
    assert np.array_equal(host(hip.q4_0_quantize(dev(B))), orc.q4_0_quantize(B))
    assert np.array_equal(host(hip.q8_0_quantize(dev(B))), orc.q8_0_quantize(B))


def near_half_blocks(seed, N, K):
    """N x K activations whose quotients x / d sit within a few ulps of a
    half-integer, so that the rounding of the binary32 quotient decides each
    code.  Element 0 of most blocks is +-127 d, which makes binary16(amax / 127)
    exactly d; d spans normal and subnormal binary16 values; about a third of
    the elements are ordinary values of the block's range."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    bits = np.where(rng.random((N, nb)) < 0.2, rng.integers(1, 0x400, (N, nb)), rng.integers(0x0400, 0x5BFF, (N, nb)))
    d = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    k = rng.integers(-127, 127, (N, nb, 32))
    x = ((k + 0.5) * d[..., None]).astype(np.float32)
    nudge = rng.integers(-3, 4, (N, nb, 32))
    for step in range(1, 4):
        x = np.where(nudge >= step, np.nextafter(x, np.float32(np.inf)), x)
        x = np.where(-nudge >= step, np.nextafter(x, np.float32(-np.inf)), x)
    plain = (rng.uniform(-126.9, 126.9, (N, nb, 32)) * d[..., None]).astype(np.float32)
    x = np.where(rng.random((N, nb, 32)) < 0.33, plain, x)
    x[..., 0] = (np.where(rng.random((N, nb)) < 0.5, -127.0, 127.0) * d).astype(np.float32)
    # A quarter of the blocks: amax / 127 = (m + u) 2^-24 with u < 1/2 rounds
    # down to the binary16 subnormal d = m 2^-24, so quotients reach 127 (1 + u/m)
    # (up to ~184, clamped to 127 when rounded), near half-integers up there too.
    m = rng.integers(1, 24, (N, nb)).astype(np.float64)
    u = rng.uniform(0.0, 0.45, (N, nb))
    top = 127.0 * (m + u) / m  # amax / d
    kk = np.floor(rng.uniform(-1.0, 1.0, (N, nb, 32)) * (top[..., None] - 1.0))
    xs = ((kk + 0.5) * (m * 2.0 ** -24)[..., None]).astype(np.float32)
    for step in range(1, 4):
        xs = np.where(nudge >= step, np.nextafter(xs, np.float32(np.inf)), xs)
        xs = np.where(-nudge >= step, np.nextafter(xs, np.float32(-np.inf)), xs)
    xs[..., 0] = (np.where(rng.random((N, nb)) < 0.5, -1.0, 1.0) * top * m * 2.0 ** -24).astype(np.float32)
    x = np.where((rng.random((N, nb)) < 0.25)[..., None], xs, x)
    return np.ascontiguousarray(x.reshape(N, K), dtype=np.float32)


def margin_blocks(seed, N, K):
    """N x K activations whose quotients x / d all lie between 2^-12.6 and
    2^-9 from a half-integer (never closer): the quantizers round these
    without a division, and a wrong direction would change the code.
    Element 0 of every block is +-127 d (d exact, as in near_half_blocks)."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    bits = np.where(rng.random((N, nb)) < 0.2, rng.integers(1, 0x400, (N, nb)), rng.integers(0x0400, 0x5BFF, (N, nb)))
    d = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    k = rng.integers(-127, 127, (N, nb, 32))
    off = 2.0 ** rng.uniform(-12.6, -9.0, (N, nb, 32)) * np.where(rng.random((N, nb, 32)) < 0.5, -1.0, 1.0)
    x = ((k + 0.5 + off) * d[..., None]).astype(np.float32)
    x[..., 0] = (np.where(rng.random((N, nb)) < 0.5, -127.0, 127.0) * d).astype(np.float32)
    return np.ascontiguousarray(x.reshape(N, K), dtype=np.float32)


def unit_code_weights(K):
    """K x K Q4_0 blocks, all scales 1.0, whose row r has the single nonzero
    code +1 at element r: every product element is then one activation code
    times its block scale, exact in fp32, so Y shows each code."""
    nb = K // 32
    Wq = np.zeros((K, nb, 18), np.uint8)
    Wq[:, :, 1] = 0x3C  # binary16 1.0, little-endian
    Wq[:, :, 2:] = 0x88  # nibble 8 = code 0
    r = np.arange(K)
    j = r % 32
    Wq[r, r // 32, 2 + j // 2] = np.where(j % 2 == 0, 0x89, 0x98)
    return Wq.reshape(K, nb * 18)


def test_quantizer_half_integer_quotients(hip, orc):
    X = near_half_blocks(31, 64, 4096)
    assert np.array_equal(host(hip.q8_0_quantize(dev(X))), orc.q8_0_quantize(X))
    X = margin_blocks(32, 64, 4096)
    assert np.array_equal(host(hip.q8_0_quantize(dev(X))), orc.q8_0_quantize(X))


@pytest.mark.parametrize("K", [768, 4096, 14336])
def test_activation_codes_in_every_product_path(hip, orc, K):
    """Quotients at half-integers through the activation quantizer of each
    product kernel (streaming decode, task kernel, two-phase, matrix cores):
    with unit_code_weights the fp32 result must equal the oracle's exactly."""
    Wq_o = unit_code_weights(K)
    dq = orc.q4_0_dequantize(Wq_o, K)
    assert np.array_equal(dq, np.eye(K, dtype=np.float32))
    Wq = dev(Wq_o)
    for N, make in [(n, f) for n in ((1, 8, 9) if K > 4096 else (1, 3, 8, 9, 130))
                    for f in (near_half_blocks, margin_blocks)]:
        print("%s K=%d N=%d" % (make.__name__, K, N), flush=True)
        X = make(4000 + K + N, N, K)
        want = orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(X), K)
        Xt = dev(X)
        got = host(hip.mul_mat_q4_0_q8_0(Wq, Xt)).astype(np.float64)
        assert np.array_equal(got, want), (K, N, int((got != want).sum()))
        ws = hip.workspace(K, K, N)
        got = host(hip.mul_mat_q4_0_q8_0_prepared(Wq, hip.q4bq_quantize_activations(Xt, ws), N, K))
        assert np.array_equal(got.astype(np.float64), want), ("two-phase", K, N)


# ---------------------------------------------------------------------------
# block dots and the product on a shape sweep (tiles, ragged tails, odd K/32)
# ---------------------------------------------------------------------------

SWEEP_K = [32, 64, 96, 160, 768, 4096]
SWEEP_ROWS = [1, 31, 64, 129, 1000]
SWEEP_N = [1, 2, 3, 4, 5, 7, 8, 9, 16, 63, 64, 65, 130]


def _case(rows, K, N, seed):
    W = inputs.random_matrix(seed, rows, K, 0.02)
    W[inputs.random_matrix(seed + 1, rows, K) > 2.33] *= 10.0
    X = inputs.random_matrix(seed + 2, N, K)
    return W, X


@pytest.mark.parametrize("K", SWEEP_K)
@pytest.mark.parametrize("rows", SWEEP_ROWS)
def test_product_sweep(hip, orc, rows, K):
    for N in SWEEP_N:
        if rows * K * N > 40_000_000:
            continue
        print("sweep rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = _case(rows, K, N, 10 * rows + K + 100000 * N)
        Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
        Wq = hip.q4_0_quantize(dev(W))
        Xt = dev(X)
        D = host(hip.q4_0_q8_0_block_dots(Wq, hip.q8_0_quantize(Xt), K))
        assert np.array_equal(D, orc.block_dots(Wq_o, Xq_o, K)), (rows, K, N)
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert Y.shape == (N, rows)
        assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))


@pytest.mark.parametrize("K", [65536, 98336])
def test_decode_rows_beyond_lds(hip, orc, K):
    """One to eight tokens on rows whose quantized activations exceed the
    decode kernels' 64 KB LDS budget (K = 98336: an odd block count): the
    activations are read from the quantizer's buffer in global memory.  Oracle
    bar, and the same bits from every entry point."""
    for rows in (3, 70):
        for N in (1, 3, 8):
            print("beyond lds rows=%d K=%d N=%d" % (rows, K, N), flush=True)
            W, X = _case(rows, K, N, 777 + rows + 3 * N)
            Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
            Wq = hip.q4_0_quantize(dev(W))
            Xt = dev(X)
            Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
            assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
            assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
            assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), (rows, K, N)
            assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)


def test_prefill_very_long_rows(hip, orc):
    """More tokens than the decode kernels take on rows of 8200 blocks: the
    prefill activation records walk the blocks in more than one pass of the
    grid (at most 8192 blocks per pass), the prefill kernel runs 4100 stages.
    Oracle bar, the block dots, and the same bits from the pre-quantized
    input."""
    rows, K = 3, 8200 * 32
    for N in (9, 40):
        print("very long rows rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = _case(rows, K, N, 4242 + N)
        Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
        Wq = hip.q4_0_quantize(dev(W))
        Xt = dev(X)
        Xq = hip.q8_0_quantize(Xt)
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, Xq, K)), Y), (rows, K, N)
        D = host(hip.q4_0_q8_0_block_dots(Wq, Xq, K))
        assert np.array_equal(D, orc.block_dots(Wq_o, Xq_o, K)), (rows, K, N)


def test_paths_agree_bitwise(hip, orc):
    """Fused quantization, pre-quantized input, caller workspace and the
    stream-ordered scratch give the same bits; so do repeated calls and a
    non-default stream."""
    for rows, K, N in [(777, 4096, 1), (300, 768, 8), (129, 160, 5), (1000, 4096, 70), (513, 4096, 5),
                       (300, 8192, 3), (129, 14336, 2)]:
        W, X = _case(rows, K, N, 555 + rows)
        Wq = hip.q4_0_quantize(dev(W))
        Xt = dev(X)
        Y1 = hip.mul_mat_q4_0_q8_0(Wq, Xt)
        Y2 = hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)
        Y3 = hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))
        Y4 = hip.mul_mat_q4_0_q8_0(Wq, Xt)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            Y5 = hip.mul_mat_q4_0_q8_0(Wq, Xt)
        s.synchronize()
        ws = hip.workspace(rows, K, N)
        Y6 = hip.mul_mat_q4_0_q8_0_prepared(Wq, hip.q4bq_quantize_activations(Xt, ws), N, K)
        ref = host(Y1)
        for other in (Y2, Y3, Y4, Y5, Y6):
            assert np.array_equal(host(other), ref), (rows, K, N)


@pytest.mark.parametrize("K", [3008, 3072, 6144, 8192, 12288, 14336, 16384, 16416])
def test_long_rows_few_tokens(hip, orc, K):
    """One to eight tokens on long rows, where whole waves stream each row: the
    oracle bar on ragged row counts, and the same bits from fused quantization,
    the pre-quantized input and the repacked weights.  K = 3008 (47 pairs per
    row) takes that kernel's short-row form; K = 16416 (an odd block count) and
    the larger token counts on the longest rows sit outside its range and check
    the other one."""
    for rows in (1, 17, 300):
        for N in (1, 2, 3, 4, 8):
            if rows * K * N > 12_000_000:
                continue
            print("long rows rows=%d K=%d N=%d" % (rows, K, N), flush=True)
            W, X = _case(rows, K, N, 900 + rows + K + 7 * N)
            Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
            Wq = hip.q4_0_quantize(dev(W))
            Xt = dev(X)
            Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
            assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
            assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
            assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)


@pytest.mark.parametrize("K", [448, 512, 768, 3008])
def test_short_rows_either_side_of_row_limit(hip, orc, K):
    """Rows of 7 to 47 block pairs: whole waves stream each row (most lanes
    idle) on matrices of up to 16384 rows, the task kernel above that and
    below 8 pairs.  Both sides of the row limit against the oracle, and the
    same bits from the pre-quantized input and the repacked weights."""
    for rows in (16384, 16385):
        for N in (1, 3):
            print("short rows rows=%d K=%d N=%d" % (rows, K, N), flush=True)
            W, X = _case(rows, K, N, 4100 + rows + K + N)
            Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
            Wq = hip.q4_0_quantize(dev(W))
            Xt = dev(X)
            Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
            assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
            assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
            assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)


@pytest.mark.parametrize("rows,K,Ns", [(2048, 64, (5, 6, 8)), (2049, 192, (5, 6, 8)), (3000, 768, (5, 6, 8)),
                                       (2080, 2048, (5, 6, 8)), (2080, 4096, (5, 6, 8)), (4100, 8192, (5, 6, 8)),
                                       (2048, 8256, (5, 6, 8)), (32800, 2048, (4, 8))])
def test_matrix_core_decode(hip, orc, rows, K, Ns):
    """Four to eight tokens on matrices of 2048 rows and more (the matrix-core
    decode kernels, one 32-row tile and block per instruction): the oracle bar,
    ragged row counts (tiles cut by the end of a workgroup's rows or of the
    matrix), short rows (block counts under 64 or not a multiple of 8 take the
    kernel with 36-byte lane loads, whose last chunk of four blocks can pass
    the row end), K = 2048 (the shortest rows of the contiguous-load kernel),
    K = 8192 (the longest rows the matrix cores take) and K = 8256 (past it:
    the other kernels), 32800 rows (long enough for four tokens on the matrix
    cores; 1025 tiles over the grid); the same bits from fused quantization,
    the pre-quantized input, a caller's workspace and the repacked weights."""
    for N in Ns:
        if rows * K * N > 600_000_000:
            continue
        print("matrix-core decode rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = _case(rows, K, N, 6100 + rows + K + N)
        Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
        Wq = hip.q4_0_quantize(dev(W))
        Xt = dev(X)
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)


@pytest.mark.parametrize("rows,K,Ns", [(66000, 3072, (1, 2, 4)), (70000, 4096, (1,))])
def test_long_matrices_contiguous_row_loads(hip, orc, rows, K, Ns):
    """One to four tokens on matrices with 16 rows or more per wave: the row
    kernel loads each row as consecutive 16-byte pieces and reorders them
    through LDS (rows of 108 and 144 pieces: two and three load instructions,
    the last one partly used; ragged row counts).  Against the oracle, and bit
    for bit against the repacked weights (which keep the lanes' own pair
    loads), the pre-quantized input and a caller's workspace; the multi-matrix
    form over two such matrices against separate calls."""
    for N in Ns:
        print("contiguous row loads rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = _case(rows, K, N, 9300 + rows + K + N)
        Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
        Wq = hip.q4_0_quantize(dev(W))
        Xt = dev(X)
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert_close(Y, orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
        assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), (rows, K, N)
        if N == 1:
            half = rows // 2 // 32 * 32
            Ys = hip.mul_mat_q4_0_q8_0_multi([Wq[:half], Wq[half:]], Xt)
            assert np.array_equal(np.concatenate([host(Ys[0]), host(Ys[1])], axis=1), Y), (rows, K, N)


@pytest.mark.parametrize("rows,K,Ns", [(66001, 4096, (5, 8)), (70000, 3072, (6,)), (68000, 2048, (4, 7))])
def test_matrix_core_whole_tiles(hip, orc, rows, K, Ns):
    """Matrix-core decode with 8 tiles of 32 rows or more per workgroup: the
    workgroup loads each tile as one contiguous run into an LDS tile (rows of
    64, 96 and 128 blocks; a ragged last tile).  Sampled rows against the
    oracle; bit for bit against the per-wave item kernel (a 40000-row prefix:
    too few tiles for this form), the repacked weights, the pre-quantized
    input and a caller's workspace; the multi-matrix form over two halves
    against the single call."""
    head = 40000
    for N in Ns:
        print("whole-tile matrix-core decode rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = _case(rows, K, N, 9500 + rows + K + N)
        sample = _sample_rows(rows, 1500, 9501 + rows + N)
        Wq_o, Xq_o = orc.q4_0_quantize(W[sample]), orc.q8_0_quantize(X)
        Wq = hip.q4_0_quantize(dev(W))
        del W
        Xt = dev(X)
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert_close(Y[:, sample], orc.mul_mat_ref(Wq_o, Xq_o, K), "rows=%d K=%d N=%d" % (rows, K, N))
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0(Wq[:head], Xt)), Y[:, :head]), ("prefix", rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), (rows, K, N)
        half = rows // 2 // 32 * 32
        Ys = hip.mul_mat_q4_0_q8_0_multi([Wq[:half], Wq[half:]], Xt)
        assert np.array_equal(np.concatenate([host(Ys[0]), host(Ys[1])], axis=1), Y), ("multi", rows, K, N)


@pytest.mark.parametrize("rows,K,Ns", [(14336, 4096, (9, 16)), (2304, 768, (9, 17, 31, 32)), (300, 3072, (9, 15, 16))])
def test_decode_groups_between_9_and_32_tokens(hip, orc, rows, K, Ns):
    """9..16 tokens (up to 32 where the matrix-core kernel would not split K:
    the 2304 x 768 matrix) run as groups of up to 8 through the decode kernels:
    every output against the oracle, and bit for bit against separate calls on
    each group of tokens, and across the workspace, pre-quantized, repacked and
    multi-matrix forms."""
    W, X = _case(rows, K, 32, 9700 + rows + K)
    Wq_o = orc.q4_0_quantize(W)
    Wq = hip.q4_0_quantize(dev(W))
    Wr = hip.q4_0_repack(Wq, K)
    for N in Ns:
        print("decode groups rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        Xt = dev(X[:N])
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        assert_close(Y, orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(X[:N]), K), "rows=%d K=%d N=%d" % (rows, K, N))
        parts = [host(hip.mul_mat_q4_0_q8_0_ex(Wq, dev(X[n0:min(N, n0 + 8)]), hip.workspace(rows, K, 8)))
                 for n0 in range(0, N, 8)]
        assert np.array_equal(Y, np.concatenate(parts, axis=0)), ("groups", rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y), (rows, K, N)
        assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(Wr, Xt)), Y), (rows, K, N)
        half = rows // 2 // 32 * 32
        Ys = hip.mul_mat_q4_0_q8_0_multi([Wq[:half], Wq[half:]], Xt)
        assert np.array_equal(np.concatenate([host(Ys[0]), host(Ys[1])], axis=1), Y), ("multi", rows, K, N)


@pytest.mark.parametrize("rows,K,N", [(4096, 4096, 512), (2000, 4160, 200)])
def test_prefill_split_k(hip, orc, rows, K, N):
    """Matrix-core kernel with K split into ranges (fewer than 256 workgroup
    tiles: 3 ranges of 44, 44 and 40 blocks; 4 of 34, 34, 34 and 28 over 130
    blocks and two token tiles, the second ragged): sampled rows against the
    oracle; the repacked weights, the pre-quantized input and the prepared form
    bit for bit; the fused LayerNorm + GELU form against the oracle."""
    print("split K rows=%d K=%d N=%d" % (rows, K, N), flush=True)
    W, X = _case(rows, K, N, 9900 + rows + K)
    sample = _sample_rows(rows, 300, 9901 + rows)
    Wq_o = orc.q4_0_quantize(W[sample])
    Xq_o = orc.q8_0_quantize(X)
    Wq = hip.q4_0_quantize(dev(W))
    del W
    Xt = dev(X)
    Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
    assert_close(Y[:, sample], orc.mul_mat_ref(Wq_o, Xq_o, K), "split K rows=%d K=%d N=%d" % (rows, K, N))
    assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(hip.q4_0_repack(Wq, K), Xt)), Y)
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, hip.q8_0_quantize(Xt), K)), Y)
    ws = hip.workspace(1, K, N)
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_prepared(Wq, hip.q4bq_quantize_activations(Xt, ws), N, K)), Y)
    gamma = inputs.random_matrix(9902, 1, K, 0.5)[0] + 1.0
    beta = inputs.random_matrix(9903, 1, K, 0.1)[0]
    bias = inputs.random_matrix(9904, 1, rows, 0.1)[0]
    Yf = host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, dev(gamma), dev(beta), 1e-5, dev(bias), hip.ACT_GELU, None))
    ref = orc.epilogue(orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(orc.layernorm(X, gamma, beta, 1e-5)), K),
                       bias=bias[sample], act=hip.ACT_GELU, mul=None)
    assert_close(Yf[:, sample], ref, "fused split K")


def test_prepared_workspace_sized_for_its_matrix(hip, orc):
    """The two-phase form with a workspace sized for the matrix it serves
    (q4bq_workspace_size(14336, K, 512): 256 workgroup tiles, no room for split
    sums) rather than for one row (whose size does hold such room): the
    activations fit, and the prepared product equals the operator bit for
    bit."""
    rows, K, N = 14336, 1024, 512
    W, X = _case(rows, K, N, 9950)
    Wq = hip.q4_0_quantize(dev(W))
    Xt = dev(X)
    ws = hip.workspace(rows, K, N)
    assert ws.numel() < hip.q4bq_workspace_size(1, K, N)
    Y = host(hip.mul_mat_q4_0_q8_0_prepared(Wq, hip.q4bq_quantize_activations(Xt, ws), N, K))
    assert np.array_equal(Y, host(hip.mul_mat_q4_0_q8_0(Wq, Xt)))


SET_CASES = [
    ("gpt2_layer", [(2304, 768), (768, 768), (3072, 768), (768, 3072)], True),
    ("llama3_8b_decode", [(4096, 4096), (14336, 4096), (4096, 14336)], True),
    ("ragged", [(37, 64), (1000, 2048), (2049, 1536), (5, 16384)], False),
    ("one", [(300, 4096)], True),
    ("odd_blocks", [(100, 96), (64, 4096)], False),        # K = 96: three blocks, the products one by one
    ("long_tokens", [(64, 32768), (64, 4096)], False),     # 1152 activation blocks: one by one
]


@pytest.mark.parametrize("name,shapes,same_bits", SET_CASES, ids=[c[0] for c in SET_CASES])
def test_product_set(hip, orc, name, shapes, same_bits):
    """Independent one-token products in one launch (mul_mat_q4_0_q8_0_set):
    every output against the oracle; on the GPT-2- and Llama-3-8B-shaped
    matrices (and a single product) bitwise equal to separate calls, which run
    the row kernel with the same chunks; sets the launch does not take (an odd
    block count, more than 1024 activation blocks in all) run one by one."""
    print("product set %s %s" % (name, shapes), flush=True)
    Ws = [_case(r, K, 1, 8100 + 13 * i + r + K)[0] for i, (r, K) in enumerate(shapes)]
    Xs = [inputs.random_matrix(8200 + 13 * i + K, 1, K) for i, (r, K) in enumerate(shapes)]
    Wqs = [hip.q4_0_quantize(dev(W)) for W in Ws]
    Xts = [dev(X) for X in Xs]
    Ys = hip.mul_mat_q4_0_q8_0_set(Wqs, Xts)
    for i, (r, K) in enumerate(shapes):
        Y = host(Ys[i])
        assert Y.shape == (1, r)
        assert_close(Y, orc.mul_mat_ref(orc.q4_0_quantize(Ws[i]), orc.q8_0_quantize(Xs[i]), K),
                     "set %s product %d" % (name, i))
        Y1 = host(hip.mul_mat_q4_0_q8_0(Wqs[i], Xts[i]))
        if same_bits:
            assert np.array_equal(Y, Y1), (name, i)
        else:
            assert_close(Y, Y1.astype(np.float64), "set %s product %d against its own call" % (name, i))


def test_matrix_core_decode_multi(hip, orc):
    """The multi-matrix form on the matrix cores: matrices starting on 32-row
    boundaries share its 32-row tiles' loop (a tile never spans two matrices);
    with a matrix that does not, the other kernels run; 32768 rows in all take
    six tokens on the matrix cores.  Every output against the oracle, with and
    without a workspace."""
    for K, shapes in ((4096, [2048, 1024, 1024]), (4096, [2048, 1000, 1024]), (2048, [16384, 8192, 8192])):
        Ws = [_case(r, K, 1, 6300 + 7 * r)[0] for r in shapes]
        X = inputs.random_matrix(6400, 8, K)
        Wqs = [hip.q4_0_quantize(dev(W)) for W in Ws]
        Wq_os = [orc.q4_0_quantize(W) for W in Ws]
        for N in (6, 8):
            print("matrix-core multi %s K=%d N=%d" % (shapes, K, N), flush=True)
            Xt = dev(X[:N])
            Xq_o = orc.q8_0_quantize(X[:N])
            Ys = hip.mul_mat_q4_0_q8_0_multi(Wqs, Xt)
            Ys_ws = hip.mul_mat_q4_0_q8_0_multi(Wqs, Xt, ws=hip.workspace(1, K, N))
            for i, r in enumerate(shapes):
                Y = host(Ys[i])
                assert np.array_equal(host(Ys_ws[i]), Y), (shapes, N, i)
                assert_close(Y, orc.mul_mat_ref(Wq_os[i], Xq_o, K), "multi %s N=%d matrix %d" % (shapes, N, i))


@pytest.mark.parametrize("rows,K,n", [(1, 32, 1), (37, 96, 50), (1000, 768, 7), (300, 4096, 513),
                                      (32768, 4096, 512)])
def test_get_rows(hip, orc, rows, K, n):
    """Decoded rows of a Q4_0 table, bit-exact against the oracle (every
    element (nibble - 8) * d is exact in fp32), with repeated, unordered and
    out-of-range ids (rows of NaN).  The last case is a 32768-row table drawn
    like the Llama-3-8B-shaped embedding table, with a 512-token batch."""
    if rows == 32768:
        W = inputs.weights(4, 0, rows, K)
    else:
        W = inputs.random_matrix(7000 + rows + K, rows, K, 0.02)
    rng = np.random.default_rng(rows + n)
    ids = rng.integers(-2, rows + 2, n).astype(np.int32)
    ids[: min(n, 3)] = [0, rows - 1, 0][: min(n, 3)]
    print("get_rows rows=%d K=%d n=%d" % (rows, K, n), flush=True)
    got = host(hip.q4_0_get_rows(hip.q4_0_quantize(dev(W)), K, dev(ids)))
    want = orc.q4_0_get_rows(orc.q4_0_quantize(W), K, ids)
    assert got.shape == (n, K)
    assert np.array_equal(got, want, equal_nan=True)
    bad = (ids < 0) | (ids >= rows)
    assert np.all(np.isnan(got[bad])) and not np.any(np.isnan(got[~bad]))


def test_unaligned_but_valid_pointers(hip, orc):
    """Q4_0 data may start on any 2-byte boundary, fp32 data on any 4-byte one."""
    rows, K, N = 65, 4096, 3
    W, X = _case(rows, K, N, 4242)
    Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
    nbytes = Wq_o.size
    buf = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    Wq_off = buf[2:2 + nbytes]                       # 2 mod 4 address
    hip.q4_0_quantize(dev(W), Wq_off)
    xbuf = torch.zeros(N * K + 4, dtype=torch.float32, device="cuda")
    X_off = xbuf[1:1 + N * K].view(N, K)             # 4 mod 16 address
    X_off.copy_(dev(X))
    assert np.array_equal(host(Wq_off).reshape(rows, -1), Wq_o)
    Yref = orc.mul_mat_ref(Wq_o, Xq_o, K)
    assert_close(host(hip.mul_mat_q4_0_q8_0(Wq_off, X_off)), Yref, "unaligned gemv")
    Xn = inputs.random_matrix(4343, 40, K)
    xbuf2 = torch.zeros(40 * K + 4, dtype=torch.float32, device="cuda")
    Xn_off = xbuf2[1:1 + 40 * K].view(40, K)
    Xn_off.copy_(dev(Xn))
    assert_close(host(hip.mul_mat_q4_0_q8_0(Wq_off, Xn_off)),
                 orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(Xn), K), "unaligned gemm")


def _e2m3_value(code):
    """FP6 E2M3 (OCP MX formats): sign bit, 2 exponent bits (bias 1), 3 mantissa bits."""
    s, e, m = code >> 5, (code >> 3) & 3, code & 7
    v = m / 8.0 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 1)
    return -v if s else v


def _repack_expected(Wq_h, rows, K):
    """The repacked byte layout, written out from its definition: every block's
    16 nibble bytes in block order, every block's 2 scale bytes, zero padding to
    a multiple of 256, then the block-major 32-byte records (24 bytes of E2M3
    codes of (nibble - 8)/8, code c at bits 6c, code 4m + i for element
    8(m//2) + 2i + m%2; the scale bytes; 6 zero bytes; 16-byte halves swapped
    in rows where bit 2 xor bit 3 is set) and one plane of zero records."""
    nb = K // 32
    blocks = Wq_h.reshape(rows * nb, 18)
    head = np.concatenate([blocks[:, 2:].reshape(-1), blocks[:, :2].reshape(-1)])
    R = (head.size + 255) // 256 * 256
    # element j of a block: nibble j % 2 of byte j // 2 (low first)
    nib = np.empty((rows * nb, 32), dtype=np.int64)
    nib[:, 0::2] = blocks[:, 2:] & 15
    nib[:, 1::2] = blocks[:, 2:] >> 4
    code_of = {}
    for code in range(64):
        code_of.setdefault(_e2m3_value(code), code)  # +0 before -0
    lut = np.array([code_of[(n - 8) / 8.0] for n in range(16)], dtype=np.uint8)
    c = np.arange(32)
    elem = 8 * ((c // 4) // 2) + 2 * (c % 4) + (c // 4) % 2
    codes = lut[nib[:, elem]]
    bits = ((codes[:, :, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(-1, 192)
    rec = np.zeros((rows * nb, 32), dtype=np.uint8)
    rec[:, :24] = np.packbits(bits, axis=1, bitorder="little")
    rec[:, 24:26] = blocks[:, :2]
    rec = rec.reshape(rows, nb, 32)
    r = np.arange(rows)
    swap = (((r >> 2) ^ (r >> 3)) & 1) != 0
    rec[swap] = np.concatenate([rec[swap][:, :, 16:], rec[swap][:, :, :16]], axis=2)
    planes = np.zeros((nb + 1, rows, 32), dtype=np.uint8)
    planes[:nb] = rec.transpose(1, 0, 2)
    return np.concatenate([head, np.zeros(R - head.size, dtype=np.uint8), planes.reshape(-1)])


@pytest.mark.parametrize("rows,K", [(1, 32), (5, 96), (129, 160), (300, 768), (1000, 4096)])
def test_repacked_weights(hip, orc, rows, K):
    """q4_0_repack moves bytes only, and the product on the repacked weights
    gives exactly the bits of the product on the blocks, decode and prefill."""
    W, X = _case(rows, K, 130, 777 + rows + K)
    Wq = hip.q4_0_quantize(dev(W))
    Wr = hip.q4_0_repack(Wq, K)
    assert np.array_equal(host(Wr), _repack_expected(host(Wq), rows, K)), (rows, K)
    Wq_o = orc.q4_0_quantize(W)
    for N in (1, 2, 3, 8, 9, 64, 130):
        print("repacked rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        Xt = dev(X[:N])
        Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
        Yr = host(hip.mul_mat_q4_0r_q8_0(Wr, Xt))
        Yx = host(hip.mul_mat_q4_0r_q8_0_ex(Wr, Xt, hip.workspace(rows, K, N)))
        assert np.array_equal(Yr, Y), (rows, K, N)
        assert np.array_equal(Yx, Y), (rows, K, N)
        assert_close(Yr, orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(X[:N]), K), "repacked N=%d" % N)


@pytest.mark.parametrize("K", [96, 768, 4096])
def test_multi_matrix(hip, orc, K):
    """Several matrices sharing one token matrix: every output matches the
    oracle; above 8 tokens it is the single-matrix result bit for bit."""
    shapes = [300, 77, 77, 1000]
    Ws = [_case(r, K, 1, 3100 + 7 * r + K)[0] for r in shapes]
    X = inputs.random_matrix(3200 + K, 70, K)
    Wqs = [hip.q4_0_quantize(dev(W)) for W in Ws]
    Wq_os = [orc.q4_0_quantize(W) for W in Ws]
    for N in (1, 2, 5, 8, 9, 70):
        print("multi K=%d N=%d" % (K, N), flush=True)
        Xt = dev(X[:N])
        Xq_o = orc.q8_0_quantize(X[:N])
        Ys = hip.mul_mat_q4_0_q8_0_multi(Wqs, Xt)
        Ys_ws = hip.mul_mat_q4_0_q8_0_multi(Wqs, Xt, ws=hip.workspace(1, K, N))
        for i, r in enumerate(shapes):
            Y = host(Ys[i])
            assert Y.shape == (N, r)
            assert np.array_equal(host(Ys_ws[i]), Y), (K, N, i)
            assert_close(Y, orc.mul_mat_ref(Wq_os[i], Xq_o, K), "multi K=%d N=%d matrix %d" % (K, N, i))
            if N > 8:
                assert np.array_equal(Y, host(hip.mul_mat_q4_0_q8_0(Wqs[i], Xt))), (K, N, i)


def test_multi_matrix_llama_decode_full_size(hip, orc):
    """The two K = 4096 matrices of the Llama decode set in one launch, at full
    size, N = 1 and 4, outputs sampled against the oracle."""
    wl = inputs.WORKLOADS[3]
    mats = [(m, rk) for m, rk in enumerate(wl.mats) if rk[1] == 4096]
    Wqs, Wq_os, samples = [], [], []
    for m, (rows, K) in mats:
        W = inputs.weights(3, m, rows, K, outliers=wl.outliers)
        Wqs.append(hip.q4_0_quantize(dev(W)))
        samples.append(_sample_rows(rows, 1024, 9500 + m))
        Wq_os.append(orc.q4_0_quantize(W[samples[-1]]))
        del W
    X = inputs.activations(3, 0, max(wl.ns), 4096)
    for N in wl.ns:
        print("multi llama decode N=%d" % N, flush=True)
        Xq_o = orc.q8_0_quantize(X[:N])
        Ys = hip.mul_mat_q4_0_q8_0_multi(Wqs, dev(X[:N]))
        for i in range(len(mats)):
            assert_close(host(Ys[i])[:, samples[i]], orc.mul_mat_ref(Wq_os[i], Xq_o, 4096), "multi N=%d" % N)


# ---------------------------------------------------------------------------
# Q8_0 weights (Q8_0 weight blocks, from the same Q8_0 rule as the activations)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rows,K,N", [(1, 32, 1), (37, 96, 3), (300, 768, 9), (129, 4096, 2), (5, 20480, 3)])
def test_q8w_block_dots(hip, orc, rows, K, N):
    """Q8_0 weight bytes and every per-block int32 dot, bit for bit."""
    W, X = _case(rows, K, N, 4100 + rows + K)
    print("q8w block dots rows=%d K=%d N=%d" % (rows, K, N), flush=True)
    Wq8 = hip.q8_0_quantize(dev(W))
    Wq8_o = orc.q8_0_quantize(W)
    assert np.array_equal(host(Wq8).reshape(-1), Wq8_o.reshape(-1))
    Xq_o = orc.q8_0_quantize(X)
    D = host(hip.q8_0_q8_0_block_dots(Wq8, dev(Xq_o), K))
    assert np.array_equal(D, orc.block_dots_q8(Wq8_o, Xq_o, K))


Q8W_K = [32, 96, 768, 2048, 3072, 4096, 4128, 8192, 14336, 16384, 16416, 20480, 32768]


@pytest.mark.parametrize("K", Q8W_K)
def test_q8w_product(hip, orc, K):
    """Every lane-block count (1 to 16 per lane, ragged), token groups of 1..8
    and the grouping above 8 tokens (or above 2 on rows over 16384)."""
    rows = 301 if K <= 4128 else 67
    W, X = _case(rows, K, 17, 4200 + K)
    Wq8 = hip.q8_0_quantize(dev(W))
    Wq8_o = orc.q8_0_quantize(W)
    for N in (1, 2, 3, 5, 8, 9, 17):
        print("q8w product rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        Y = host(hip.mul_mat_q8_0_q8_0(Wq8, dev(X[:N])))
        assert Y.shape == (N, rows)
        assert_close(Y, orc.mul_mat_q8_ref(Wq8_o, orc.q8_0_quantize(X[:N]), K), "q8w K=%d N=%d" % (K, N))


@pytest.mark.parametrize("rows,K", [(14336, 4096), (4096, 14336)])
def test_q8w_full_size(hip, orc, rows, K):
    """Llama-size Q8_0 matrices at N = 1 and 8, in the benchmark's launch
    configuration; outputs sampled on the first, last and random rows."""
    W, X = _case(rows, K, 8, 4300 + rows)
    Wq8 = hip.q8_0_quantize(dev(W))
    Wq8_o = orc.q8_0_quantize(W)
    sample = np.unique(np.concatenate([[0, 1, rows - 1], np.random.default_rng(rows).integers(0, rows, 61)]))
    Ws = Wq8_o.reshape(rows, -1)[sample]
    for N in (1, 8):
        print("q8w full size rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        Y = host(hip.mul_mat_q8_0_q8_0(Wq8, dev(X[:N])))
        assert_close(Y[:, sample], orc.mul_mat_q8_ref(Ws, orc.q8_0_quantize(X[:N]), K), "q8w full N=%d" % N)


@pytest.mark.parametrize("rows,K,Ns", [(66000, 3072, (1, 2, 4, 8)), (70000, 4096, (1, 3, 8))])
def test_q8w_long_matrices_contiguous_row_loads(hip, orc, rows, K, Ns):
    """Q8_0 weights on matrices long enough for the contiguous row loads (16
    rows per wave or more): sampled rows against the oracle, and every row of
    a 20000-row prefix bit for bit against the product on that prefix alone
    (too few rows for that form: each lane loads its own blocks; the folds are
    the same)."""
    W, X = _case(rows, K, max(Ns), 4600 + rows)
    Wq8 = hip.q8_0_quantize(dev(W))
    sample = _sample_rows(rows, 200, 4601 + rows)
    Ws = orc.q8_0_quantize(W[sample])
    assert np.array_equal(host(Wq8)[sample], Ws.reshape(len(sample), -1))
    del W
    head = 20000
    for N in Ns:
        print("q8w contiguous row loads rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        Xn = dev(X[:N])
        Y = host(hip.mul_mat_q8_0_q8_0(Wq8, Xn))
        assert_close(Y[:, sample], orc.mul_mat_q8_ref(Ws, orc.q8_0_quantize(X[:N]), K), "q8w long N=%d" % N)
        Yh = host(hip.mul_mat_q8_0_q8_0(Wq8[:head], Xn))
        assert np.array_equal(Y[:, :head], Yh), ("prefix", rows, K, N)


@pytest.mark.parametrize("K", [32, 96, 160, 4096, 4128])
def test_q8w_many_tokens(hip, orc, K):
    """More than eight tokens (the int8 matrix-core kernel): ragged row and token
    tiles, block counts that are not a multiple of the 4-block stage, the
    oracle bar on Y and every block dot bit for bit."""
    for rows in (1, 129, 300):
        for N in (9, 64, 130, 257):
            if rows * K * N > 20_000_000:
                continue
            print("q8w many tokens rows=%d K=%d N=%d" % (rows, K, N), flush=True)
            W, X = _case(rows, K, N, 4400 + rows + K + N)
            Wq8 = hip.q8_0_quantize(dev(W))
            Wq8_o = orc.q8_0_quantize(W)
            Xq_o = orc.q8_0_quantize(X)
            Y = host(hip.mul_mat_q8_0_q8_0(Wq8, dev(X)))
            assert Y.shape == (N, rows)
            assert_close(Y, orc.mul_mat_q8_ref(Wq8_o, Xq_o, K), "q8w rows=%d K=%d N=%d" % (rows, K, N))
            D = host(hip.q8_0_q8_0_block_dots(Wq8, dev(Xq_o), K))
            assert np.array_equal(D, orc.block_dots_q8(Wq8_o, Xq_o, K)), (rows, K, N)


def test_q8w_prefill_full_size(hip, orc):
    """Q8_0 weights 14336 x 4096 against 512 tokens (the prefill shape), in the
    benchmark's launch configuration; outputs sampled on the first, last and
    random rows for every token, block dots sampled."""
    rows, K, N = 14336, 4096, 512
    W = inputs.weights(5, 0, rows, K)
    X = inputs.activations(5, 0, N, K)
    Wq8 = hip.q8_0_quantize(dev(W))
    sample = _sample_rows(rows, 512, 4500)
    Wq8_o = orc.q8_0_quantize(W[sample])
    Xq_o = orc.q8_0_quantize(X)
    print("q8w prefill full size", flush=True)
    Y = host(hip.mul_mat_q8_0_q8_0(Wq8, dev(X)))
    assert_close(Y[:, sample], orc.mul_mat_q8_ref(Wq8_o, Xq_o, K), "q8w prefill")
    Dg = hip.q8_0_q8_0_block_dots(Wq8, dev(Xq_o), K)
    tok = np.unique(np.r_[0, N - 1, np.arange(1, N, 37)])
    Ds = host(Dg.index_select(0, torch.from_numpy(tok).cuda()).index_select(1, torch.from_numpy(sample).cuda()))
    assert np.array_equal(Ds, orc.block_dots_q8(Wq8_o, Xq_o[tok], K))


# ---------------------------------------------------------------------------
# the steps around the product: LayerNorm before it, bias / activation /
# element-wise factor after it, SwiGLU
# ---------------------------------------------------------------------------

def _fusion_inputs(rows, K, N, seed):
    W, X = _case(rows, K, N, seed)
    X = X * 3.0 + 1.5                                   # a mean and scale for the LayerNorm to remove
    gamma = inputs.random_matrix(seed + 10, 1, K, 0.5)[0] + 1.0
    beta = inputs.random_matrix(seed + 11, 1, K, 0.1)[0]
    bias = inputs.random_matrix(seed + 12, 1, rows, 0.1)[0]
    mul = inputs.random_matrix(seed + 13, N, rows)
    return W, X.astype(np.float32), gamma, beta, bias, mul


# decode task kernel (K = 768), row kernel (K = 4096), groups of 8 tokens through
# the decode kernels (N = 9), prefill kernel (N = 130)
@pytest.mark.parametrize("rows,K,N", [(3072, 768, 1), (3072, 768, 4), (2304, 768, 6), (300, 4096, 1), (300, 4096, 5),
                                      (1000, 4096, 9), (777, 768, 130)])
def test_fused_product(hip, orc, rows, K, N):
    W, X, gamma, beta, bias, mul = _fusion_inputs(rows, K, N, 5100 + rows + K + N)
    eps = 1e-5
    Wq = hip.q4_0_quantize(dev(W))
    Wq_o = orc.q4_0_quantize(W)
    Xt, gt, bt, bit, mt = dev(X), dev(gamma), dev(beta), dev(bias), dev(mul)
    Y_plain = orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(X), K)
    Y_ln = orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(orc.layernorm(X, gamma, beta, eps)), K)
    cases = [(False, None, hip.ACT_NONE, None), (True, None, hip.ACT_NONE, None),
             (True, bias, hip.ACT_GELU, None), (False, bias, hip.ACT_SILU, None),
             (True, None, hip.ACT_SILU, mul), (False, bias, hip.ACT_NONE, mul)]
    for ln, b, act, m in cases:
        print("fused rows=%d K=%d N=%d ln=%d bias=%d act=%d mul=%d"
              % (rows, K, N, ln, b is not None, act, m is not None), flush=True)
        Y = host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, gt if ln else None, bt if ln else None, eps,
                                             bit if b is not None else None, act, mt if m is not None else None))
        ref = orc.epilogue(Y_ln if ln else Y_plain, bias=b, act=act, mul=m)
        assert_close(Y, ref, "fused ln=%d act=%d" % (ln, act))
    # nothing fused: the same bits as the operator
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt)), host(hip.mul_mat_q4_0_q8_0(Wq, Xt)))
    # a caller's workspace gives the same bits
    ws = hip.fused_workspace(rows, K, N)
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, gt, bt, eps, bit, hip.ACT_GELU, mt, ws=ws)),
                          host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, gt, bt, eps, bit, hip.ACT_GELU, mt)))
    # the factor read in place
    Yo = host(hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, gt, bt, eps, None, hip.ACT_SILU, mt))
    Yi = mt.clone()
    hip.mul_mat_q4_0_q8_0_fused(Wq, Xt, gt, bt, eps, None, hip.ACT_SILU, Yi, Y=Yi)
    assert np.array_equal(host(Yi), Yo)


@pytest.mark.parametrize("K", [32, 768, 4096, 8192, 14336, 32768, 40960])
def test_fused_layernorm_k_sweep(hip, orc, K):
    """The LayerNorm + quantization kernel at every register layout (1, 2, 4, 8
    quads per thread, and re-reading above 32768 values), into both activation
    layouts: the decode kernels' (N = 1, and N = 11 as groups of 8 and 3 tokens
    where a decode kernel takes the rows) and the prefill kernel's (N = 11 at
    K = 32 and K >= 32768)."""
    rows = 37
    W, X, gamma, beta, _, _ = _fusion_inputs(rows, K, 11, 5700 + K)
    Wq = hip.q4_0_quantize(dev(W))
    Wq_o = orc.q4_0_quantize(W)
    for N in (1, 11):
        print("fused layernorm K=%d N=%d" % (K, N), flush=True)
        Y = host(hip.mul_mat_q4_0_q8_0_fused(Wq, dev(X[:N]), dev(gamma), dev(beta), 1e-5))
        ref = orc.mul_mat_ref(Wq_o, orc.q8_0_quantize(orc.layernorm(X[:N], gamma, beta, 1e-5)), K)
        assert_close(Y, ref, "layernorm K=%d N=%d" % (K, N))


@pytest.mark.parametrize("rows,K,N", [(1000, 4096, 1), (1000, 4096, 3), (600, 768, 2), (2048, 4096, 7),
                                      (300, 4096, 40)])
def test_swiglu(hip, orc, rows, K, N):
    Wg, X, gamma, beta, _, _ = _fusion_inputs(rows, K, N, 5300 + rows + N)
    Wu = _case(rows, K, 1, 5400 + rows)[0]
    eps = 1e-6
    print("swiglu rows=%d K=%d N=%d" % (rows, K, N), flush=True)
    H = host(hip.mul_mat_q4_0_q8_0_swiglu(hip.q4_0_quantize(dev(Wg)), hip.q4_0_quantize(dev(Wu)), dev(X),
                                          dev(gamma), dev(beta), eps))
    Xq = orc.q8_0_quantize(orc.layernorm(X, gamma, beta, eps))
    g = orc.epilogue(orc.mul_mat_ref(orc.q4_0_quantize(Wg), Xq, K), act=orc.ACT_SILU)
    ref = orc.epilogue(orc.mul_mat_ref(orc.q4_0_quantize(Wu), Xq, K), mul=g)
    assert_close(H, ref, "swiglu N=%d" % N)


def test_swiglu_llama_full_size(hip, orc):
    """The Llama-3-8B feed-forward's gate and up matrices (14336 x 4096) at one
    token, sampled rows."""
    rows, K = 14336, 4096
    Wg = inputs.weights(3, 1, rows, K, outliers=True)   # the workload's 14336 x 4096 matrix as the gate
    Wu = inputs.weights(3, 4, rows, K, outliers=True)   # an up matrix of the same shape, its own seed
    X = inputs.activations(3, 0, 1, K)
    gamma = inputs.random_matrix(5500, 1, K, 0.5)[0] + 1.0
    beta = inputs.random_matrix(5501, 1, K, 0.1)[0]
    H = host(hip.mul_mat_q4_0_q8_0_swiglu(hip.q4_0_quantize(dev(Wg)), hip.q4_0_quantize(dev(Wu)), dev(X),
                                          dev(gamma), dev(beta), 1e-5))
    sample = np.unique(np.concatenate([[0, rows - 1], np.random.default_rng(7).integers(0, rows, 62)]))
    Xq = orc.q8_0_quantize(orc.layernorm(X, gamma, beta, 1e-5))
    g = orc.epilogue(orc.mul_mat_ref(orc.q4_0_quantize(Wg[sample]), Xq, K), act=orc.ACT_SILU)
    ref = orc.epilogue(orc.mul_mat_ref(orc.q4_0_quantize(Wu[sample]), Xq, K), mul=g)
    assert_close(H[:, sample], ref, "swiglu llama")


def test_repack_rejects_misaligned_output(hip):
    Wq = torch.zeros((4, 36), dtype=torch.uint8, device="cuda")
    buf = torch.zeros(4 * 36 + 32, dtype=torch.uint8, device="cuda")
    with pytest.raises(hip.Q4BQError) as e:
        hip.q4_0_repack(Wq, 64, buf[8:8 + 4 * 36])
    assert e.value.status == hip.Q4BQ_EINVAL


def test_empty_inputs_are_rejected(hip):
    Wq = torch.zeros((4, 36), dtype=torch.uint8, device="cuda")
    with pytest.raises(hip.Q4BQError) as e:
        hip.mul_mat_q4_0_q8_0(Wq, torch.zeros((0, 64), dtype=torch.float32, device="cuda"))
    assert e.value.status == hip.Q4BQ_EINVAL


# ---------------------------------------------------------------------------
# the five workloads at full size, in the benchmark's launch configuration
# ---------------------------------------------------------------------------

def _sample_rows(rows, n, seed):
    rng = np.random.default_rng(seed)
    pick = np.concatenate([np.arange(min(rows, 256)), np.arange(max(0, rows - 256), rows),
                           rng.integers(0, rows, n)])
    return np.unique(pick)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_full_size(hip, orc, cid):
    wl = inputs.WORKLOADS[cid]
    nmax = max(wl.ns)
    for m, (rows, K) in enumerate(wl.mats):
        print("workload %s matrix %d (%d x %d)" % (wl.name, m, rows, K), flush=True)
        W = inputs.weights(cid, m, rows, K, outliers=wl.outliers)
        X = inputs.activations(cid, m, nmax, K)
        Wt = dev(W)
        Wq = hip.q4_0_quantize(Wt)
        del Wt
        sample = _sample_rows(rows, 2048, 9000 + cid * 10 + m) if rows * K > 20_000_000 else np.arange(rows)
        Wq_o = orc.q4_0_quantize(W[sample])
        del W
        Wq_h = host(Wq)
        assert np.array_equal(Wq_h[sample], Wq_o), "Q4_0 bytes differ"
        for N in wl.ns:
            Xt = dev(X[:N])
            Xq = hip.q8_0_quantize(Xt)
            Xq_o = orc.q8_0_quantize(X[:N])
            assert np.array_equal(host(Xq), Xq_o), "Q8_0 bytes differ"
            ws = hip.workspace(rows, K, N)
            Y = host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, ws))
            assert_close(Y[:, sample], orc.mul_mat_ref(Wq_o, Xq_o, K), "%s N=%d" % (wl.name, N))
            # the repacked weights give the same bits
            Wr = hip.q4_0_repack(Wq, K)
            assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0_ex(Wr, Xt, ws)), Y), "%s N=%d repacked" % (wl.name, N)
            del Wr
            # block dots on a sample of outputs
            tok = np.arange(N) if N <= 8 else np.unique(np.r_[0, N - 1, np.arange(1, N, 37)])
            Dg = hip.q4_0_q8_0_block_dots(Wq, Xq, K)
            idx_r = torch.from_numpy(sample).cuda()
            idx_t = torch.from_numpy(tok).cuda()
            Ds = host(Dg.index_select(0, idx_t).index_select(1, idx_r))
            del Dg
            assert np.array_equal(Ds, orc.block_dots(Wq_o, Xq_o[tok], K)), "block dots differ"
        del Wq
        torch.cuda.empty_cache()
