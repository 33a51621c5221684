"""Zero and subnormal block scales through every product kernel.

The scale of a block is a stored binary16 ("llama.cpp 深度解读", section 2: the
block_q4_0 struct keeps d as fp16; the Q8_0 activation block of section 3 does
the same), so d_w or d_x can be zero (an all-zero block, or amax/8 below half
the smallest subnormal) or an fp16 subnormal (weights with amax < 8 * 2^-14 =
4.9e-4, activations with amax < 127 * 2^-14 = 7.8e-3).  These tests feed such
blocks to the decode row kernel (K = 4096, 14336), the decode task kernel
(K = 768) and the matrix-core kernel (N = 9, 130, 512) on both weight layouts,
the fused and multi-matrix forms and the block-dot exports, against the oracle:

  * block dots bit-exact;
  * Y within |Y - Y_ref| <= 1e-4 |Y_ref| + 1e-5 (the operator's bar), on inputs
    where a tiny block meets a large one, so its contribution is far above
    1e-5;
  * on inputs where BOTH operands are subnormal-scaled everywhere (|Y| around
    1e-5), the same bar applied to Y / max|Y_ref|, so that a flushed scale
    product cannot hide under the absolute term.

All inputs are seeded and synthetic; the oracle quantizes its own copy.
"""
import numpy as np
import pytest
import torch

from q4_block_quantized_amd import inputs

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-5

# Per-block magnitudes (multipliers of N(0, 1) values).  Tiny weights: 0 and
# 1e-9 give d_w = 0, 1e-4 and 3e-5 an fp16-subnormal d_w; tiny activations: 0
# and 1e-9 give d_x = 0, 1e-3 and 2e-3 a subnormal d_x.
W_TINY = np.array([0.0, 1e-9, 1e-4, 3e-5], np.float32)
X_TINY = np.array([0.0, 1e-9, 1e-3, 2e-3], np.float32)


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


def assert_close(Y, Yref, what, scale=1.0):
    """The operator's bar on Y / scale (scale = 1: the bar itself)."""
    Y = Y.astype(np.float64) / scale
    Yref = Yref / scale
    err = np.abs(Y - Yref)
    lim = RTOL * np.abs(Yref) + ATOL
    bad = err > lim
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside tolerance; first at %s: got %r want %r (scale %g)"
                             % (what, int(bad.sum()), Y.size, i, Y[i] * scale, Yref[i] * scale, scale))


def mixed_scales(rows, K, N, seed):
    """W (rows x K) and X (N x K) with zero and subnormal block scales whose
    contributions are all visible: every block index b has one regime, shared
    by all rows and tokens of this K -- tiny weights against activations of
    magnitude 300, weights of magnitude 50 against tiny activations, or the
    workloads' 0.02 against 1 -- so every block term is of order 0.1 to 1 (a
    flushed subnormal scale moves Y by far more than the bar, and no term
    dwarfs the sum, which an fp32 accumulation could not follow).  Row 0 and
    (N >= 3) token 0 are all zero; row 1 and (N >= 2) token 1 are tiny in
    every block."""
    nb = K // 32
    regime = np.random.default_rng(K).choice(3, size=nb, p=[0.25, 0.25, 0.5])
    rng = np.random.default_rng(seed)
    W = inputs.random_matrix(seed, rows, K, 1.0)
    X = inputs.random_matrix(seed + 1, N, K, 1.0)
    wl = np.where(regime == 0, rng.choice(W_TINY, size=(rows, nb)), np.where(regime == 1, 50.0, 0.02))
    xl = np.where(regime == 0, 300.0, np.where(regime == 1, rng.choice(X_TINY, size=(N, nb)), 1.0))
    wl[0] = 0.0
    if rows > 1:
        wl[1] = rng.choice(W_TINY[2:], size=nb)
    if N >= 3:
        xl[0] = 0.0
    if N >= 2:
        xl[1] = rng.choice(X_TINY[2:], size=nb)
    W *= np.repeat(wl.astype(np.float32), 32, axis=1)
    X *= np.repeat(xl.astype(np.float32), 32, axis=1)
    return W.astype(np.float32), X.astype(np.float32)


def all_subnormal(rows, K, N, seed):
    """Every weight block and every activation block with an fp16-subnormal
    scale."""
    rng = np.random.default_rng(seed)
    nb = K // 32
    W = inputs.random_matrix(seed, rows, K, 1.0) * np.repeat(rng.choice(W_TINY[2:], size=(rows, nb)), 32, axis=1)
    X = inputs.random_matrix(seed + 1, N, K, 1.0) * np.repeat(rng.choice(X_TINY[2:], size=(N, nb)), 32, axis=1)
    return W.astype(np.float32), X.astype(np.float32)


def _scale_kinds(Bq, nbytes):
    d = Bq.reshape(-1, nbytes)[:, 0:2].copy().view(np.float16)[:, 0]
    a = np.abs(d.astype(np.float64))
    return int((a == 0).sum()), int(((a > 0) & (a < 2.0 ** -14)).sum()), int((a >= 2.0 ** -14).sum())


def _check(hip, orc, W, X, what, scaled=False, repacked=True, dots=True):
    rows, K = W.shape
    N = X.shape[0]
    Wq_o, Xq_o = orc.q4_0_quantize(W), orc.q8_0_quantize(X)
    zw, sw, _ = _scale_kinds(Wq_o, 18)
    zx, sx, _ = _scale_kinds(Xq_o, 34)
    assert sw > 0 and sx > 0, "the inputs must hold subnormal scales on both sides"
    if not scaled:
        assert zw > 0 and zx > 0, "the inputs must hold zero scales on both sides"
    Wq = hip.q4_0_quantize(dev(W))
    Xt = dev(X)
    Xq = hip.q8_0_quantize(Xt)
    assert np.array_equal(host(Wq).reshape(-1), Wq_o.reshape(-1)), what
    assert np.array_equal(host(Xq).reshape(-1), Xq_o.reshape(-1)), what
    Yref = orc.mul_mat_ref(Wq_o, Xq_o, K)
    scale = float(np.abs(Yref).max()) if scaled else 1.0
    assert scale > 0
    Y = host(hip.mul_mat_q4_0_q8_0(Wq, Xt))
    assert_close(Y, Yref, what, scale)
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_pq(Wq, Xq, K)), Y), what
    assert np.array_equal(host(hip.mul_mat_q4_0_q8_0_ex(Wq, Xt, hip.workspace(rows, K, N))), Y), what
    if repacked:
        Wr = hip.q4_0_repack(Wq, K)
        assert np.array_equal(host(hip.mul_mat_q4_0r_q8_0(Wr, Xt)), Y), what + " repacked"
    if dots:
        assert np.array_equal(host(hip.q4_0_q8_0_block_dots(Wq, Xq, K)), orc.block_dots(Wq_o, Xq_o, K)), what
    return Wq, Wq_o, Yref


# decode row kernel (K = 4096 / 14336, N = 1..8), decode task kernel (K = 768),
# matrix-core kernel (N > 8)
@pytest.mark.parametrize("rows,K,Ns", [(300, 4096, (1, 2, 3, 4, 8)), (70, 14336, (1, 4, 8)),
                                       (257, 768, (1, 2, 5, 8)), (300, 4096, (9, 130, 512))])
def test_mixed_zero_and_subnormal_scales(hip, orc, rows, K, Ns):
    for N in Ns:
        print("mixed scales rows=%d K=%d N=%d" % (rows, K, N), flush=True)
        W, X = mixed_scales(rows, K, N, 61000 + rows + K + N)
        _check(hip, orc, W, X, "mixed rows=%d K=%d N=%d" % (rows, K, N))


@pytest.mark.parametrize("rows,K,N", [(129, 4096, 1), (129, 4096, 8), (65, 14336, 3), (100, 768, 4),
                                      (129, 4096, 9), (230, 4096, 130)])
def test_all_subnormal_scales(hip, orc, rows, K, N):
    print("all subnormal rows=%d K=%d N=%d" % (rows, K, N), flush=True)
    W, X = all_subnormal(rows, K, N, 62000 + rows + K + N)
    _check(hip, orc, W, X, "subnormal rows=%d K=%d N=%d" % (rows, K, N), scaled=True)


@pytest.mark.parametrize("N", [1, 4, 9, 70])
def test_multi_and_fused_with_edge_scales(hip, orc, N):
    """The multi-matrix form (one decode launch over concatenated rows, or one
    matrix-core launch per matrix) and the fused form (bias and SiLU in the
    store) on the same edge-scale inputs."""
    K = 4096
    shapes = [300, 129]
    Ws = [mixed_scales(r, K, N, 63000 + r + N)[0] for r in shapes]
    X = mixed_scales(2, K, N, 63500 + N)[1]
    Xq_o = orc.q8_0_quantize(X)
    Wqs = [hip.q4_0_quantize(dev(W)) for W in Ws]
    Xt = dev(X)
    print("multi edge scales N=%d" % N, flush=True)
    Ys = hip.mul_mat_q4_0_q8_0_multi(Wqs, Xt)
    for i, W in enumerate(Ws):
        Wq_o = orc.q4_0_quantize(W)
        Yref = orc.mul_mat_ref(Wq_o, Xq_o, K)
        assert_close(host(Ys[i]), Yref, "multi N=%d matrix %d" % (N, i))
        bias = inputs.random_matrix(63900 + i, 1, W.shape[0], 0.1)[0]
        print("fused edge scales N=%d matrix %d" % (N, i), flush=True)
        Yf = host(hip.mul_mat_q4_0_q8_0_fused(Wqs[i], Xt, None, None, 0.0, dev(bias), hip.ACT_SILU, None))
        assert_close(Yf, orc.epilogue(Yref, bias=bias, act=orc.ACT_SILU), "fused N=%d matrix %d" % (N, i))


@pytest.mark.parametrize("rows,K,N", [(300, 4096, 1), (300, 4096, 8), (257, 768, 9), (300, 4096, 130)])
def test_q8_0_weights_with_edge_scales(hip, orc, rows, K, N):
    """Q8_0 weights (the same binary16 block scale) with zero and subnormal
    scales on both sides, through the decode kernel (N <= 8) and the int8
    matrix-core kernel (N > 8): Y against the oracle and the block dots."""
    print("q8_0 weights edge scales rows=%d K=%d N=%d" % (rows, K, N), flush=True)
    W, X = mixed_scales(rows, K, N, 65000 + rows + K + N)
    Wq8_o, Xq_o = orc.q8_0_quantize(W), orc.q8_0_quantize(X)
    assert _scale_kinds(Wq8_o, 34)[1] > 0 and _scale_kinds(Xq_o, 34)[1] > 0
    Wq8 = hip.q8_0_quantize(dev(W))
    assert np.array_equal(host(Wq8).reshape(-1), Wq8_o.reshape(-1))
    Y = host(hip.mul_mat_q8_0_q8_0(Wq8, dev(X)))
    assert_close(Y, orc.mul_mat_q8_ref(Wq8_o, Xq_o, K), "q8w edge N=%d" % N)
    assert np.array_equal(host(hip.q8_0_q8_0_block_dots(Wq8, dev(Xq_o), K)), orc.block_dots_q8(Wq8_o, Xq_o, K))


@pytest.mark.parametrize("N", [1, 3, 11])
def test_layernorm_mean_off_the_fp32_grid(hip, orc, N):
    """Tokens whose mean is not an fp32 value (4096 plus a few fp32 ulps on a
    few elements): the fused LayerNorm must take its statistics in fp64, as the
    oracle does, to land on the same Q8_0 codes."""
    rows, K = 300, 4096
    rng = np.random.default_rng(64000 + N)
    X = np.full((N, K), 4096.0, np.float32)
    for n in range(N):
        idx = rng.choice(K, size=5 + n, replace=False)
        X[n, idx] += np.float32(2.0 ** -11) * rng.integers(1, 4, idx.size).astype(np.float32)
    W = inputs.random_matrix(64100 + N, rows, K, 0.02)
    gamma, beta = np.ones(K, np.float32), np.zeros(K, np.float32)
    print("layernorm off-grid mean N=%d" % N, flush=True)
    Wq = hip.q4_0_quantize(dev(W))
    Y = host(hip.mul_mat_q4_0_q8_0_fused(Wq, dev(X), dev(gamma), dev(beta), 0.0))
    Xn = orc.layernorm(X, gamma, beta, 0.0)
    Yref = orc.mul_mat_ref(orc.q4_0_quantize(W), orc.q8_0_quantize(Xn), K)
    assert_close(Y, Yref, "layernorm N=%d" % N)
