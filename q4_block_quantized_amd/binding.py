"""Python binding of libq4bq.so: argument marshalling only.

Every function has the name of the C entry point it calls (include/q4bq.h),
takes torch tensors that live on the current HIP device, passes their raw
pointers and the current torch stream, and raises ``Q4BQError`` on a non-zero
status.  All arithmetic happens in the library's HIP kernels; a missing or
unloadable library raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4bq.so")

QK = 32
Q4_0_BYTES = 18
Q8_0_BYTES = 34

Q4BQ_OK = 0
Q4BQ_EINVAL = -1
Q4BQ_EHIP = -2
Q4BQ_ENOMEM = -3
Q4BQ_ESCRATCH = -4
NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

EXPORTS = (
    "q4_0_quantize", "q8_0_quantize", "mul_mat_q4_0_q8_0", "q4bq_workspace_size",
    "mul_mat_q4_0_q8_0_ex", "mul_mat_q4_0_q8_0_pq", "q4_0_q8_0_block_dots",
    "q4bq_status_string", "q4bq_version", "q4bq_quantize_activations", "mul_mat_q4_0_q8_0_prepared",
    "q4_0_repack", "mul_mat_q4_0r_q8_0", "mul_mat_q4_0r_q8_0_ex", "mul_mat_q4_0_q8_0_multi", "mul_mat_q4_0_q8_0_set",
    "q4_0_get_rows", "q4bq_repack_size", "mul_mat_q8_0_q8_0", "q8_0_q8_0_block_dots",
    "mul_mat_q4_0_q8_0_fused", "mul_mat_q4_0_q8_0_swiglu", "q4bq_fused_workspace_size",
    "mul_mat_q4_0_q8_0_noalloc",
)

ACT_NONE, ACT_GELU, ACT_SILU = 0, 1, 2


class Q4BQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %d (%s)" % (where, status, status_string(status)))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library, with argument and result types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libq4bq.so is not built (%s); run `python -m q4_block_quantized_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "q4_0_quantize": (I, [P, I64, I64, P, P]),
        "q8_0_quantize": (I, [P, I64, I64, P, P]),
        "mul_mat_q4_0_q8_0": (I, [P, I64, I64, P, I64, P, P]),
        "mul_mat_q4_0_q8_0_noalloc": (I, [P, I64, I64, P, I64, P, P]),
        "q4bq_workspace_size": (ctypes.c_size_t, [I64, I64, I64]),
        "mul_mat_q4_0_q8_0_ex": (I, [P, I64, I64, P, I64, P, P, ctypes.c_size_t, P]),
        "mul_mat_q4_0_q8_0_pq": (I, [P, I64, I64, P, I64, P, P]),
        "q4_0_repack": (I, [P, I64, I64, P, P]),
        "q4bq_repack_size": (ctypes.c_size_t, [I64, I64]),
        "mul_mat_q8_0_q8_0": (I, [P, I64, I64, P, I64, P, P]),
        "mul_mat_q4_0_q8_0_fused": (I, [P, I64, I64, P, I64, P, P, ctypes.c_float, P, I, P, P, P, ctypes.c_size_t,
                                        P]),
        "mul_mat_q4_0_q8_0_swiglu": (I, [P, P, I64, I64, P, I64, P, P, ctypes.c_float, P, P, ctypes.c_size_t, P]),
        "q4bq_fused_workspace_size": (ctypes.c_size_t, [I64, I64, I64]),
        "q8_0_q8_0_block_dots": (I, [P, I64, I64, P, I64, P, P]),
        "q4_0_get_rows": (I, [P, I64, I64, P, I64, P, P]),
        "mul_mat_q4_0_q8_0_multi": (I, [ctypes.c_int, P, P, I64, P, I64, P, P, ctypes.c_size_t, P]),
        "mul_mat_q4_0_q8_0_set": (I, [ctypes.c_int, P, P, P, P, P, P]),
        "mul_mat_q4_0r_q8_0": (I, [P, I64, I64, P, I64, P, P]),
        "mul_mat_q4_0r_q8_0_ex": (I, [P, I64, I64, P, I64, P, P, ctypes.c_size_t, P]),
        "q4_0_q8_0_block_dots": (I, [P, I64, I64, P, I64, P, P]),
        "q4bq_quantize_activations": (I, [P, I64, I64, P, ctypes.c_size_t, P]),
        "mul_mat_q4_0_q8_0_prepared": (I, [P, I64, I64, P, I64, P, P]),
        "q4bq_status_string": (ctypes.c_char_p, [I]),
        "q4bq_version": (I, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().q4bq_status_string(int(status)).decode()


def _check(rc: int, where: str) -> None:
    if rc != Q4BQ_OK:
        raise Q4BQError(rc, where)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _nb(K: int) -> int:
    if K < QK or K % QK:
        raise ValueError("K must be a positive multiple of 32, got %d" % K)
    return K // QK


# --- entry points -------------------------------------------------------------

def q4_0_quantize(W: torch.Tensor, Wq: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 rows x K -> uint8 rows x (K/32*18) Q4_0 blocks."""
    rows, K = W.shape
    nb = _nb(K)
    if Wq is None:
        Wq = torch.empty((rows, nb * Q4_0_BYTES), dtype=torch.uint8, device=W.device)
    _check(lib().q4_0_quantize(_dev(W, torch.float32, "W"), rows, K, _dev(Wq, torch.uint8, "Wq"),
                               _stream(stream)), "q4_0_quantize")
    return Wq


def q8_0_quantize(X: torch.Tensor, Xq: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """fp32 N x K -> uint8 N x (K/32*34) Q8_0 blocks."""
    N, K = X.shape
    nb = _nb(K)
    if Xq is None:
        Xq = torch.empty((N, nb * Q8_0_BYTES), dtype=torch.uint8, device=X.device)
    _check(lib().q8_0_quantize(_dev(X, torch.float32, "X"), N, K, _dev(Xq, torch.uint8, "Xq"),
                               _stream(stream)), "q8_0_quantize")
    return Xq


def _rows(Wq: torch.Tensor, K: int) -> int:
    nb = _nb(K)
    if Wq.numel() % (nb * Q4_0_BYTES):
        raise ValueError("Wq size %d is not a whole number of rows of K=%d" % (Wq.numel(), K))
    return Wq.numel() // (nb * Q4_0_BYTES)


def q4bq_repack_size(rows: int, K: int) -> int:
    return int(lib().q4bq_repack_size(rows, K))


def _repacked_rows(Wr: torch.Tensor, K: int) -> int:
    """The row count whose repacked size is Wr's byte count."""
    nb = _nb(K)
    n = Wr.numel()
    r = n // (nb * Q4_0_BYTES + (nb + 1) * 32)  # at most a few rows above the answer (alignment padding)
    while r > 0 and q4bq_repack_size(r, K) > n:
        r -= 1
    if r < 1 or q4bq_repack_size(r, K) != n:
        raise ValueError("Wr size %d is not a repacked matrix of K=%d" % (n, K))
    return r


def mul_mat_q4_0_q8_0(Wq: torch.Tensor, X: torch.Tensor, Y: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Y (N x rows, fp32) = Q4_0 weights Wq times fp32 activations X (N x K)."""
    N, K = X.shape
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0_q8_0(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(X, torch.float32, "X"), N,
                                   _dev(Y, torch.float32, "Y"), _stream(stream)), "mul_mat_q4_0_q8_0")
    return Y


def mul_mat_q4_0_q8_0_noalloc(Wq: torch.Tensor, X: torch.Tensor, Y: torch.Tensor | None = None,
                              stream=None) -> torch.Tensor:
    """mul_mat_q4_0_q8_0 with the library's fixed per-GPU scratch: the call
    allocates nothing (Y must be given where the caller cannot allocate)."""
    N, K = X.shape
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0_q8_0_noalloc(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(X, torch.float32, "X"), N,
                                           _dev(Y, torch.float32, "Y"), _stream(stream)),
           "mul_mat_q4_0_q8_0_noalloc")
    return Y


def q4bq_workspace_size(rows: int, K: int, N: int) -> int:
    return int(lib().q4bq_workspace_size(rows, K, N))


def workspace(rows: int, K: int, N: int, device=None) -> torch.Tensor:
    """A device buffer big enough for mul_mat_q4_0_q8_0_ex at these sizes."""
    n = q4bq_workspace_size(rows, K, N)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def mul_mat_q4_0_q8_0_ex(Wq: torch.Tensor, X: torch.Tensor, ws: torch.Tensor, Y: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    N, K = X.shape
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0_q8_0_ex(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(X, torch.float32, "X"), N,
                                      _dev(Y, torch.float32, "Y"), _dev(ws, torch.uint8, "workspace"),
                                      ws.numel(), _stream(stream)), "mul_mat_q4_0_q8_0_ex")
    return Y


def _opt(t, dtype, what):
    return None if t is None else _dev(t, dtype, what)


def fused_workspace(rows: int, K: int, N: int, device=None) -> torch.Tensor:
    """A device buffer for the fused forms at these sizes."""
    return torch.empty(max(int(lib().q4bq_fused_workspace_size(rows, K, N)), 16), dtype=torch.uint8,
                       device=device or "cuda")


def _ws(ws):
    return (None, 0) if ws is None else (_dev(ws, torch.uint8, "workspace"), ws.numel())


def mul_mat_q4_0_q8_0_fused(Wq: torch.Tensor, X: torch.Tensor, ln_gamma=None, ln_beta=None, ln_eps: float = 1e-5,
                            bias=None, act: int = ACT_NONE, mul=None, Y: torch.Tensor | None = None, ws=None,
                            stream=None) -> torch.Tensor:
    """Y = act(LN(X) @ W^T + bias) * mul, LayerNorm and epilogue optional;
    ws: optional workspace (fused_workspace), else the library allocates."""
    N, K = X.shape
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0_q8_0_fused(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(X, torch.float32, "X"), N,
                                         _opt(ln_gamma, torch.float32, "ln_gamma"),
                                         _opt(ln_beta, torch.float32, "ln_beta"), float(ln_eps),
                                         _opt(bias, torch.float32, "bias"), int(act),
                                         _opt(mul, torch.float32, "mul"), _dev(Y, torch.float32, "Y"), *_ws(ws),
                                         _stream(stream)), "mul_mat_q4_0_q8_0_fused")
    return Y


def mul_mat_q4_0_q8_0_swiglu(Wgate: torch.Tensor, Wup: torch.Tensor, X: torch.Tensor, ln_gamma=None, ln_beta=None,
                             ln_eps: float = 1e-5, H: torch.Tensor | None = None, ws=None,
                             stream=None) -> torch.Tensor:
    """H = SiLU(LN(X) @ Wgate^T) * (LN(X) @ Wup^T)."""
    N, K = X.shape
    rows = _rows(Wgate, K)
    if _rows(Wup, K) != rows:
        raise ValueError("gate and up matrices differ in rows")
    if H is None:
        H = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0_q8_0_swiglu(_dev(Wgate, torch.uint8, "Wgate"), _dev(Wup, torch.uint8, "Wup"), rows, K,
                                          _dev(X, torch.float32, "X"), N, _opt(ln_gamma, torch.float32, "ln_gamma"),
                                          _opt(ln_beta, torch.float32, "ln_beta"), float(ln_eps),
                                          _dev(H, torch.float32, "H"), *_ws(ws), _stream(stream)),
           "mul_mat_q4_0_q8_0_swiglu")
    return H


def _rows_q8(Wq8: torch.Tensor, K: int) -> int:
    nb = _nb(K)
    if Wq8.numel() % (nb * Q8_0_BYTES):
        raise ValueError("Wq8 size %d is not a whole number of Q8_0 rows of K=%d" % (Wq8.numel(), K))
    return Wq8.numel() // (nb * Q8_0_BYTES)


def mul_mat_q8_0_q8_0(Wq8: torch.Tensor, X: torch.Tensor, Y: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Y = X @ W^T with Q8_0 weights (from q8_0_quantize(W)); X fp32 N x K."""
    N, K = X.shape
    rows = _rows_q8(Wq8, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q8_0_q8_0(_dev(Wq8, torch.uint8, "Wq8"), rows, K, _dev(X, torch.float32, "X"), N,
                                   _dev(Y, torch.float32, "Y"), _stream(stream)), "mul_mat_q8_0_q8_0")
    return Y


def q8_0_q8_0_block_dots(Wq8: torch.Tensor, Xq: torch.Tensor, K: int, D: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """Every per-block int32 dot of Q8_0 weights with Q8_0 activations (N x rows x K/32)."""
    rows = _rows_q8(Wq8, K)
    N = _rows_q8(Xq, K)
    if D is None:
        D = torch.empty((N, rows, K // 32), dtype=torch.int32, device=Wq8.device)
    _check(lib().q8_0_q8_0_block_dots(_dev(Wq8, torch.uint8, "Wq8"), rows, K, _dev(Xq, torch.uint8, "Xq"), N,
                                      _dev(D, torch.int32, "D"), _stream(stream)), "q8_0_q8_0_block_dots")
    return D


def q4_0_get_rows(Wq: torch.Tensor, K: int, ids: torch.Tensor, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Rows `ids` (int32, device) of a Q4_0 table, decoded to fp32 (n x K)."""
    rows = _rows(Wq, K)
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=torch.float32, device=Wq.device)
    _check(lib().q4_0_get_rows(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(ids, torch.int32, "ids"), n,
                               _dev(out, torch.float32, "out"), _stream(stream)), "q4_0_get_rows")
    return out


def q4_0_repack(Wq: torch.Tensor, K: int, Wr: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Q4_0 blocks -> repacked weights (nibble stream, scale stream, matrix-core
    weight records; q4bq_repack_size bytes)."""
    rows = _rows(Wq, K)
    if Wr is None:
        n = lib().q4bq_repack_size(rows, K)
        if n == 0:
            raise Q4BQError(Q4BQ_EINVAL, "q4bq_repack_size")
        Wr = torch.empty(n, dtype=torch.uint8, device=Wq.device)  # the allocator aligns to 256 bytes
    _check(lib().q4_0_repack(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(Wr, torch.uint8, "Wr"), _stream(stream)),
           "q4_0_repack")
    return Wr


def mul_mat_q4_0r_q8_0(Wr: torch.Tensor, X: torch.Tensor, Y: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """mul_mat_q4_0_q8_0 on repacked weights."""
    N, K = X.shape
    rows = _repacked_rows(Wr, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0r_q8_0(_dev(Wr, torch.uint8, "Wr"), rows, K, _dev(X, torch.float32, "X"), N,
                                    _dev(Y, torch.float32, "Y"), _stream(stream)), "mul_mat_q4_0r_q8_0")
    return Y


def mul_mat_q4_0r_q8_0_ex(Wr: torch.Tensor, X: torch.Tensor, ws: torch.Tensor, Y: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    N, K = X.shape
    rows = _repacked_rows(Wr, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=X.device)
    _check(lib().mul_mat_q4_0r_q8_0_ex(_dev(Wr, torch.uint8, "Wr"), rows, K, _dev(X, torch.float32, "X"), N,
                                       _dev(Y, torch.float32, "Y"), _dev(ws, torch.uint8, "workspace"),
                                       ws.numel(), _stream(stream)), "mul_mat_q4_0r_q8_0_ex")
    return Y


def mul_mat_q4_0_q8_0_multi(Wqs, X: torch.Tensor, Ys=None, ws: torch.Tensor | None = None,
                            stream=None) -> list:
    """Y[i] = mul_mat_q4_0_q8_0(Wqs[i], X) for every i, one launch for N <= 8."""
    N, K = X.shape
    count = len(Wqs)
    rows = [_rows(W, K) for W in Wqs]
    if Ys is None:
        Ys = [torch.empty((N, r), dtype=torch.float32, device=X.device) for r in rows]
    wp = (ctypes.c_void_p * count)(*[_dev(W, torch.uint8, "Wq[%d]" % i) for i, W in enumerate(Wqs)])
    yp = (ctypes.c_void_p * count)(*[_dev(Y, torch.float32, "Y[%d]" % i) for i, Y in enumerate(Ys)])
    rp = (ctypes.c_int64 * count)(*rows)
    wsp, wsn = (None, 0) if ws is None else (_dev(ws, torch.uint8, "workspace"), ws.numel())
    _check(lib().mul_mat_q4_0_q8_0_multi(count, ctypes.cast(wp, ctypes.c_void_p), ctypes.cast(rp, ctypes.c_void_p), K,
                                         _dev(X, torch.float32, "X"), N, ctypes.cast(yp, ctypes.c_void_p), wsp, wsn,
                                         _stream(stream)), "mul_mat_q4_0_q8_0_multi")
    return Ys


def mul_mat_q4_0_q8_0_set(Wqs, Xs, Ys=None, stream=None) -> list:
    """Y[i] = mul_mat_q4_0_q8_0(Wqs[i], Xs[i]) for every i, one token each (Xs[i]: 1 x K_i or K_i values),
    in one launch where the set fits it."""
    count = len(Wqs)
    if len(Xs) != count:
        raise ValueError("mul_mat_q4_0_q8_0_set: %d weight matrices, %d tokens" % (count, len(Xs)))
    Ks = [int(X.numel()) for X in Xs]
    rows = [_rows(W, K) for W, K in zip(Wqs, Ks)]
    if Ys is None:
        Ys = [torch.empty((1, r), dtype=torch.float32, device=X.device) for r, X in zip(rows, Xs)]
    wp = (ctypes.c_void_p * count)(*[_dev(W, torch.uint8, "Wq[%d]" % i) for i, W in enumerate(Wqs)])
    xp = (ctypes.c_void_p * count)(*[_dev(X, torch.float32, "X[%d]" % i) for i, X in enumerate(Xs)])
    yp = (ctypes.c_void_p * count)(*[_dev(Y, torch.float32, "Y[%d]" % i) for i, Y in enumerate(Ys)])
    rp = (ctypes.c_int64 * count)(*rows)
    kp = (ctypes.c_int64 * count)(*Ks)
    _check(lib().mul_mat_q4_0_q8_0_set(count, ctypes.cast(wp, ctypes.c_void_p), ctypes.cast(rp, ctypes.c_void_p),
                                       ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(xp, ctypes.c_void_p),
                                       ctypes.cast(yp, ctypes.c_void_p), _stream(stream)), "mul_mat_q4_0_q8_0_set")
    return Ys


def q4bq_quantize_activations(X: torch.Tensor, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """Quantize X (N x K fp32) into the workspace for mul_mat_q4_0_q8_0_prepared."""
    N, K = X.shape
    _nb(K)
    _check(lib().q4bq_quantize_activations(_dev(X, torch.float32, "X"), N, K, _dev(ws, torch.uint8, "workspace"),
                                           ws.numel(), _stream(stream)), "q4bq_quantize_activations")
    return ws


def mul_mat_q4_0_q8_0_prepared(Wq: torch.Tensor, ws: torch.Tensor, N: int, K: int, Y: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=Wq.device)
    _check(lib().mul_mat_q4_0_q8_0_prepared(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(ws, torch.uint8, "workspace"),
                                            N, _dev(Y, torch.float32, "Y"), _stream(stream)),
           "mul_mat_q4_0_q8_0_prepared")
    return Y


def mul_mat_q4_0_q8_0_pq(Wq: torch.Tensor, Xq: torch.Tensor, K: int, Y: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    nb = _nb(K)
    if Xq.numel() % (nb * Q8_0_BYTES):
        raise ValueError("Xq size is not a whole number of Q8_0 rows")
    N = Xq.numel() // (nb * Q8_0_BYTES)
    rows = _rows(Wq, K)
    if Y is None:
        Y = torch.empty((N, rows), dtype=torch.float32, device=Xq.device)
    _check(lib().mul_mat_q4_0_q8_0_pq(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(Xq, torch.uint8, "Xq"), N,
                                      _dev(Y, torch.float32, "Y"), _stream(stream)), "mul_mat_q4_0_q8_0_pq")
    return Y


def q4_0_q8_0_block_dots(Wq: torch.Tensor, Xq: torch.Tensor, K: int, D: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """int32 N x rows x (K/32): every per-block integer dot."""
    nb = _nb(K)
    N = Xq.numel() // (nb * Q8_0_BYTES)
    rows = _rows(Wq, K)
    if D is None:
        D = torch.empty((N, rows, nb), dtype=torch.int32, device=Xq.device)
    _check(lib().q4_0_q8_0_block_dots(_dev(Wq, torch.uint8, "Wq"), rows, K, _dev(Xq, torch.uint8, "Xq"), N,
                                      _dev(D, torch.int32, "D"), _stream(stream)), "q4_0_q8_0_block_dots")
    return D


def q4bq_version() -> int:
    return int(lib().q4bq_version())
