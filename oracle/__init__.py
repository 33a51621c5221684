"""CPU oracle for the Q4_0 x Q8_0 quantized matrix product.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the HIP library never imports, links or calls it, and
this package imports nothing from the HIP side.

The arithmetic lives in ``q4bq_oracle.c`` (plain C loops, fp64 accumulation,
built with ``gcc -O2 -ffp-contract=off``); this module only loads it with
ctypes and converts between NumPy arrays and raw pointers.  Every function
follows "llama.cpp 深度解读" (luoboask.github.io) section 2 (the Q4_0 block and
its encode/decode) and section 3 (ggml_vec_dot_q4_0_q8_0), with the readings
R1-R6 / G1 / G5 stated at the top of the C file.

Layouts (all row-major, innermost dimension contiguous):
  W  : rows x K fp32            Wq : rows x (K/32) blocks of 18 bytes
                                Wq8: rows x (K/32) Q8_0 weight blocks of 34 bytes
  X  : N x K fp32               Xq : N x (K/32) blocks of 34 bytes
  Y  : N x rows                 D  : N x rows x (K/32) int32
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

QK = 32
Q4_BYTES = 18
Q8_BYTES = 34

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4bq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    sig = {
        "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
        "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f32_to_f16_array": (None, [P, I64, P]),
        "orc_q4_0_quantize": (None, [P, I64, I64, P]),
        "orc_q4_0_dequantize": (None, [P, I64, I64, P]),
        "orc_q8_0_quantize": (None, [P, I64, I64, P]),
        "orc_block_dot": (ctypes.c_int32, [P, P]),
        "orc_block_dots": (None, [P, I64, I64, P, I64, P]),
        "orc_mul_mat_ref": (None, [P, I64, I64, P, I64, P]),
        "orc_mul_mat_pages_f32": (None, [P, I64, I64, P, I64, P]),
        "orc_mul_mat": (ctypes.c_int, [P, I64, I64, P, I64, P, ctypes.c_int]),
        "orc_block_dot_q8": (ctypes.c_int32, [P, P]),
        "orc_block_dots_q8": (None, [P, I64, I64, P, I64, P]),
        "orc_mul_mat_q8_ref": (None, [P, I64, I64, P, I64, P]),
        "orc_layernorm": (None, [P, I64, I64, P, P, ctypes.c_float, P]),
        "orc_gelu": (ctypes.c_double, [ctypes.c_double]),
        "orc_silu": (ctypes.c_double, [ctypes.c_double]),
        "orc_epilogue": (None, [P, I64, I64, P, ctypes.c_int, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check_k(K: int) -> int:
    if K <= 0 or K % QK != 0:
        raise ValueError("K must be a positive multiple of 32, got %d" % K)
    return K // QK


# --- scalar conversions (R6) -------------------------------------------------

def f32_to_f16_bits(x: float) -> int:
    return int(_load().orc_f32_to_f16(ctypes.c_float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(ctypes.c_uint16(h)))


def f32_to_f16_bits_array(x: np.ndarray) -> np.ndarray:
    """Element-wise fp32 -> fp16 bits by the oracle's converter."""
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(flat.size, dtype=np.uint16)
    _load().orc_f32_to_f16_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


# --- encoders / decoder --------------------------------------------------------

def q4_0_quantize(W: np.ndarray) -> np.ndarray:
    """fp32 rows x K -> uint8 rows x (K/32*18), the page's block layout."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    rows, K = W.shape
    nb = _check_k(K)
    out = np.empty((rows, nb * Q4_BYTES), dtype=np.uint8)
    _load().orc_q4_0_quantize(_ptr(W), rows, K, _ptr(out))
    return out


def q4_0_dequantize(Wq: np.ndarray, K: int) -> np.ndarray:
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq.size // (nb * Q4_BYTES)
    out = np.empty((rows, K), dtype=np.float32)
    _load().orc_q4_0_dequantize(_ptr(Wq), rows, K, _ptr(out))
    return out


def q4_0_get_rows(Wq: np.ndarray, K: int, ids: np.ndarray) -> np.ndarray:
    """Rows `ids` of a Q4_0 matrix, dequantized: out[i] = row ids[i] decoded
    by section 2's rule, (nibble - 8) * d.  This is ggml_get_rows on a Q4_0
    table, the token-embedding lookup of the Llama graph in section 4
    ("inpL = ggml_get_rows(tok_embeddings, inp_tokens)"; "llama.cpp 深度解读")
    and of GPT-2's wte/wpe in the ggml GPT-2 walkthrough (section 3.5).
    Reading taken: an id outside [0, rows) yields a row of NaN (the pages do
    not say; ggml asserts)."""
    nb = _check_k(K)
    table = q4_0_dequantize(Wq, K)
    rows = table.shape[0]
    ids = np.asarray(ids, dtype=np.int64).ravel()
    out = np.full((ids.size, nb * QK), np.nan, dtype=np.float32)
    ok = (ids >= 0) & (ids < rows)
    out[ok] = table[ids[ok]]
    return out


def q8_0_quantize(X: np.ndarray) -> np.ndarray:
    """fp32 N x K -> uint8 N x (K/32*34), natural element order."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    N, K = X.shape
    nb = _check_k(K)
    out = np.empty((N, nb * Q8_BYTES), dtype=np.uint8)
    _load().orc_q8_0_quantize(_ptr(X), N, K, _ptr(out))
    return out


# --- dots and products ------------------------------------------------------------

def block_dot(wblk: np.ndarray, xblk: np.ndarray) -> int:
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    xblk = np.ascontiguousarray(xblk, dtype=np.uint8)
    assert wblk.size == Q4_BYTES and xblk.size == Q8_BYTES
    return int(_load().orc_block_dot(_ptr(wblk), _ptr(xblk)))


def block_dots(Wq: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
    """int32 N x rows x (K/32): every per-block integer dot."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq.size // (nb * Q4_BYTES)
    N = Xq.size // (nb * Q8_BYTES)
    D = np.empty((N, rows, nb), dtype=np.int32)
    _load().orc_block_dots(_ptr(Wq), rows, K, _ptr(Xq), N, _ptr(D))
    return D


def mul_mat_ref(Wq: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
    """fp64 N x rows: exact per-block terms summed in fp64 (the parity target)."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq.size // (nb * Q4_BYTES)
    N = Xq.size // (nb * Q8_BYTES)
    Y = np.empty((N, rows), dtype=np.float64)
    _load().orc_mul_mat_ref(_ptr(Wq), rows, K, _ptr(Xq), N, _ptr(Y))
    return Y


def block_dot_q8(wblk: np.ndarray, xblk: np.ndarray) -> int:
    """Integer dot of one Q8_0 weight block with one Q8_0 activation block
    (34 bytes each): sum of int8 products, no offset."""
    wblk = np.ascontiguousarray(wblk, dtype=np.uint8)
    xblk = np.ascontiguousarray(xblk, dtype=np.uint8)
    return int(_load().orc_block_dot_q8(_ptr(wblk), _ptr(xblk)))


def block_dots_q8(Wq8: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
    """int32 N x rows x (K/32): every per-block dot of Q8_0 weights with Q8_0
    activations."""
    Wq8 = np.ascontiguousarray(Wq8, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq8.size // (nb * Q8_BYTES)
    N = Xq.size // (nb * Q8_BYTES)
    D = np.empty((N, rows, nb), dtype=np.int32)
    _load().orc_block_dots_q8(_ptr(Wq8), rows, K, _ptr(Xq), N, _ptr(D))
    return D


def mul_mat_q8_ref(Wq8: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
    """fp64 N x rows for Q8_0 weights (section 1's type table lists Q8_0 as a
    weight type; its block is the block_q8_0 of the activations): exact
    per-block terms d_w * d_x * s summed in fp64."""
    Wq8 = np.ascontiguousarray(Wq8, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq8.size // (nb * Q8_BYTES)
    N = Xq.size // (nb * Q8_BYTES)
    Y = np.empty((N, rows), dtype=np.float64)
    _load().orc_mul_mat_q8_ref(_ptr(Wq8), rows, K, _ptr(Xq), N, _ptr(Y))
    return Y


ACT_NONE, ACT_GELU, ACT_SILU = 0, 1, 2


def layernorm(X: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm of each row of X (the GPT-2 walkthrough, section 3.1:
    gamma * (x - mu) / sqrt(sigma^2 + eps) + beta), statistics and arithmetic
    in fp64, the result rounded to fp32."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    N, K = X.shape
    g = np.ascontiguousarray(gamma, dtype=np.float32).reshape(K)
    b = np.ascontiguousarray(beta, dtype=np.float32).reshape(K)
    out = np.empty((N, K), dtype=np.float32)
    _load().orc_layernorm(_ptr(X), N, K, _ptr(g), _ptr(b), float(eps), _ptr(out))
    return out


def gelu(x: float) -> float:
    """GELU in GPT-2's tanh form."""
    return float(_load().orc_gelu(float(x)))


def silu(x: float) -> float:
    """SiLU(x) = x * sigmoid(x) ("llama.cpp 深度解读" section 4)."""
    return float(_load().orc_silu(float(x)))


def epilogue(Y: np.ndarray, bias=None, act: int = ACT_NONE, mul=None) -> np.ndarray:
    """act(Y + bias) * mul in fp64 (bias per row, mul N x rows; either may be
    None): the bias add and GELU after GPT-2's c_mlp_fc, and SiLU(gate) * up."""
    Y = np.array(Y, dtype=np.float64, order="C", copy=True)
    N, rows = Y.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32).reshape(rows)
    m = None if mul is None else np.ascontiguousarray(mul, dtype=np.float64).reshape(N, rows)
    _load().orc_epilogue(_ptr(Y), N, rows, None if b is None else _ptr(b), int(act), None if m is None else _ptr(m))
    return Y


def mul_mat_pages_f32(Wq: np.ndarray, Xq: np.ndarray, K: int) -> np.ndarray:
    """fp32 N x rows with the page's own sequential fp32 accumulation."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    Xq = np.ascontiguousarray(Xq, dtype=np.uint8)
    nb = _check_k(K)
    rows = Wq.size // (nb * Q4_BYTES)
    N = Xq.size // (nb * Q8_BYTES)
    Y = np.empty((N, rows), dtype=np.float32)
    _load().orc_mul_mat_pages_f32(_ptr(Wq), rows, K, _ptr(Xq), N, _ptr(Y))
    return Y


def mul_mat(Wq: np.ndarray, X: np.ndarray, nthreads: int = 1) -> np.ndarray:
    """Whole operator from fp32 activations: Q8_0-quantize X, then the fp64
    reference product.  Returns fp64 N x rows."""
    Wq = np.ascontiguousarray(Wq, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.float32)
    N, K = X.shape
    nb = _check_k(K)
    rows = Wq.size // (nb * Q4_BYTES)
    Y = np.empty((N, rows), dtype=np.float64)
    rc = _load().orc_mul_mat(_ptr(Wq), rows, K, _ptr(X), N, _ptr(Y), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle scratch allocation failed")
    return Y
