"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects bad arguments before anything reaches the GPU.  No compute call
is made here (there is no device in this test's environment)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "q4bq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def L():
    import torch  # noqa: F401  (one HIP runtime per process: torch's)
    from q4_block_quantized_amd import binding
    return binding.lib()


def test_header_declares_the_boundary():
    names = set(_declared())
    assert {"q4_0_quantize", "q8_0_quantize", "mul_mat_q4_0_q8_0", "q4bq_workspace_size",
            "mul_mat_q4_0_q8_0_ex", "mul_mat_q4_0_q8_0_pq", "q4_0_q8_0_block_dots",
            "q4bq_status_string", "q4bq_version"} <= names


def test_every_declared_symbol_is_exported(L):
    from q4_block_quantized_amd import binding
    for name in _declared():
        assert hasattr(L, name), name
        assert name in binding.EXPORTS, name


def test_status_strings(L):
    for rc in (0, -1, -2, -3, 7):
        assert isinstance(L.q4bq_status_string(rc), bytes)
    assert L.q4bq_status_string(0) == b"ok"
    assert L.q4bq_version() >= 100


def test_workspace_size(L):
    assert L.q4bq_workspace_size(4096, 4096, 1) == 128 * 40 + (256 - (128 * 40) % 256) % 256
    assert L.q4bq_workspace_size(14336, 4096, 512) == 512 * 128 * 64
    # few workgroup tiles (4096 rows x 512 tokens: 19 x 4 < 256): the
    # activations, then room for up to 4 ranges of fp32 sums of the split K
    assert L.q4bq_workspace_size(4096, 4096, 512) == 512 * 128 * 64 + 4 * 512 * 4096 * 4
    # rows of fewer than 32 blocks never split
    assert L.q4bq_workspace_size(4096, 768, 512) == 512 * 24 * 64
    assert L.q4bq_workspace_size(1, 31, 1) == 0
    assert L.q4bq_workspace_size(0, 32, 1) == 0
    assert L.q4bq_workspace_size(1, 32, 0) == 0


A = 0x100000          # fake, well-aligned device addresses: never dereferenced,
B = 0x200000          # every call below must fail validation first
C = 0x300000
WS = 0x400000
EINVAL, ENOMEM = -1, -3


def _bad_product_calls(L):
    f = L.mul_mat_q4_0_q8_0
    yield f(None, 4, 64, B, 1, C, None)            # null weights
    yield f(A, 4, 64, None, 1, C, None)            # null activations
    yield f(A, 4, 64, B, 1, None, None)            # null output
    yield f(A, 0, 64, B, 1, C, None)               # rows < 1
    yield f(A, 4, 64, B, 0, C, None)               # N < 1
    yield f(A, 4, -32, B, 1, C, None)              # K < 0
    yield f(A, 4, 0, B, 1, C, None)                # K = 0
    yield f(A, 4, 16, B, 1, C, None)               # K < 32
    yield f(A, 4, 48, B, 1, C, None)               # K % 32 != 0
    yield f(A + 1, 4, 64, B, 1, C, None)           # Q4_0 data on an odd address
    yield f(A, 4, 64, B + 2, 1, C, None)           # fp32 X not 4-byte aligned
    yield f(A, 4, 64, B, 1, C + 2, None)           # Y not 4-byte aligned
    yield f(A, 4, 64, B, 1, A + 8, None)           # Y overlaps the weights
    yield f(A, 4, 64, B, 2, B + 16, None)          # Y overlaps X
    yield f(A, 1 << 41, 64, B, 1, C, None)         # absurd row count
    # a matrix-core grid of 2^22 * 2 workgroups x 512 threads = 2^32 work-items:
    # one past HIP's limit (rows = 2^22 * 224, N = 129 -> 2 token tiles)
    yield f(1 << 40, (1 << 22) * 224, 32, 2 << 40, 129, 3 << 40, None)
    g = L.mul_mat_q4_0_q8_0_pq
    yield g(A, 4, 64, B + 1, 1, C, None)           # Q8_0 data on an odd address
    yield g(A, 4, 80, B, 1, C, None)               # K % 32 != 0
    d = L.q4_0_q8_0_block_dots
    yield d(A, 4, 64, B, 1, C + 1, None)           # D misaligned
    yield d(A, 4, 64, B, 1, None, None)
    e = L.mul_mat_q4_0_q8_0_ex
    yield e(A, 4, 64, B, 1, C, None, 1 << 20, None)         # null workspace
    yield e(A, 4, 64, B, 1, C, WS + 8, 1 << 20, None)       # workspace not 16-byte aligned
    yield e(A, 4, 64, B, 1, C, A, 1 << 20, None)            # workspace overlaps the weights
    q4 = L.q4_0_quantize
    yield q4(None, 4, 64, B, None)
    yield q4(A, 4, 48, B, None)
    yield q4(A + 2, 4, 64, B, None)
    yield q4(A, 4, 64, B + 1, None)
    yield q4(A, 4, 64, A + 4, None)                # output inside the input
    rp = L.q4_0_repack
    yield rp(None, 4, 64, B, None)
    yield rp(A, 4, 64, None, None)
    yield rp(A, 4, 48, B, None)                    # K % 32 != 0
    yield rp(A + 1, 4, 64, B, None)                # Q4_0 data on an odd address
    yield rp(A, 4, 64, B + 8, None)                # repacked output not 16-byte aligned
    yield rp(A, 4, 64, A + 16, None)               # output overlaps the input
    yield rp(A + 256, 4, 64, A, None)              # the record stream would overlap the input
    r = L.mul_mat_q4_0r_q8_0
    yield r(A + 2, 4, 64, B, 1, C, None)           # repacked weights must be 16-byte aligned
    yield r(A, 4, 64, B, 1, A + 8, None)           # Y overlaps the weights
    yield r(A, 4, 64, B, 1, A + 600, None)         # Y overlaps the repacked record stream
    yield r(A, 4, 48, B, 1, C, None)
    rx = L.mul_mat_q4_0r_q8_0_ex
    yield rx(A + 8, 4, 64, B, 1, C, WS, 1 << 20, None)
    yield rx(A, 4, 64, B, 1, C, WS + 8, 1 << 20, None)
    mm = L.mul_mat_q4_0_q8_0_multi
    ptrs = lambda *v: ctypes.cast((ctypes.c_void_p * len(v))(*v), ctypes.c_void_p)
    i64s = lambda *v: ctypes.cast((ctypes.c_int64 * len(v))(*v), ctypes.c_void_p)
    yield mm(0, ptrs(A), i64s(4), 64, B, 1, ptrs(C), None, 0, None)            # count < 1
    yield mm(9, ptrs(*[A] * 9), i64s(*[4] * 9), 64, B, 1, ptrs(*[C + 256 * i for i in range(9)]), None, 0, None)
    yield mm(2, None, i64s(4, 4), 64, B, 1, ptrs(C, C + 256), None, 0, None)   # null weight array
    yield mm(2, ptrs(A, A + 4096), i64s(4, 4), 64, B, 1, ptrs(C, C + 8), None, 0, None)       # outputs overlap
    yield mm(2, ptrs(A, A + 4096), i64s(4, 4), 64, B, 1, ptrs(C, A + 4100), None, 0, None)    # output inside a weight
    yield mm(2, ptrs(A, A + 4096), i64s(4, 0), 64, B, 1, ptrs(C, C + 256), None, 0, None)     # a matrix with 0 rows
    yield mm(2, ptrs(A, A + 4096), i64s(4, 4), 48, B, 1, ptrs(C, C + 256), None, 0, None)     # K % 32 != 0
    yield mm(2, ptrs(A, A + 4096), i64s(4, 4), 64, B, 1, ptrs(C, C + 256), WS + 8, 1 << 20, None)  # workspace misaligned
    st = L.mul_mat_q4_0_q8_0_set
    yield st(0, ptrs(A), i64s(4), i64s(64), ptrs(B), ptrs(C), None)                                # count < 1
    yield st(9, ptrs(*[A] * 9), i64s(*[4] * 9), i64s(*[64] * 9), ptrs(*[B] * 9),
             ptrs(*[C + 256 * i for i in range(9)]), None)                                             # count > 8
    yield st(2, None, i64s(4, 4), i64s(64, 64), ptrs(B, B + 256), ptrs(C, C + 256), None)             # null weight array
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), None, ptrs(B, B + 256), ptrs(C, C + 256), None)        # null K array
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), i64s(64, 48), ptrs(B, B + 256), ptrs(C, C + 256), None)  # K % 32 != 0
    yield st(2, ptrs(A, A + 4096), i64s(4, 0), i64s(64, 64), ptrs(B, B + 256), ptrs(C, C + 256), None)  # 0 rows
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), i64s(64, 64), ptrs(B, None), ptrs(C, C + 256), None)    # null token
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), i64s(64, 64), ptrs(B, B + 256), ptrs(C, C + 8), None)   # outputs overlap
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), i64s(64, 64), ptrs(B, B + 256), ptrs(B + 260, C), None)  # output in a token
    yield st(2, ptrs(A, A + 4096), i64s(4, 4), i64s(64, 64), ptrs(B, B + 256), ptrs(C, A + 8), None)   # output in weights
    gr = L.q4_0_get_rows
    yield gr(None, 4, 64, B, 3, C, None)           # null table
    yield gr(A, 4, 64, None, 3, C, None)           # null ids
    yield gr(A, 4, 64, B, 3, None, None)           # null output
    yield gr(A, 4, 64, B, 0, C, None)              # n < 1
    yield gr(A, 4, 48, B, 3, C, None)              # K % 32 != 0
    yield gr(A + 1, 4, 64, B, 3, C, None)          # Q4_0 data on an odd address
    yield gr(A, 4, 64, B + 2, 3, C, None)          # ids not 4-byte aligned
    yield gr(A, 4, 64, B, 3, C + 4, None)          # output not 16-byte aligned
    yield gr(A, 4, 64, B, 3, A + 16, None)         # output overlaps the table
    yield gr(A, 4, 64, B, 3, B - 512, None)        # output overlaps ids
    fu = L.mul_mat_q4_0_q8_0_fused
    yield fu(A, 4, 64, B, 1, WS, None, ctypes.c_float(1e-5), None, 0, None, C, None, 0, None)   # gamma without beta
    yield fu(A, 4, 64, B, 1, WS, WS + 256, ctypes.c_float(-1.0), None, 0, None, C, None, 0, None)  # eps < 0
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), None, 3, None, C, None, 0, None)    # unknown activation
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), C + 4, 0, None, C, None, 0, None)   # bias overlaps Y
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), None, 0, C + 4, C, None, 0, None)   # factor partly over Y
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), WS + 2, 0, None, C, None, 0, None)  # bias misaligned
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), None, 0, None, C, WS + 8, 1 << 20, None)  # ws misaligned
    yield fu(A, 4, 64, B, 1, None, None, ctypes.c_float(0.0), None, 0, None, C, C, 1 << 20, None)       # ws over Y
    # LayerNorm runs one 1024-thread workgroup per token: N = 2^22 is past HIP's grid limit
    yield fu(1 << 40, 4, 32, 2 << 40, 1 << 22, 3 << 40, (3 << 40) + 1024, ctypes.c_float(0.0), None, 0, None,
             4 << 40, None, 0, None)
    sw = L.mul_mat_q4_0_q8_0_swiglu
    yield sw(A, None, 4, 64, B, 1, None, None, ctypes.c_float(0.0), C, None, 0, None)   # null up matrix
    yield sw(A, A + 4096, 4, 64, B, 1, WS, None, ctypes.c_float(0.0), C, None, 0, None)  # beta missing
    yield sw(A, A + 4096, 4, 64, B, 1, None, None, ctypes.c_float(0.0), A + 4100, None, 0, None)  # H in a weight
    m8 = L.mul_mat_q8_0_q8_0
    yield m8(None, 4, 64, B, 1, C, None)           # null weights
    yield m8(A, 4, 48, B, 1, C, None)              # K % 32 != 0
    yield m8(A, 4, 32800, B, 1, C, None)           # K / 32 above 1024
    yield m8(A + 1, 4, 64, B, 1, C, None)          # Q8_0 weights on an odd address
    yield m8(A, 4, 64, B + 2, 1, C, None)          # X not 4-byte aligned
    yield m8(A, 4, 64, B, 1, A + 32, None)         # Y overlaps the weights
    yield m8(A, 4, 64, B, 0, C, None)              # N < 1
    d8 = L.q8_0_q8_0_block_dots
    yield d8(A, 4, 64, None, 1, C, None)           # null activations
    yield d8(A, 4, 64, B + 1, 1, C, None)          # activations on an odd address
    yield d8(A, 4, 64, B, 1, C + 2, None)          # D not 4-byte aligned
    yield d8(A, 4, 64, B, 1, B + 4, None)          # D overlaps the activations
    q8 = L.q8_0_quantize
    yield q8(A, 0, 64, B, None)
    yield q8(A, 4, 33, B, None)
    yield q8(A, 4, 64, B + 1, None)


def test_bad_arguments_return_einval(L):
    for i, rc in enumerate(_bad_product_calls(L)):
        assert rc == EINVAL, "case %d returned %d" % (i, rc)


def test_repack_size(L):
    # nibble + scale streams (rounded up to 256 bytes), then (K/32 + 1) planes of 32-byte records
    assert L.q4bq_repack_size(4, 64) == 256 + 3 * 4 * 32
    assert L.q4bq_repack_size(128256, 4096) == 128256 * 128 * 18 + 129 * 128256 * 32
    assert L.q4bq_repack_size(1, 32) == 256 + 2 * 32
    assert L.q4bq_repack_size(0, 64) == 0
    assert L.q4bq_repack_size(4, 48) == 0


def test_fused_workspace_size(L):
    # the activation records (N <= 8: 40 bytes per block; above: 64), rounded up to 256 bytes
    assert L.q4bq_fused_workspace_size(4096, 4096, 1) == 5120
    assert L.q4bq_fused_workspace_size(14336, 4096, 3) == (3 * 128 * 40 + 255) // 256 * 256
    assert L.q4bq_fused_workspace_size(14336, 4128, 3) == (3 * 129 * 40 + 255) // 256 * 256
    assert L.q4bq_fused_workspace_size(14336, 4096, 512) == 512 * 128 * 64
    # and the room for the split K's range sums where the grid has few tiles
    assert L.q4bq_fused_workspace_size(4096, 4096, 512) == 512 * 128 * 64 + 4 * 512 * 4096 * 4
    assert L.q4bq_fused_workspace_size(4, 48, 1) == 0


def test_workspace_too_small_is_enomem(L):
    need = L.q4bq_workspace_size(4, 64, 1)
    assert L.mul_mat_q4_0_q8_0_ex(A, 4, 64, B, 1, C, WS, need - 1, None) == ENOMEM


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path; a device is present")
def test_no_device_is_ehip_not_abort(L):
    # valid arguments, no device: the library must report a HIP failure
    assert L.mul_mat_q4_0_q8_0(A, 4, 64, B, 1, C, None) == -2
    assert L.mul_mat_q4_0_q8_0_ex(A, 4, 64, B, 1, C, WS, 1 << 20, None) == -2
    assert L.q4_0_quantize(A, 4, 64, B, None) == -2
    assert L.q4_0_q8_0_block_dots(A, 4, 64, B, 1, C, None) == -2
    assert L.q4_0_repack(A, 4, 64, B, None) == -2
    assert L.q4_0_get_rows(A, 4, 64, B, 3, C, None) == -2
    assert L.mul_mat_q8_0_q8_0(A, 4, 64, B, 1, C, None) == -2
    assert L.mul_mat_q4_0_q8_0_fused(A, 4, 64, B, 1, WS, WS + 256, ctypes.c_float(1e-5), None, 2, None, C,
                                     None, 0, None) == -2
    assert L.q8_0_q8_0_block_dots(A, 4, 64, B, 1, C, None) == -2
    assert L.mul_mat_q4_0r_q8_0(A, 4, 64, B, 1, C, None) == -2
