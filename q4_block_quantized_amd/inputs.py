"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantization, no dots), so both the HIP path and the CPU oracle
can be fed from it without sharing any of the computation.

Shapes are the matrices the pages multiply by a Q4_0 weight:
  * GPT-2 117M ("ggml GPT-2 walkthrough", aicoding.csdn.net, sections 3.2 and
    3.5): c_attn [768 -> 2304], c_attn_proj [768 -> 768], c_mlp_fc [768 -> 3072],
    c_mlp_proj [3072 -> 768];
  * Llama-3-8B ("llama.cpp 深度解读", section 1, the GGUF example): the Q4_0
    token-embedding/vocabulary matrix 128256 x 4096, plus the 4096 / 14336
    attention and feed-forward projections.

Distributions: weights N(0, 0.02) in fp32; activations N(0, 1) in fp32; for the
Llama-3-8B decode set an independent Bernoulli(0.01) mask multiplies 1 % of
the weights by 10.  Generator: NumPy PCG64 (``np.random.default_rng``) with
seed = 20260000 + 100 * config + 10 * matrix + {0: weights, 1: mask, 2: x}.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260000
KIND_W, KIND_MASK, KIND_X = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    cid: int                      # 1..5
    name: str
    mats: tuple                   # ((rows, K), ...)
    ns: tuple                     # token counts measured / tested
    outliers: bool = False
    back_to_back: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    1: Workload(1, "gpt2_qkv_n1", ((2304, 768),), (1,),
                notes="GPT-2 QKV projection, one token"),
    2: Workload(2, "gpt2_layer_n1", ((2304, 768), (768, 768), (3072, 768), (768, 3072)), (1,),
                back_to_back=True, notes="GPT-2 117M decode layer: qkv, proj, mlp up, mlp down"),
    3: Workload(3, "llama3_8b_decode", ((4096, 4096), (14336, 4096), (4096, 14336)), (1, 4),
                outliers=True, back_to_back=True,
                notes="Llama-3-8B-shaped decode projections, 1 % outliers x10"),
    4: Workload(4, "llama3_8b_head", ((128256, 4096),), (1, 8),
                notes="Llama-3-8B vocabulary projection"),
    5: Workload(5, "llama3_8b_prefill", ((14336, 4096),), (512,),
                notes="Llama-3-8B feed-forward prefill, 512 tokens"),
}


def seed(cid: int, matrix: int, kind: int) -> int:
    return SEED_BASE + 100 * cid + 10 * matrix + kind


def weights(cid: int, matrix: int, rows: int, K: int, outliers: bool = False,
            row_slice: slice | None = None) -> np.ndarray:
    """fp32 rows x K, N(0, 0.02), optionally with 1 % x10 outliers.

    ``row_slice`` returns only those rows of the same full matrix (the full
    matrix is drawn; the slice is taken afterwards) -- used to give the oracle a
    bounded sample of a large workload.
    """
    rng = np.random.default_rng(seed(cid, matrix, KIND_W))
    W = rng.standard_normal((rows, K), dtype=np.float32)
    W *= np.float32(0.02)
    if outliers:
        mrng = np.random.default_rng(seed(cid, matrix, KIND_MASK))
        mask = mrng.random((rows, K)) < 0.01
        W[mask] *= np.float32(10.0)
        del mask
    if row_slice is not None:
        W = np.ascontiguousarray(W[row_slice])
    return W


def activations(cid: int, matrix: int, N: int, K: int) -> np.ndarray:
    """fp32 N x K, N(0, 1).  Smaller N are the first rows of a larger draw only
    when drawn with the same N; callers that need nesting draw max(N) once."""
    rng = np.random.default_rng(seed(cid, matrix, KIND_X))
    return rng.standard_normal((N, K), dtype=np.float32)


def random_matrix(seed_value: int, rows: int, K: int, scale: float = 1.0) -> np.ndarray:
    """Free-form N(0, scale) fp32 matrix for shape sweeps and edge cases."""
    rng = np.random.default_rng(seed_value)
    A = rng.standard_normal((rows, K), dtype=np.float32)
    if scale != 1.0:
        A *= np.float32(scale)
    return A
