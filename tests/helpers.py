"""Shared helpers of the GPU parity tests: exact conversion of device tensors
to float64 for the oracle, CSR unpacking and error summaries."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.numerics import bf16_bits_to_f64

BF16_MAX_ABS = 2e-2     # attention tolerances for bf16 inputs, fp32 accumulation
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5      # fp32 path
LSE_BF16 = 1e-4
LSE_F32 = 1e-5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_gilbert_amd as bsa  # noqa: F401  (fails loudly if not built)
    return "cuda:0"


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 or fp32 tensor."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy())
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    raise TypeError(t.dtype)


def csr_lists(row_ptr: torch.Tensor, col_idx: torch.Tensor, heads: int, nqb: int):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    return [[ci[rp[h * nqb + i]:rp[h * nqb + i + 1]] for i in range(nqb)] for h in range(heads)]


def assert_lists_equal(got_head, ref_head, tag=""):
    assert len(got_head) == len(ref_head)
    for i, (g, r) in enumerate(zip(got_head, ref_head)):
        assert np.array_equal(np.asarray(g), np.asarray(r)), "%s row %d: got %s expected %s" % (tag, i, g, r)


def err_summary(got: np.ndarray, ref: np.ndarray, rows_mask=None):
    e = np.abs(got - ref)
    if rows_mask is not None:
        e = e[rows_mask]
    return float(e.max()), float(e.mean())


def valid_rows(q_len, bs):
    m = np.zeros(len(q_len) * bs, dtype=bool)
    for i, n in enumerate(q_len):
        m[i * bs: i * bs + int(n)] = True
    return m
