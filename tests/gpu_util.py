"""Helpers for the GPU parity tests: device upload, comparison rules, near-tie counting.

Comparison rules (the tolerances the method is checked to):
* integer / index outputs (accepted lengths, paths, token ids, top-k ids): exact, except a
  top-k rank whose two contested tokens have oracle logits closer than TOPK_TIE_GAP, which
  is counted and reported;
* fp32 outputs: max abs difference <= 1e-4;
* bf16 outputs (attention output, logits): |gpu - ref| <= 1e-2 + 1e-2 |ref|;
* log-sum-exp: 1e-4 (fp32 inputs) / 1e-3 (bf16 inputs).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

TOPK_TIE_GAP = 1e-4
FP32_ATOL = 1e-4
BF16_ATOL = 1e-2
BF16_RTOL = 1e-2

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "medusa_tree_attention_verify_amd", "libmedusa_verify.so")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        pytest.fail(f"HIP library not built: {LIB}")


def dev(x, dtype=torch.float32):
    """Host numpy -> device tensor (bf16 values must already be bf16-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if t.dtype != dtype:
        t = t.to(dtype)
    return t.to("cuda")


def dev_i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def assert_fp32(got, ref, atol=FP32_ATOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err.max(initial=0.0) <= atol, f"{what}: max abs err {err.max():.3g} > {atol}"


def assert_bf16(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bad = np.abs(got - ref) > BF16_ATOL + BF16_RTOL * np.abs(ref)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside atol/rtol 1e-2; "
                           f"worst {np.abs(got - ref).max():.3g}")


def check_topk(got_ids, ref_logits, widths, gap=TOPK_TIE_GAP):
    """got_ids [B,K,s_max] vs the oracle's fp64 logits [B,K,V].  Returns #near-tie ranks."""
    got_ids = np.asarray(got_ids)
    B, K, s_max = got_ids.shape
    ties = 0
    for b in range(B):
        for k in range(K):
            s = widths[k]
            z = ref_logits[b, k]
            ref = np.argsort(-z, kind="stable")[:s]
            got = got_ids[b, k, :s]
            assert np.all(got_ids[b, k, s:] == -1), f"padding of (b={b},k={k}) not -1"
            if np.array_equal(got, ref):
                continue
            assert len(set(got.tolist())) == s, f"duplicate ids {got}"
            for r in range(s):
                if got[r] != ref[r]:
                    d = abs(z[got[r]] - z[ref[r]])
                    assert d < gap, (f"top-k mismatch at (b={b},k={k},rank {r}): gpu {got[r]} "
                                     f"vs oracle {ref[r]}, logit gap {d:.3g} >= {gap}")
                    ties += 1
    return ties
