"""The allocation-free heads entry point (mv_medusa_heads_noalloc, scratch in a device array
inside the library) against the workspace entry point (mv_medusa_heads), through the C ABI:
two calls in a row, the second smaller, each compared with a workspace call on the same
inputs.  Both run the same kernels, so every output must agree exactly (the bar for fp32
outputs, 1e-4, is met with zero difference)."""
import ctypes

import numpy as np
import pytest
import torch

from medusa_tree_attention_verify_amd import _lib as L
from medusa_tree_attention_verify_amd import workloads as W
from tests.gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(B, d, V, K, seed):
    h = W.normal(seed, "na_h", (B, d), 1.0, True)
    w_res = W.normal(seed, "na_wres", (K, d, d), 0.02, True)
    w_head = W.normal(seed, "na_whead", (K, V, d), 0.02, True)
    bf = torch.bfloat16
    return dev(h, bf), dev(w_res, bf), dev(w_head, bf)


def _outputs(B, d, V, K, s_max):
    f = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    return {"hk": f(B, K, d), "ids": torch.full((B, K, s_max), -7, dtype=torch.int32, device="cuda"),
            "vals": f(B, K, s_max), "lse": f(B, K)}


def _call(noalloc, B, d, V, K, widths, x):
    lib = L.lib()
    s_max = max(widths)
    o = _outputs(B, d, V, K, s_max)
    s = L.int_array(widths)
    st = torch.cuda.current_stream().cuda_stream
    h, w_res, w_head = (t.data_ptr() for t in x)
    common = (L.MV_BF16, B, d, V, K, s, s_max, h, w_res, w_head, o["hk"].data_ptr(), None,
              o["ids"].data_ptr(), o["vals"].data_ptr(), 0, o["lse"].data_ptr())
    if noalloc:
        r = lib.mv_medusa_heads_noalloc(*common, st)
    else:
        nbytes = lib.mv_medusa_heads_workspace(L.MV_BF16, B, d, V, K, s_max)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        r = lib.mv_medusa_heads(*common, ws.data_ptr(), ctypes.c_size_t(nbytes), st)
    assert r == 0, L.status_string(r)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in o.items()}


@pytest.mark.parametrize("order", ["noalloc_first", "workspace_first"])
def test_noalloc_heads_match_workspace_two_calls(order):
    require_gpu()
    cases = [(8, 4096, 32000, 4, [4, 3, 2, 1], 71),     # batch 8 at the Llama-3-8B head shape
             (1, 1024, 5000, 3, [2, 2, 1], 72)]         # then a smaller call
    for B, d, V, K, widths, seed in cases:
        print(f"noalloc heads B={B} d={d} V={V} K={K} widths={widths} ({order})", flush=True)
        x = _inputs(B, d, V, K, seed)
        if order == "noalloc_first":
            a = _call(True, B, d, V, K, widths, x)
            b = _call(False, B, d, V, K, widths, x)
        else:
            b = _call(False, B, d, V, K, widths, x)
            a = _call(True, B, d, V, K, widths, x)
        np.testing.assert_array_equal(a["ids"], b["ids"])
        for k in range(K):      # ranks past a head's width are padding (id -1, value -inf)
            assert np.all(a["ids"][:, k, :widths[k]] >= 0)
            assert np.all(a["ids"][:, k, widths[k]:] == -1)
            assert np.all(a["vals"][:, k, widths[k]:] == -np.inf)
            assert np.all(np.isfinite(a["vals"][:, k, :widths[k]]))
            assert np.max(np.abs(a["vals"][:, k, :widths[k]] - b["vals"][:, k, :widths[k]])) <= 1e-4
        for k in ("hk", "lse"):
            assert np.all(np.isfinite(a[k])), k
            assert np.max(np.abs(a[k] - b[k])) <= 1e-4, k


def test_noalloc_heads_rejects_oversize_before_launch():
    require_gpu()
    lib = L.lib()
    big = L.int_array([16] * 16)
    r = lib.mv_medusa_heads_noalloc(L.MV_BF16, 32, 8192, 128256, 16, big, 16, None, None, None,
                                    None, None, None, None, 0, None, None)
    assert r == L.MV_ERR_UNSUPPORTED
