"""The C-ABI library loads, exports every symbol its header declares, and rejects bad
arguments on the host before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

from medusa_tree_attention_verify_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "medusa_verify.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"^MV_API\s+[\w\s\*]+?\b(mv_\w+)\s*\(", text, flags=re.M)


def test_header_symbols_exported():
    names = _declared()
    assert len(names) == 23, names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert sorted(n for n, _, _ in L.SIGNATURES) == sorted(names)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("MV_MAX_NODES", "MV_MAX_DEPTH", "MV_MAX_TOPK", "MV_MAX_BATCH_HEADS",
                 "MV_MAX_HEADS", "MV_DEV_BAD_PARENT", "MV_DEV_BAD_RANK", "MV_DEV_TOO_DEEP",
                 "MV_DEV_BAD_PREFIX", "MV_DEV_BAD_TOKEN", "MV_DEV_BAD_PATH", "MV_TARGET_IDS"):
        m = re.search(rf"#define {name}\s+(0x[0-9a-fA-F]+|\d+)", text)
        assert m and int(m.group(1), 0) == getattr(L, name), name
    for name in ("MV_F32", "MV_BF16", "MV_ACCEPT_GREEDY", "MV_ACCEPT_SPECULATIVE",
                 "MV_ACCEPT_MULTICAND"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(L, name), name


def test_noalloc_scratch_size_matches_binding():
    text = open(HEADER).read()
    m = re.search(r"#define MV_HEADS_NOALLOC_SCRATCH_BYTES\s+\((\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.MV_HEADS_NOALLOC_SCRATCH_BYTES


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert L.status_string(s) not in ("", "unknown status")
    assert L.status_string(-99) == "unknown status"


def test_workspace_queries():
    lib = L.lib()
    assert lib.mv_medusa_heads_workspace(L.MV_BF16, 1, 4096, 32000, 4, 4) > 0
    assert lib.mv_medusa_heads_workspace(L.MV_BF16, 1, 4095, 32000, 4, 4) == 0   # d % 32
    assert lib.mv_tree_attn_verify_workspace(L.MV_BF16, 1, 64, 32, 8, 128, 4096) > 0
    assert lib.mv_tree_attn_verify_workspace(L.MV_BF16, 1, 64, 32, 8, 96, 4096) == 0  # dh
    assert lib.mv_tree_attn_verify_workspace(L.MV_F32, 1, 8, 4, 4, 64, 128) == 0    # no split
    # the launch beside other kernels plans its own split (persistent grid): same checks
    assert lib.mv_tree_attn_verify_beside_workspace(L.MV_BF16, 1, 64, 32, 8, 128, 4096) > 0
    assert lib.mv_tree_attn_verify_beside_workspace(L.MV_BF16, 1, 64, 32, 8, 96, 4096) == 0
    assert lib.mv_tree_attn_verify_beside_workspace(L.MV_F32, 1, 8, 4, 4, 64, 128) == 0
    assert lib.mv_tree_attn_verify_beside_workspace(L.MV_BF16, 8, 64, 64, 8, 128, 32768) > 0
    assert lib.mv_accept_paths_workspace(L.MV_ACCEPT_GREEDY, 1, 64, 32000) > 0
    assert lib.mv_accept_paths_workspace(L.MV_ACCEPT_SPECULATIVE, 64, 64, 128256) > 0
    assert (lib.mv_accept_paths_workspace(L.MV_ACCEPT_MULTICAND, 64, 64, 128256)
            == lib.mv_accept_paths_workspace(L.MV_ACCEPT_SPECULATIVE, 64, 64, 128256))
    assert lib.mv_accept_paths_workspace(3, 64, 64, 128256) == 0
    assert lib.mv_lm_head_workspace(L.MV_BF16, 65, 4096, 32000) >= 65 * 500 * 12  # 3 x [T][V/64]
    # from 129 rows (d % 128 == 0) the tiled kernel keeps partials per 256-row vocabulary block
    assert 520 * 125 * 12 <= lib.mv_lm_head_workspace(L.MV_BF16, 520, 4096, 32000) < 520 * 500 * 12
    assert lib.mv_lm_head_workspace(L.MV_BF16, 520, 4064, 32000) >= 520 * 500 * 12  # d % 128 != 0
    assert lib.mv_lm_head_workspace(L.MV_F32, 65, 4096, 32000) == 0               # bf16 only
    assert lib.mv_lm_head_workspace(L.MV_BF16, 65, 4080, 32000) == 0              # d % 32


def test_host_argument_checks():
    lib = L.lib()
    P = ctypes.c_void_p(16)   # never dereferenced: every call below fails its host checks
    ws = lambda: (None, 0)
    # heads
    assert lib.mv_medusa_residual(7, 1, 64, 1, P, P, None, None, 0, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_medusa_residual(L.MV_BF16, 1, 48, 1, P, P, None, None, 0, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_medusa_residual(L.MV_BF16, 65, 64, 1, P, P, None, None, 0, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_medusa_residual(L.MV_F32, 33, 64, 1, P, P, None, None, 0, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_medusa_residual(L.MV_BF16, 64, 64, 1, P, P, None, None, 0, None) == L.MV_ERR_WORKSPACE
    assert lib.mv_medusa_residual(L.MV_BF16, 1, 64, 1, P, P, None, None, 0, None) == L.MV_ERR_WORKSPACE
    assert lib.mv_medusa_residual(L.MV_BF16, 1, 64, 1, None, P, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    s = L.int_array([4, 3])
    s_bad = L.int_array([5, 3])
    for proj in (lib.mv_medusa_head_project,):
        assert proj(L.MV_BF16, 1, 64, 100, 2, s, 17, P, None, P, 1 << 20, None) == L.MV_ERR_UNSUPPORTED
        assert proj(L.MV_BF16, 1, 64, 100, 2, s_bad, 4, P, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
        assert proj(L.MV_BF16, 1, 64, 100, 2, s, 4, P, None, None, 0, None) == L.MV_ERR_WORKSPACE
        assert proj(L.MV_BF16, 1, 64, 100, 2, s, 4, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_medusa_head_select(L.MV_BF16, 1, 64, 100, 2, s, 4, P, P, 3, None, P, 1 << 20,
                                     None) == L.MV_ERR_INVALID_ARG                 # ld_topk
    assert lib.mv_medusa_head_select(L.MV_BF16, 1, 64, 100, 2, s, 4, None, P, 0, None, P,
                                     1 << 20, None) == L.MV_ERR_INVALID_ARG
    # allocation-free heads: sizes beyond the device scratch are refused before any device
    # call (every pointer below is null, so nothing could have been launched)
    big = L.int_array([16] * 16)
    assert (lib.mv_medusa_heads_workspace(L.MV_BF16, 32, 8192, 128256, 16, 16)
            > L.MV_HEADS_NOALLOC_SCRATCH_BYTES)
    assert lib.mv_medusa_heads_noalloc(L.MV_BF16, 32, 8192, 128256, 16, big, 16, None, None, None,
                                       None, None, None, None, 0, None, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_medusa_heads_noalloc(7, 1, 64, 100, 1, big, 4, None, None, None, None, None,
                                       None, None, 0, None, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_medusa_heads_noalloc(L.MV_BF16, 1, 64, 100, 1, big, 17, None, None, None, None,
                                       None, None, None, 0, None, None) == L.MV_ERR_UNSUPPORTED
    # top-k rows
    assert lib.mv_topk_rows(L.MV_F32, 1, 10, 11, P, 10, P, None, 11, None, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_topk_rows(L.MV_F32, 1, 10, 2, P, 9, P, None, 2, None, None) == L.MV_ERR_INVALID_ARG
    # tree
    assert lib.mv_build_tree_mask(0, P, 0, 0, 0, None, None, P, None, None, None, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_build_tree_mask(257, P, 0, 0, 0, None, None, P, None, None, None, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_build_tree_mask(8, P, 1, 17, 2, None, P, P, None, P, None, None) == L.MV_ERR_UNSUPPORTED
    # attention (both launches check their arguments the same way)
    args = (P, P, P, P, P, 0, 0.0, P, None, None)
    bad_stride = (P, P, P, P, P, 7, 0.0, P, None, None)     # N * W = 8 words per sequence
    for attn in (lib.mv_tree_attn_verify, lib.mv_tree_attn_verify_beside):
        assert attn(L.MV_BF16, 1, 8, 6, 4, 128, 200, 100, *args, None, 0, None) == L.MV_ERR_INVALID_ARG
        assert attn(L.MV_BF16, 1, 8, 8, 4, 96, 200, 100, *args, None, 0, None) == L.MV_ERR_UNSUPPORTED
        assert attn(L.MV_BF16, 1, 8, 8, 4, 128, 100, 100, *args, None, 0, None) == L.MV_ERR_INVALID_ARG
        assert attn(L.MV_BF16, 1, 8, 8, 4, 128, 10000, 8000, *args, None, 0, None) == L.MV_ERR_WORKSPACE
        # a (sequence, KV head) slice of 2 GiB or more does not fit the bf16 path's buffer offsets
        assert attn(L.MV_BF16, 1, 8, 8, 4, 128, 1 << 23, 100, *args, None, 0, None) == L.MV_ERR_UNSUPPORTED
        assert attn(L.MV_BF16, 2, 8, 8, 4, 128, 200, 100, *bad_stride, None, 0, None) == L.MV_ERR_INVALID_ARG
    # acceptance
    assert lib.mv_accept_paths(L.MV_ACCEPT_SPECULATIVE, L.MV_BF16, 1, 4, 10, 2, P, 0, P, P, P, P, P, P,
                               P, None, None, None, P, 1 << 20, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_accept_paths(L.MV_ACCEPT_SPECULATIVE, L.MV_F32, 1, 4, 10, 2, P, 0, P, P, None, P, P,
                               P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_accept_paths(L.MV_ACCEPT_GREEDY, L.MV_F32, 1, 4, 10, 17, P, 0, P, P, None, None, P,
                               P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_accept_paths(L.MV_ACCEPT_GREEDY, L.MV_F32, 1, 4, 10, 2, P, 0, P, P, None, None, P,
                               P, P, None, None, None, None, 0, None) == L.MV_ERR_WORKSPACE
    assert lib.mv_accept_paths(L.MV_ACCEPT_MULTICAND, L.MV_BF16, 1, 4, 10, 2, P, 0, P, P, P, P, P, P,
                               P, None, None, None, P, 1 << 20, None) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_accept_paths(L.MV_ACCEPT_MULTICAND, L.MV_F32, 1, 4, 10, 2, P, 0, P, P, P, None, P,
                               P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_accept_paths(3, L.MV_F32, 1, 4, 10, 2, P, 0, P, P, P, P, P,
                               P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    # a per-sequence parents stride shorter than N
    assert lib.mv_accept_paths(L.MV_ACCEPT_GREEDY, L.MV_F32, 2, 4, 10, 2, P, 3, P, P, None, None, P,
                               P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    # argmax-id targets: greedy only
    assert lib.mv_accept_paths(L.MV_ACCEPT_SPECULATIVE, L.MV_TARGET_IDS, 1, 4, 10, 2, P, 0, P, P, P, P,
                               P, P, P, None, None, None, P, 1 << 20, None) == L.MV_ERR_INVALID_ARG
    # speculative acceptance from the LM head
    lm = lambda ddt, d, **kw: lib.mv_accept_speculative_lm(
        ddt, 1, 4, 100, d, 2, kw.get("par", P), 0, P, P, P, P, P, P, P, P, P, P, None, None, None,
        kw.get("ws", P), kw.get("wsn", 1 << 20), None)
    assert lm(7, 64) == L.MV_ERR_INVALID_ARG                   # draft dtype
    assert lm(L.MV_F32, 60) == L.MV_ERR_UNSUPPORTED            # d % 32
    assert lm(L.MV_F32, 40) == L.MV_ERR_UNSUPPORTED
    assert lm(L.MV_F32, 64, par=None) == L.MV_ERR_INVALID_ARG
    assert lm(L.MV_F32, 64, ws=None, wsn=0) == L.MV_ERR_WORKSPACE
    assert lib.mv_accept_speculative_lm_workspace(64, 64, 128256) > 64 * 128256 * 8
    # dynamic tree
    dyn = lambda D, smax, s, N: lib.mv_build_dynamic_tree(
        1, D, smax, L.int_array(s) if s else None, N, P, P, None, P, P, P, P, None, None, None)
    assert dyn(16, 4, None, 8) == L.MV_ERR_UNSUPPORTED          # depth above 15
    assert dyn(2, 17, None, 8) == L.MV_ERR_UNSUPPORTED          # more than 16 candidates
    assert dyn(2, 4, [2, 2], 7) == L.MV_ERR_INVALID_ARG         # 2 + 4 = 6 paths < 7 nodes
    assert dyn(2, 4, [5, 2], 8) == L.MV_ERR_INVALID_ARG         # width above s_max
    # KV commit
    kv = lambda dh, L_cap, D, pre=P, out=P: lib.mv_kv_commit(
        L.MV_BF16, 1, 8, dh, L_cap, 8, D, P, P, pre, out, P, P, None, None)
    assert kv(96, 200, 4) == L.MV_ERR_UNSUPPORTED
    assert kv(128, 7, 4) == L.MV_ERR_INVALID_ARG
    assert kv(128, 200, 17) == L.MV_ERR_UNSUPPORTED
    assert kv(128, 200, 4, pre=None) == L.MV_ERR_INVALID_ARG
    assert kv(128, 200, 4, out=None) == L.MV_ERR_INVALID_ARG
    # LM head
    args = (P, P, P, None, None, P, 1 << 30, None)
    assert lib.mv_lm_head_argmax(L.MV_F32, 65, 4096, 32000, *args) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_lm_head_argmax(L.MV_BF16, 65, 4080, 32000, *args) == L.MV_ERR_UNSUPPORTED
    assert lib.mv_lm_head_argmax(L.MV_BF16, 0, 4096, 32000, *args) == L.MV_ERR_INVALID_ARG
    assert lib.mv_lm_head_argmax(L.MV_BF16, 65, 4096, 32000, P, P, None, None, None, P, 1 << 30,
                                 None) == L.MV_ERR_INVALID_ARG
    assert lib.mv_lm_head_argmax(L.MV_BF16, 65, 4096, 32000, P, P, P, None, None, None, 0,
                                 None) == L.MV_ERR_WORKSPACE


def test_host_tree_validation():
    from medusa_tree_attention_verify_amd.ops import validate_parents
    validate_parents([-1, 0, 1, 1, 0, -1, 5])
    for bad in ([0], [-1, 1], [-1, -2], [], list(range(-1, 256))):
        with pytest.raises(ValueError):
            validate_parents(bad)
