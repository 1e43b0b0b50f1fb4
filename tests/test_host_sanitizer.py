"""Host code under UndefinedBehaviorSanitizer and AddressSanitizer.

The library is rebuilt with a sanitizer on the host side only (device code unchanged), then a
child process loads that build and runs every host-side ABI case of test_abi.py: argument
validation, workspace and plan arithmetic, status strings, tree-spec validation.
* UBSan in trap mode: undefined behaviour (signed overflow, bad shifts, out-of-range
  conversions, misaligned or null accesses the checks can see) traps.
* ASan (the shared runtime, preloaded into the child): out-of-bounds reads and writes of host
  arrays (the per-call parameter blocks, the tree-spec checks, the workspace carving) and
  use-after-free abort the child.  Leak checking is off: the interpreter itself never frees
  some of its memory.
The child's exit status fails the test.  No GPU is needed: every call fails its host checks
before a launch, or only sizes a workspace.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

UBSAN_HOST = ["-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fsanitize-trap=undefined"]
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan",
             "-Xarch_host", "-fno-omit-frame-pointer"]

CASES = ("test_header_symbols_exported", "test_header_constants_match_binding",
         "test_status_strings", "test_workspace_queries", "test_host_argument_checks",
         "test_host_tree_validation")


def _asan_runtime():
    pats = ["/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
            "/opt/rocm-*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for p in pats:
        hits = sorted(glob.glob(p))
        if hits:
            return hits[-1]
    return None


def _run_cases(lib, env=None):
    code = "\n".join([
        "import sys",
        f"sys.path.insert(0, {ROOT!r})",
        "from medusa_tree_attention_verify_amd import _lib",
        f"_lib.LIB_PATH = {lib!r}",
        "import tests.test_abi as t",
        f"for name in {CASES!r}:",
        "    getattr(t, name)()",
        "    print('ok', name, flush=True)",
    ])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600,
                       cwd=ROOT, env=env)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.count("ok ") == len(CASES), r.stdout


def test_host_checks_under_ubsan(tmp_path):
    from medusa_tree_attention_verify_amd import build as B
    lib = B.build(out_path=str(tmp_path / "libmedusa_verify_ubsan.so"), extra_flags=UBSAN_HOST,
                  objdir=str(tmp_path / "obj"))
    _run_cases(lib)


def test_host_checks_under_asan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's shared ASan runtime is not installed")
    from medusa_tree_attention_verify_amd import build as B
    lib = B.build(out_path=str(tmp_path / "libmedusa_verify_asan.so"), extra_flags=ASAN_HOST,
                  objdir=str(tmp_path / "obj"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    _run_cases(lib, env)
