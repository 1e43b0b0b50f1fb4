"""Host code under UndefinedBehaviorSanitizer.

The library is rebuilt with UBSan in trap mode on the host side only (device code unchanged),
then a child process loads that build and runs every host-side ABI case of test_abi.py:
argument validation, workspace and plan arithmetic, status strings, tree-spec validation.
Undefined behaviour (signed overflow, bad shifts, out-of-range conversions, misaligned or null
accesses the checks can see) traps, and the child's exit status fails the test.  No GPU is
needed: every call fails its host checks before a launch, or only sizes a workspace.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

UBSAN_HOST = ["-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fsanitize-trap=undefined"]

CASES = ("test_header_symbols_exported", "test_header_constants_match_binding",
         "test_status_strings", "test_workspace_queries", "test_host_argument_checks",
         "test_host_tree_validation")


def test_host_checks_under_ubsan(tmp_path):
    from medusa_tree_attention_verify_amd import build as B
    lib = B.build(out_path=str(tmp_path / "libmedusa_verify_ubsan.so"), extra_flags=UBSAN_HOST,
                  objdir=str(tmp_path / "obj"))
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
                       cwd=ROOT)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert r.stdout.count("ok ") == len(CASES), r.stdout
