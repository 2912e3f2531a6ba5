"""The C oracle under sanitizers (no GPU): tests/sanitize_oracle.c drives every
oracle entry point on a small ragged, paged, split case with buffers of exact
size; built with AddressSanitizer + UndefinedBehaviorSanitizer (out-of-bounds
accesses, use after free, undefined arithmetic) and, separately, with
ThreadSanitizer (the oracle's pthread pool over (sequence, head) pairs)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "sanitize_oracle.c"), os.path.join(ROOT, "oracle", "mla_oracle.c")]


def _build_and_run(tmp_path, flags):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sanitized_oracle")
    build = subprocess.run([cc, "-O1", "-g", "-fno-omit-frame-pointer", *flags, *SOURCES, "-lm", "-lpthread",
                            "-o", exe], capture_output=True, text=True)
    if build.returncode != 0:
        if "cannot find" in build.stderr or "libasan" in build.stderr or "libtsan" in build.stderr:
            pytest.skip("sanitizer runtime not installed: " + build.stderr.strip()[:200])
        raise AssertionError(build.stderr)
    env = dict(os.environ)
    # (a process that already preloads a library still runs the instrumented code)
    env["ASAN_OPTIONS"] = "verify_asan_link_order=0"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr


def test_oracle_clean_under_address_and_undefined_sanitizers(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


def test_oracle_thread_pool_clean_under_thread_sanitizer(tmp_path):
    _build_and_run(tmp_path, ["-fsanitize=thread"])
