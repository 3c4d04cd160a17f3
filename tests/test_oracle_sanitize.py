"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only): a driver runs every oracle function on small inputs in
buffers of exactly the documented sizes, including the refused calls (a
repeated id, an id out of range) and the FFN over each token's true set
against the dense FFN.  Any out-of-bounds access, leak or undefined
arithmetic aborts the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_sanitizers():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    out = os.path.join(tempfile.mkdtemp(prefix="orc_san_"), "orc_san")
    flags = ["-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    cmd = [gcc] + flags + [os.path.join(ROOT, "oracle", "asf_oracle.c"),
                           os.path.join(HERE, "oracle_sanitize_main.c"), "-lm", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("no sanitizer runtime: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([out], capture_output=True, text=True, env=env, timeout=120)
    if p.returncode != 0 and "does not come first" in p.stderr:
        pytest.skip("a preloaded library keeps the sanitizer runtime from loading first")
    assert p.returncode == 0 and p.stdout.strip() == "ok", (p.stdout[-500:], p.stderr[-3000:])
