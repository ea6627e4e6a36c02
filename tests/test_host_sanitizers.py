"""libgpt2's host runtime under the host compiler's address and
undefined-behaviour sanitizers, on the CPU: every HIP source of the library
and tests/host_checks.cpp are compiled with the sanitizers on the host side
only (device code as usual) and the checks run without a GPU -- every
configuration and argument check, and the host plan gpt2_init builds for
valid configurations (workspace layout, AdamW chunks and tiles, grouped
weight-gradient and column-sum tables) up to its first device call."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_only_transformer_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# each sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-munsafe-fp-atomics",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]


def _cc(src, out):
    cmd = [HIPCC, *FLAGS, *HOST_SAN, "-c", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_runtime_under_asan_ubsan(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(ROOT, "tests",
                                                                          "host_checks.cpp")]
    outs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda a: _cc(*a), zip(srcs, outs)))
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, *outs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode == 77:
        pytest.skip("a GPU is visible: these checks run on hosts without one")
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert "host checks passed" in r.stdout
