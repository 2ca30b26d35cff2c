"""Host-side memory and undefined-behaviour checks (CPU only).

The oracle is rebuilt with gcc's AddressSanitizer and UndefinedBehavior-
Sanitizer (every report fatal) and its pins run against that build; the HIP
library is rebuilt with both sanitizers on its host pass and the C-ABI's
host-side tests (argument checks, workspace layout, ring layout, table
marshalling) run through it.  Each run is a child process with the
sanitizer runtime preloaded; a report ends it with a non-zero status."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(env_extra, args):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    import oracle
    lib = oracle.build(str(tmp_path / "libmok_oracle_san.so"), sanitize=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = {"LD_PRELOAD": asan, "MOK_ORACLE_LIB": lib}
    out = _run(env, ["-c", "import oracle; print(oracle.lib()._name)"])
    assert lib in out
    pins = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    _run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *pins])


def test_abi_host_checks_under_address_and_ub_sanitizers(tmp_path):
    from combine_router_top_expert_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not present")
    lib = build.build(out=str(tmp_path / "libmok_san.so"), sanitize=True)
    env = {"LD_PRELOAD": build.sanitizer_runtime(), "MOK_LIB": lib}
    out = _run(env, ["-c", "import combine_router_top_expert_amd as m; m.lib(); print(m.LIB_PATH)"])
    assert lib in out
    _run(env, ["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
               os.path.join(ROOT, "tests", "test_abi.py"),
               os.path.join(ROOT, "tests", "test_host_tools.py")])
