"""The CPU tier again under AddressSanitizer and UndefinedBehaviorSanitizer
(gcc's; no GPU involved):
  * the oracle built with both sanitizers runs every pin, and every planted
    mistake is built with them too and still caught;
  * a planted out-of-bounds read in a call of the sanitized oracle is
    reported (the tier is live);
  * the host side of libqmv -- argument validation, the device check and
    status strings, compiled with both sanitizers and linked with the
    unchanged kernel objects -- runs the ABI tests (every bad shape, null
    or misaligned pointer returns its status; with no GPU every valid call
    returns QMV_E_DEVICE).
Each runs in a child Python with the sanitizer runtime preloaded; any
report aborts the child."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import oracle as orc  # noqa: E402

SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ORACLE_FLAGS = [f for f in orc.CFLAGS if not f.startswith("-O")] + SAN


def _env():
    env = dict(os.environ)
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests")])
    return env


def _child(script: str, tmp_path, timeout=600):
    path = tmp_path / "child.py"
    path.write_text(script)
    return subprocess.run([sys.executable, str(path)], env=_env(), capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def _sanitized_oracle(src: str, out: str) -> str:
    c = out + ".c"
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", *ORACLE_FLAGS, c, "-o", out, "-lm"])
    return out


def _no_reports(r):
    text = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    so = _sanitized_oracle(open(os.path.join(ROOT, "oracle", "qmv_oracle.c")).read(), str(tmp_path / "orc_san.so"))
    script = f"""
import pins
from oracle import oracle as orc
with orc.use_build({so!r}):
    bad = pins.failing_checks()
assert not bad, bad
print("ok")
"""
    r = _child(script, tmp_path)
    _no_reports(r)
    assert "ok" in r.stdout


def test_planted_mistakes_under_sanitizers(tmp_path):
    """Each planted mistake, built with the sanitizers, is caught: by a pin,
    or by a sanitizer report where the mistake reads out of bounds."""
    from test_oracle_mutants import MUTANTS, SRC, _apply
    src = open(SRC).read()

    def one(m):
        name, old, new, count = m
        d = tmp_path / name
        d.mkdir()
        so = _sanitized_oracle(_apply(src, old, new, count), str(d / "mut.so"))
        script = f"""
import pins
from oracle import oracle as orc
with orc.use_build({so!r}):
    print("caught" if pins.failing_checks() else "missed")
"""
        r = _child(script, d)
        text = r.stdout + r.stderr
        if r.returncode == 0:
            return name, "caught" in r.stdout
        return name, ("ERROR: AddressSanitizer" in text or "runtime error:" in text)

    with cf.ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, MUTANTS))
    missed = [n for n, ok in res if not ok]
    assert not missed, missed


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    so = _sanitized_oracle(open(os.path.join(ROOT, "oracle", "qmv_oracle.c")).read(), str(tmp_path / "orc_san.so"))
    script = f"""
import numpy as np
from oracle import oracle as orc
with orc.use_build({so!r}) as L:
    x = np.zeros(64, np.float32)
    q = np.zeros(64, np.int8)
    d = np.zeros(2, np.float32)
    L.orc_quantize_q8(x.ctypes.data, 96, q.ctypes.data, d.ctypes.data)  # claims a third block
print("not reported")
"""
    r = _child(script, tmp_path)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.stdout + r.stderr)[-2000:]


def test_host_library_under_sanitizers(tmp_path):
    from block_quantized_decode_amd import build
    csrc = os.path.join(ROOT, "block_quantized_decode_amd", "csrc")
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    objs = [os.path.join(build.BUILD, os.path.basename(s) + ".o") for s in srcs]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(s) for s, o in zip(srcs, objs)):
        build.build()
    api = str(tmp_path / "qmv_api.o")
    subprocess.check_call(["g++", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I" + os.path.join(ROOT, "include"), "-I" + csrc, *SAN, "-c",
                           os.path.join(csrc, "qmv_api.cpp"), "-o", api])
    lib = str(tmp_path / "libqmv_san.so")
    subprocess.check_call(["g++", "-shared", "-fsanitize=address,undefined", api, *objs, "-L/opt/rocm/lib",
                           "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", lib])
    env = _env()
    env["QMV_ABI_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    _no_reports(r)
    assert " passed" in r.stdout, r.stdout[-2000:]
