"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (plain C) is built with gcc's sanitizers and the oracle pin suites
run against it; the C ABI of the HIP library is built with its host code
sanitized (clang, host side only) and the host-side ABI tests (argument
validation, sizes, error paths) run against it (device code is compiled as usual but never launched: every call in
those tests is rejected on the host, or finds no device).  Any out-of-bounds
access, use of undefined behaviour (signed overflow,
misaligned access, bad shifts, ...) aborts the run.  A planted out-of-bounds
write in a copy of the oracle shows that the sanitized build does catch one.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
CSRC = os.path.join(ROOT, "ternary_weight_absmean_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ORACLE_PINS = ["test_oracle_absmean.py", "test_oracle_act_linear.py", "test_oracle_glu.py",
               "test_oracle_backward.py", "test_oracle_b3.py"]


def gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_oracle(src, out):
    # gcc, host C only (no HIP source on this line)
    cmd = ["gcc", "-O1", "-g", "-std=gnu11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def run_pytest(files, env):
    # -s: a sanitizer report goes to the process's stderr, not to pytest's capture
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", *files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def asan_env():
    libasan = gcc_runtime("libasan.so")
    if libasan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def test_oracle_pins_pass_under_asan_and_ubsan(asan_env, tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    build_oracle(ORACLE_C, so)
    res = run_pytest([os.path.join("tests", f) for f in ORACLE_PINS], dict(asan_env, BITLINEAR_ORACLE_SO=so))
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]


def test_planted_out_of_bounds_write_is_caught(asan_env, tmp_path):
    with open(ORACLE_C) as f:
        src = f.read()
    site = "    for (int64_t b = 0; b < total; ++b) packed[b] = orc_b3_encode(trits + 5 * b);"
    assert src.count(site) == 1
    bad = tmp_path / "oracle_oob.c"
    bad.write_text(src.replace(site, site + "\n    packed[total] = 0;  /* planted: one byte past the buffer */"))
    so = str(tmp_path / "liboracle_oob.so")
    build_oracle(str(bad), so)
    res = run_pytest([os.path.join("tests", "test_oracle_b3.py")], dict(asan_env, BITLINEAR_ORACLE_SO=so))
    assert res.returncode != 0 and "AddressSanitizer" in (res.stdout + res.stderr)


def test_abi_host_checks_pass_under_asan_and_ubsan(tmp_path):
    rt = clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("clang's AddressSanitizer runtime or hipcc is missing")
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    sources = [s for s in sources if not s.endswith("measure.hip")]
    procs, objs = [], []
    for src in sources:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # host side only: each sanitizer flag goes to the host compilation
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-2000:]
    so = str(tmp_path / "libbitlinear_san.so")
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", *objs, "-o", so]
    subprocess.run(link, check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", BITLINEAR_LIB=so)
    res = run_pytest([os.path.join("tests", "test_abi_host.py")], env)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
