"""The C ABI layer and the host side of every launcher, built for the host only with
AddressSanitizer and UndefinedBehaviorSanitizer and run without a GPU.

`tests/host_asan/abi_driver.cpp` calls every entry point of include/bd.h: each argument check
(NULL pointers, bad and overflowing sizes, unsupported combinations, NaN scalars, short
workspaces, misalignment) with the status the header states, the workspace-size queries at
extreme sizes, and valid calls, which run the launchers' host code (plans, grids, chunking)
up to the launch.  `tests/host_asan/hip_runtime_stub.cpp` stands in for the HIP runtime:
registrations are no-ops and each launch is checked for a launchable shape and counted, never
run.  Any sanitizer report aborts the driver.  Needs hipcc (ROCm) on the host; no GPU.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_decoding_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = os.environ.get("HOST_CLANG", "/opt/rocm/llvm/bin/clang++")

# Host-only compilation; each sanitizer flag is scoped to the host side explicitly.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
COMPILE = [HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SAN]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    out = tmp_path_factory.mktemp("host_asan")
    sources = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith((".hip", ".cpp"))]
    sources += [os.path.join(HERE, "hip_runtime_stub.cpp"), os.path.join(HERE, "abi_driver.cpp")]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        _run([*COMPILE, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources))
    # Each host-only object refers to its (absent) device code object by one symbol; define them empty.
    undefined = _run(["nm", "-u", *objs]).stdout
    fatbins = sorted(set(re.findall(r"\b(__hip_fatbin_\w+)", undefined)))
    stub = os.path.join(out, "fatbin_symbols.cpp")
    with open(stub, "w") as f:
        for name in fatbins:
            f.write(f'extern "C" const char {name}[16] = {{0}};\n')
    objs.append(os.path.join(out, "fatbin_symbols.o"))
    _run([CLANG, "-std=c++17", "-c", stub, "-o", objs[-1]])
    exe = os.path.join(out, "abi_driver")
    _run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe])
    return exe


def test_abi_checks_under_host_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-8000:]
    m = re.search(r"abi driver: (\d+) checks passed, (\d+) launches", r.stdout)
    assert m and int(m.group(1)) > 100 and int(m.group(2)) > 20, r.stdout
