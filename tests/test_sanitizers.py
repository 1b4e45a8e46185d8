"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only, no GPU).

Two host libraries are rebuilt with ``-fsanitize=address,undefined`` (gcc/g++,
no device code) and the CPU suites that exercise them run against them in a
subprocess:

* the C oracle (oracle/lightning_oracle.c) under tests/test_oracle.py;
* the C ABI's host side, lightning_api.cpp (every entry point's argument,
  size-overflow and alias checks and the launch planning), linked with
  tests/host_stubs.cpp in place of the device launchers, under
  tests/test_abi.py.

Each run uses a scratch copy of the repository layout: symlinks to tests/,
include/, the kernel sources and workloads.py, and copies of the oracle and
binding packages holding the sanitized libraries. The tests' conftest puts that
root first on sys.path, so the copies shadow the regular builds. Any sanitizer
report aborts the run (``-fno-sanitize-recover=all``, ``halt_on_error``); leak
checking is off (the interpreter itself is not instrumented).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _have(tool):
    return shutil.which(tool) is not None


pytestmark = pytest.mark.skipif(not (_have("gcc") and _have("g++")), reason="needs gcc and g++")


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True, check=True)
    path = out.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no shared AddressSanitizer runtime")
    return path


def _layout(tmp):
    """Scratch root: links to the shared parts of the tree."""
    root = os.path.join(tmp, "root")
    os.makedirs(root)
    for name in ("tests", "include", "workloads.py"):
        os.symlink(os.path.join(ROOT, name), os.path.join(root, name))
    return root


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    return env


def _mapped(root, load):
    """Shared objects mapped in a process of the suite's environment after `load`."""
    code = ("import sys; sys.path.insert(0, %r)\n%s\n"
            "print('\\n'.join(sorted({l.split()[-1] for l in open('/proc/self/maps') if '.so' in l})))") % (root, load)
    res = subprocess.run([sys.executable, "-c", code], cwd=root, env=_env(), capture_output=True, text=True,
                         timeout=120, check=True)
    return res.stdout.split()


def _run_suite(root, test_file):
    env = _env()
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(root, "tests", test_file)],
                         cwd=root, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    root = _layout(str(tmp_path))
    odir = os.path.join(root, "oracle")
    os.makedirs(odir)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), odir)
    src = shutil.copy(os.path.join(ROOT, "oracle", "lightning_oracle.c"), odir)
    lib = os.path.join(odir, "liblightning_oracle.so")  # newer than the source: not rebuilt
    subprocess.run(["gcc"] + SAN + ["-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra", src, "-o", lib],
                   check=True)
    maps = _mapped(root, "import oracle; oracle._load()")
    assert lib in maps and any("libasan" in m for m in maps), maps
    out = _run_suite(root, "test_oracle.py")
    assert " passed" in out


def test_api_validation_under_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from linear_attention_amd import build as b

    root = _layout(str(tmp_path))
    os.symlink(os.path.join(ROOT, "oracle"), os.path.join(root, "oracle"))
    pkg = os.path.join(root, "linear_attention_amd")
    os.makedirs(pkg)
    for name in os.listdir(b.PKG):
        if name.endswith(".py"):
            shutil.copy(os.path.join(b.PKG, name), pkg)
    os.symlink(b.CSRC, os.path.join(pkg, "csrc"))
    # the build identity of the tree, so that the fixtures take this library as current
    cmd = ["g++", "-std=c++17"] + SAN + [
        "-fPIC", "-shared", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
        "-I", os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include"), "-I", b.INCLUDE, "-I", b.CSRC,
        '-DLT_BUILD_ID="%s"' % b.source_hash(),
        os.path.join(b.CSRC, "lightning_api.cpp"), os.path.join(ROOT, "tests", "host_stubs.cpp"),
        "-Wl,--no-undefined", "-o", os.path.join(pkg, "liblightning.so")]
    subprocess.run(cmd, check=True)
    maps = _mapped(root, "import linear_attention_amd as la; la.lib")
    assert os.path.join(pkg, "liblightning.so") in maps and any("libasan" in m for m in maps), maps
    out = _run_suite(root, "test_abi.py")
    assert " passed" in out
