"""AddressSanitizer + UndefinedBehaviorSanitizer over the CPU test suite.

The host-side C and C++ -- the oracle (oracle.c) and libada's argument
checks, pack planning and launch glue (ada_abi.cpp) -- are rebuilt with
-fsanitize=address,undefined in a scratch copy of the tree, and the whole
`-m "not gpu"` suite runs there with the sanitizer runtime preloaded.  Any
report fails the test.  The gfx950 kernel objects are built without
sanitizers (device code cannot take them); only their host launch stubs are
linked in, and no CPU test launches them.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INNER = "ADA_SANITIZER_INNER_RUN"

pytestmark = pytest.mark.slow

SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(os.environ.get(INNER) == "1", reason="inside the sanitized run itself")
@pytest.mark.skipif(shutil.which("hipcc") is None or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    work = tmp_path / "tree"
    ign = shutil.ignore_patterns("_build", "*.so", "*.so.tmp", "__pycache__", ".pytest_cache")
    for d in ("compressed_kv_attention_amd", "include", "oracle", "synth", "tests"):
        shutil.copytree(os.path.join(ROOT, d), work / d, ignore=ign)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), work / "pytest.ini")
    pkg = work / "compressed_kv_attention_amd"
    sys.path.insert(0, str(work))
    try:
        import importlib.util
        spec = importlib.util.spec_from_file_location("_san_build", pkg / "build.py")
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
    finally:
        sys.path.pop(0)
    digest = b.source_digest()
    objdir = work / "objs"
    objdir.mkdir()
    objs = []
    # kernels: the ordinary gfx950 build
    for src in b.SOURCES:
        if src.endswith(".hip"):
            o = str(objdir / (src[:-4] + ".o"))
            _run(["hipcc", *b.FLAGS, "-c", str(pkg / "csrc" / src), "-o", o])
            objs.append(o)
    # host entry points: g++ with the sanitizers
    abi_o = str(objdir / "ada_abi.o")
    host = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
            f'-DADA_BUILD_ID="{digest}"', "-I/opt/rocm/include", "-I", str(work / "include"),
            "-I", str(pkg / "csrc"), "-c", str(pkg / "csrc" / "ada_abi.cpp"), "-o", abi_o]
    _run(host + SAN)
    link = ["g++", "-shared", "-o", str(pkg / "libada.so"), abi_o, *objs, "-L/opt/rocm/lib",
            "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    _run(link + SAN)
    # the oracle with the sanitizers
    orc = ["gcc", "-O1", "-g", "-std=c99", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-o", str(work / "oracle" / "liboracle.so"), str(work / "oracle" / "oracle.c"),
           "-lm", "-lpthread"]
    _run(orc + SAN)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    env = dict(os.environ)
    env.update({INNER: "1", "LD_PRELOAD": libasan,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:"
                                "detect_odr_violation=0:abort_on_error=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "HIP_VISIBLE_DEVICES": "", "PYTHONDONTWRITEBYTECODE": "1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=work, env=env, capture_output=True, text=True,
                       timeout=1500)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-6000:]
    for bad in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert bad not in log, log[-6000:]
    assert " passed" in log
