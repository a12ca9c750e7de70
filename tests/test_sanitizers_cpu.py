"""The oracle, the seeded input generators and the C-ABI host code under
AddressSanitizer + UndefinedBehaviorSanitizer, on the CPU.

Instrumented copies are built into a temporary folder: liboracle.so and
libsynth.so from their C sources (clang, serial), and the library with
abi.hip's host code instrumented (-Xarch_host, the device code untouched),
linked with the kernel objects of the regular build.  The CPU suite then runs
against them in a child process with clang's ASan runtime preloaded, any
report aborting it.  A control case first checks that this set-up does catch
a heap overflow.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_expert_ffn_wave_amd", "csrc")
OBJS = os.path.join(CSRC, "_build")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

def library_sources():
    """The library's source list, from its build script (loaded by path)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_moe_build", os.path.join(ROOT, "quantized_expert_ffn_wave_amd",
                                                                             "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.SOURCES


# the kernel objects linked beside the instrumented abi.hip (all but abi.o)
KERNEL_OBJS = [s.replace(".hip", ".o") for s in library_sources() if s != "abi.hip"]
# the one test whose full-size routing sweep takes most of a minute serially
SLOW = "test_full_size_uniform_routing_touches_expected_expert_count"


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


pytestmark = [
    pytest.mark.skipif(os.environ.get("MOE_SANITIZED_RUN") == "1", reason="already inside the instrumented run"),
    pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                       reason="another library is preloaded here; the ASan runtime has to come first"),
    pytest.mark.skipif(asan_runtime() is None or not os.path.exists(CLANG), reason="ROCm clang sanitizer runtime missing"),
]


def run(cmd, **kw):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout[-4000:]
    return res


def child_env(**libs):
    env = dict(os.environ)
    env.update(libs)
    env.update(LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", MOE_SANITIZED_RUN="1")
    return env


@pytest.fixture(scope="module")
def instrumented(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    orc, syn = str(d / "liboracle.so"), str(d / "libsynth.so")
    run([CLANG, "-O1", "-g", "-ffp-contract=off", *SAN, "-fPIC", "-shared", "-o", orc,
         os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    run([CLANG, "-O1", "-g", "-ffp-contract=off", *SAN, "-fPIC", "-shared", "-o", syn,
         os.path.join(ROOT, "synth", "synth.c"), "-lm"])
    missing = [o for o in KERNEL_OBJS if not os.path.exists(os.path.join(OBJS, o))]
    if missing:
        pytest.skip(f"kernel objects {missing} not built (run the library build first)")
    abi_o, lib = str(d / "abi.o"), str(d / "libmoe_ffn.so")
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "abi.hip"), "-o", abi_o])
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, abi_o,
         *[os.path.join(OBJS, o) for o in KERNEL_OBJS]])
    return dict(MOE_ORACLE_LIB=orc, MOE_SYNTH_LIB=syn, MOE_FFN_LIB=lib, dir=str(d))


def test_control_overflow_is_reported(instrumented):
    """A planted heap overflow in a library built the same way aborts the child
    with an ASan report (so a clean run below means something)."""
    src = os.path.join(instrumented["dir"], "planted.c")
    with open(src, "w") as f:
        f.write("#include <stdlib.h>\nint planted(int n) { int* a = malloc(sizeof(int) * n);"
                " for (int i = 0; i < n; ++i) a[i] = i; int v = a[n]; free(a); return v; }\n")
    so = os.path.join(instrumented["dir"], "libplanted.so")
    run([CLANG, "-O0", "-g", *SAN, "-fPIC", "-shared", "-o", so, src])
    code = f"import ctypes; print(ctypes.CDLL({so!r}).planted(4))"
    res = subprocess.run([sys.executable, "-c", code], env=child_env(), stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=120)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stdout


def test_child_loads_the_instrumented_copies(instrumented):
    libs = {k: v for k, v in instrumented.items() if k.startswith("MOE_")}
    code = ("import oracle, synth, quantized_expert_ffn_wave_amd as m; oracle.lib(); synth.lib(); m.lib();"
            "print(open('/proc/self/maps').read())")
    res = subprocess.run([sys.executable, "-c", code], env=child_env(**libs), cwd=ROOT, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-3000:]
    for path in libs.values():
        assert path in res.stdout, path
    for name in ("oracle/liboracle.so", "synth/libsynth.so", "quantized_expert_ffn_wave_amd/libmoe_ffn.so"):
        assert os.path.join(ROOT, name) not in res.stdout, name


def test_cpu_suite_is_clean_under_asan_and_ubsan(instrumented):
    libs = {k: v for k, v in instrumented.items() if k.startswith("MOE_")}
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
           "-p", "no:cacheprovider", "-k", f"not built_for_gfx950 and not {SLOW} and not sanitizers"]
    res = subprocess.run(cmd, env=child_env(**libs), cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=900)
    tail = res.stdout[-6000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stdout and "runtime error:" not in res.stdout, tail
    assert " passed" in tail
