"""Run the CPU tests of the C boundary and of the oracle against builds with AddressSanitizer
and UndefinedBehaviorSanitizer on their host code.

  python tests/sanitize_cpu.py

builds, under _build/san/,
  * libmc_san.so: abi.cpp (the argument checks, workspace sizing and dispatch) compiled with
    -fsanitize=address,undefined (host code only), linked with the library's other objects
    from _build/ (run the package's build first);
  * libmc_oracle_san.so: oracle/mc_oracle.c compiled with clang and the same sanitizers;
then runs tests/test_abi_cpu.py and tests/test_oracle_pins.py with the sanitizer runtime
preloaded and MC_LIB / MC_ORACLE_LIB pointing at these builds.  Any report aborts the run
(-fno-sanitize-recover), so the exit status is the tests' and the sanitizers' verdict.
Leak detection is off: the Python interpreter itself is not built for it."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from chunked_linear_attention_segment_amd import build as b  # noqa: E402

LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]


def run(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def main() -> int:
    out = os.path.join(ROOT, "_build", "san")
    os.makedirs(out, exist_ok=True)
    objs = [os.path.join(b.BUILD_DIR, s + ".o") for s in b.SOURCES if s != "abi.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        print("build the package first (missing %s)" % missing[0])
        return 2
    abi_o = os.path.join(out, "abi_san.o")
    host = []
    for f in SAN:  # hipcc: every sanitizer flag applies to the host pass only
        host += ["-Xarch_host", f] if f.startswith("-fsanitize") else [f]
    run([b.HIPCC, "-O1", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-x", "c++"]
        + host + ["-c", os.path.join(b.CSRC, "abi.cpp"), "-o", abi_o])
    lib = os.path.join(out, "libmc_san.so")
    run([b.HIPCC, "-shared", "-fPIC", "--offload-arch=" + b.ARCH, "-shared-libsan",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-o", lib, abi_o] + objs)
    olib = os.path.join(out, "libmc_oracle_san.so")
    run([os.path.join(LLVM, "bin", "clang"), "-O1", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-shared", "-fPIC", "-shared-libsan"] + SAN +
        ["-o", olib, os.path.join(ROOT, "oracle", "mc_oracle.c"), "-lm",
         "-L" + os.path.join(LLVM, "lib"), "-Wl,-rpath," + os.path.join(LLVM, "lib")])
    rt = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                "libclang_rt.asan-x86_64.so"))
    if not rt:
        print("no AddressSanitizer runtime found under", LLVM)
        return 2
    env = dict(os.environ, LD_PRELOAD=rt[0], MC_LIB=lib, MC_ORACLE_LIB=olib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-m", "not gpu"]
    print("+", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
