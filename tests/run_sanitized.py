"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, next to the ordinary ones, sanitized copies of the oracle
(liboracle_san.so) and the input generator (libsynth_san.so) with clang, the
host emulator of the kernels (tests/emu/libnq_emu_san.so) and the library
with its host sources (the C ABI's validators and launchers) instrumented
(block_quantized_weight_nq_amd/libnq_san.so; device code as always), then
runs `pytest -m "not gpu"` against them with clang's sanitizer runtime
preloaded into the interpreter.  Any report stops the run (recovery off);
reports go to files in a fresh temporary folder, since pytest captures the
test process's stderr, and are printed once pytest has ended.  Leak checking
is off: the interpreter itself keeps its allocations.

Usage: python tests/run_sanitized.py [extra pytest arguments]
"""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")
    return libs[-1]


def main():
    env = dict(os.environ, NQ_SANITIZE="1")
    sys.path.insert(0, ROOT)
    os.environ["NQ_SANITIZE"] = "1"
    import oracle
    import synth
    from block_quantized_weight_nq_amd import build as nqbuild
    oracle.build()
    synth.build()
    san_lib = os.path.join(ROOT, "block_quantized_weight_nq_amd", "libnq_san.so")
    nqbuild.build(out=san_lib, sanitize=True)
    sys.path.insert(0, HERE)
    import emu_lib
    emu_lib.build()
    logs = tempfile.mkdtemp(prefix="nq_san_")
    env.update(NQ_TEST_LIB=san_lib, LD_PRELOAD=runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=1:halt_on_error=1:log_path={logs}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *sys.argv[1:]]
    print("running:", " ".join(cmd), flush=True)
    rc = subprocess.call(cmd, env=env, cwd=ROOT)
    reports = sorted(glob.glob(os.path.join(logs, "*")))
    for r in reports:
        print(f"--- sanitizer report {r}", flush=True)
        with open(r) as f:
            sys.stdout.write(f.read())
    print(f"sanitized run: pytest status {rc}, {len(reports)} sanitizer report(s)", flush=True)
    return rc or (1 if reports else 0)


if __name__ == "__main__":
    sys.exit(main())
