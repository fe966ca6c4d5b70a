"""CPU sanitizer tier: the fp64 oracle and the C ABI's host code under
AddressSanitizer + UndefinedBehaviorSanitizer.

    python tests/run_sanitized.py

1. builds oracle/libmoe_oracle_san.so (gcc, -fsanitize=address,undefined,
   -fno-sanitize-recover) and runs tests/test_oracle_*.py against it, with
   gcc's libasan preloaded into the Python process;
2. builds router_gemm_amd/librouter_gemm_amd_san.so (hipcc, the sanitizers on
   the host code only: -Xarch_host -fsanitize=...) and runs tests/test_abi.py
   against it (argument validation, workspace sizing, every refusal path and
   the exported symbols), with clang's ASan runtime preloaded.

Leak detection is off (the Python interpreter and torch hold allocations until
exit); any other report aborts the run.  No GPU is used: the ABI tests stop
at the host-side checks.  Exit status 0 means both runs passed clean.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _gcc_asan() -> str:
    return subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()


def _clang_asan() -> str:
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
                   + glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found")
    return found[-1]


def _run(env_extra: dict, tests: list) -> int:
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    print("+", " ".join(f"{k}={v}" for k, v in env_extra.items()), " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=ROOT, env=env)


# A child process that hands the sanitized oracle a scale buffer one group too
# short: AddressSanitizer must stop it with a heap-buffer-overflow report,
# which shows the instrumentation is live in this setup.
_OVERFLOW = """
import numpy as np
import oracle
v = np.ones(256, dtype=np.float32)
q = np.zeros(256, dtype=np.uint8)
s = np.zeros(1, dtype=np.float32)          # two 128-groups need two scales
oracle.lib().oref_quant_row(v.ctypes.data, 256, q.ctypes.data, s.ctypes.data)
print("no report")
"""


def _sanitizer_is_live() -> bool:
    env = dict(os.environ, LD_PRELOAD=_gcc_asan(), MOE_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0")
    r = subprocess.run([sys.executable, "-c", _OVERFLOW], cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def main() -> int:
    import oracle
    from router_gemm_amd import build as hb

    oracle.build(sanitize=True)
    hb.build(verbose=True, sanitize=True)
    if not _sanitizer_is_live():
        print("AddressSanitizer did not report a planted out-of-bounds write: the runs below would "
              "prove nothing", flush=True)
        return 3
    print("AddressSanitizer reports a planted out-of-bounds write (the instrumentation is live)", flush=True)
    rc = _run({"LD_PRELOAD": _gcc_asan(), "MOE_ORACLE_SANITIZE": "1"},
              sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))))
    if rc != 0:
        print(f"oracle tests under the sanitizers: exit {rc}", flush=True)
        return rc
    rc = _run({"LD_PRELOAD": _clang_asan(), "MOE_SANITIZED_HOST": "1"}, [os.path.join(ROOT, "tests", "test_abi.py")])
    if rc != 0:
        print(f"ABI tests under the sanitizers: exit {rc}", flush=True)
        return rc
    print("sanitizer runs clean", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
