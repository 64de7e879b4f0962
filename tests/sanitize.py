"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

    python tests/sanitize.py

Builds, under _build/sanitize/:
  * the oracle (oracle.c) with gcc, -fsanitize=address,undefined;
  * libdh.so with hipcc, the host side of every source with -fsanitize=address,undefined
    (each flag after -Xarch_host, so no GPU code is built with a sanitizer): the C ABI's
    argument checks, the launchers and the binding's marshalling.
Then runs ``pytest -m "not gpu"`` twice, once with each sanitized library in place of the
regular one (gcc's and clang's sanitizer runtimes cannot share a process, so each run
preloads its own runtime).  Leak detection is off (the Python interpreter is not built for
it); any address or undefined-behaviour report fails the run.  CPU only: the GPU tests are
deselected, and with no GPU visible every libdh call in them is a host-side refusal.
"""
import glob
import os
import subprocess
import sys
import textwrap

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]

PLUGIN = textwrap.dedent('''\
    """pytest plugin: load the sanitized libraries named by the environment."""
    import os


    def pytest_configure(config):
        p = os.environ.get("DH_SANITIZED_ORACLE")
        if p:
            import oracle.build
            oracle.build.LIB = p
        q = os.environ.get("DH_SANITIZED_LIBDH")
        if q:
            from few_row_vocab_amd import dh
            dh.LIB_PATH = q
    ''')


def run(cmd, **kw):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def build_oracle():
    from oracle import build as ob
    lib = os.path.join(OUT, "liboracle.so")
    flags = [f for f in ob.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                    "-fsanitize=address,undefined",
                                                    "-fno-sanitize-recover=all"]
    run(["gcc", *flags, ob.SRC, "-o", lib, "-lm"])
    return lib


def build_libdh():
    from few_row_vocab_amd import build as lb
    objs = []
    procs = []
    for src in lb.sources():
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *lb.FLAGS, *SAN_HOST, "-c", src, "-o", obj]
        print("+", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.DEVNULL))
    for p in procs:
        if p.wait() != 0:
            raise SystemExit("a sanitized compile failed")
    lib = os.path.join(OUT, "libdh.so")
    run([HIPCC, f"--offload-arch={lb.ARCH}", "-shared", "-fPIC", *SAN_HOST,
         "-Xarch_host", "-shared-libasan", *objs, "-o", lib])
    return lib


def clang_asan_runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime was not found")
    return found[0]


def suite(env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = OUT + os.pathsep + env.get("PYTHONPATH", "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x",
         "-m", "not gpu", "-p", "dh_sanitized_paths"], env=env, cwd=ROOT)


def main():
    os.makedirs(OUT, exist_ok=True)
    with open(os.path.join(OUT, "dh_sanitized_paths.py"), "w") as f:
        f.write(PLUGIN)
    orc = build_oracle()
    dhl = build_libdh()
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    print("== the oracle under gcc's AddressSanitizer + UndefinedBehaviorSanitizer", flush=True)
    suite({"LD_PRELOAD": gcc_asan, "DH_SANITIZED_ORACLE": orc})
    print("== libdh's host code under clang's AddressSanitizer + UndefinedBehaviorSanitizer",
          flush=True)
    suite({"LD_PRELOAD": clang_asan_runtime(), "DH_SANITIZED_LIBDH": dhl})
    print("sanitized CPU suite: green", flush=True)


if __name__ == "__main__":
    main()
