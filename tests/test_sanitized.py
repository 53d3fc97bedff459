"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two runs, each in a child process with its sanitizer runtime preloaded:
  * the oracle (oracle/dsa_oracle.c) and the input generator (dsa_inputs/gen.c)
    built with gcc -fsanitize=address,undefined, driving tests/test_oracle.py;
  * libdsa.so with every host part built with clang's ASan and UBSan (device
    code is built as usual), driving tests/test_abi.py: the argument checks,
    workspace sizes and status paths of the C ABI.
A sanitizer report aborts the child, and the test fails with its output.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_02_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _child_env(preload, **extra):
    env = dict(os.environ)
    env.update(extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    return env


def test_oracle_and_generator_under_gcc_sanitizers(tmp_path):
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared", "-fopenmp", "-std=c11",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    oracle_so = str(tmp_path / "liboracle_san.so")
    gen_so = str(tmp_path / "libdsa_inputs_san.so")
    _run(["gcc", *flags, os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-o", oracle_so, "-lm"])
    _run(["gcc", *flags, os.path.join(ROOT, "dsa_inputs", "gen.c"), "-o", gen_so, "-lm"])
    libasan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    libubsan = _run(["gcc", "-print-file-name=libubsan.so"]).stdout.strip()
    env = _child_env(f"{libasan}:{libubsan}", DSA_ORACLE_LIBRARY=oracle_so, DSA_INPUTS_LIBRARY=gen_so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-6000:] + r.stderr[-6000:]
    assert "passed" in r.stdout


def _clang_asan_runtime():
    r = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        for base, _, files in os.walk("/opt/rocm/llvm/lib/clang"):
            if "libclang_rt.asan-x86_64.so" in files:
                return os.path.join(base, "libclang_rt.asan-x86_64.so")
        return None
    return path


def test_c_abi_host_code_under_clang_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    runtime = _clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang ASan runtime not found")
    sources = ["indexer.hip", "topk.hip", "sparse_mla.hip", "attn_bwd.hip", "warmup.hip", "index_bwd.hip",
               "dsa_api.cpp"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        _run([HIPCC, *common, *san, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, sources))
    lib = str(tmp_path / "libdsa_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, *objs, "-o", lib])
    env = _child_env(runtime, DSA_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-6000:] + r.stderr[-6000:]
    assert "passed" in r.stdout
