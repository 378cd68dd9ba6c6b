"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer.

api.cpp (argument checks, workspace layouts, overlap checks, plans) is rebuilt with the
sanitizers on its host code only (each -fsanitize= follows -Xarch_host; the device code is not
instrumented), linked with the library's regular kernel objects, and the CPU ABI tests run
against that build in a child process with the sanitizer runtime preloaded.  No GPU is used:
every call those tests make is rejected, or answered, before any device work.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _device_objects(build, tmp):
    """The regular build's kernel objects, compiled into `tmp` if the in-tree build has none."""
    objs = []
    jobs = []
    for src in build.HIP_SOURCES:
        obj = os.path.join(build.BUILD, src + ".o")
        if not os.path.exists(obj):
            obj = os.path.join(tmp, src + ".o")
            jobs.append([build.hipcc()] + build.common_flags() + build.device_flags() +
                        ["-c", os.path.join(build.CSRC, src), "-o", obj])
        objs.append(obj)
    procs = [subprocess.Popen(j, stdout=subprocess.PIPE, stderr=subprocess.STDOUT) for j in jobs]
    for p, j in zip(procs, jobs):
        out = p.communicate()[0].decode(errors="replace")
        assert p.returncode == 0, f"{' '.join(j)}\n{out}"
    return objs


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    from efficient_transformer_attention_seq_amd import build
    rt = _asan_runtime()
    try:
        cc = build.hipcc()
    except RuntimeError:
        cc = None
    if cc is None or rt is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    tmp = str(tmp_path)
    api_obj = os.path.join(tmp, "api_san.o")
    flags = [f for f in build.common_flags() if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    r = subprocess.run([cc] + flags + build.device_flags() + san +
                       ["-c", os.path.join(build.CSRC, "api.cpp"), "-o", api_obj],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")
    lib = os.path.join(tmp, "liblinformer_san.so")
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={build.ARCH}", "-o", lib, api_obj] +
                       _device_objects(build, tmp), stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")
    # the binding is pointed at the sanitized build before the tests import it
    runner = ("import ctypes, sys; sys.path.insert(0, %r)\n"
              "ctypes.CDLL(None)['__asan_init']  # the runtime is loaded\n"
              "from efficient_transformer_attention_seq_amd import linformer as L\n"
              "L.LIB_PATH = %r\n"
              "import pytest\n"
              "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', %r]))\n"
              % (ROOT, lib, os.path.join(ROOT, "tests", "test_abi_cpu.py")))
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", runner], cwd=tmp, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    out = r.stdout.decode(errors="replace")
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
