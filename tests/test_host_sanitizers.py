"""Host sanitizers over the C ABI's argument checking.

api.cpp (every C-ABI entry point: descriptor and size validation, error
strings, workspace arithmetic) is rebuilt with AddressSanitizer and
UndefinedBehaviorSanitizer, linked with the in-tree kernel objects into a
separate library, and the host-only ABI suite (tests/test_abi.py) is run
against it in a child process. Only host code is instrumented (g++, no GPU
code is rebuilt), and no call in that suite reaches a kernel launch.

A positive control first checks that the same flags catch a planted heap
overflow and a planted signed overflow in a throwaway program, so a passing
run means the instrumented library was exercised, not that the sanitizers
were inert.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_ffn_expert_amd")
BUILD = os.path.join(PKG, "_build")
KERNEL_OBJS = ["route.hip.o", "gemm.hip.o", "combine.hip.o", "pack.hip.o", "keepquant.hip.o",
               "probe.hip.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _env(asan):
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@pytest.fixture(scope="module")
def toolchain():
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("the sanitizer runtimes are not installed")
    if not os.path.isdir("/opt/rocm/include"):
        pytest.skip("ROCm headers not found")
    missing = [o for o in KERNEL_OBJS if not os.path.exists(os.path.join(BUILD, o))]
    if missing:
        pytest.skip(f"kernel objects not built ({missing}); run __graft_entry__.build() first")
    return asan


def test_sanitizers_catch_planted_errors(toolchain, tmp_path):
    src = tmp_path / "planted.cpp"
    src.write_text(textwrap.dedent("""
        #include <cstdlib>
        #include <cstring>
        int main(int argc, char** argv) {
          if (argv[1][0] == 'h') {                  // heap overflow
            char* p = (char*)malloc(8);
            memset(p, 0, 8 + argc);
            int r = p[0];
            free(p);
            return r;
          }
          int x = 0x7fffffff - 1 + argc;            // signed overflow
          return (x + argc) & 1;
        }
    """))
    exe = tmp_path / "planted"
    subprocess.run(["g++", *SAN, str(src), "-o", str(exe)], check=True, capture_output=True)
    for arg, marker in (("h", "AddressSanitizer"), ("s", "runtime error")):
        r = subprocess.run([str(exe), arg], capture_output=True, text=True,
                           env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0",
                                "UBSAN_OPTIONS": "halt_on_error=1"})
        assert r.returncode != 0 and marker in r.stderr, (arg, r.returncode, r.stderr[-500:])


def test_abi_suite_under_asan_and_ubsan(toolchain, tmp_path):
    api_o = tmp_path / "api_san.o"
    subprocess.run(["g++", "-std=c++17", "-fPIC", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", f"-I{os.path.join(PKG, 'csrc')}",
                    "-c", os.path.join(PKG, "csrc", "api.cpp"), "-o", str(api_o)],
                   check=True, capture_output=True)
    lib = tmp_path / "libmoe_san.so"
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", str(api_o),
                    *[os.path.join(BUILD, o) for o in KERNEL_OBJS],
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(lib)],
                   check=True, capture_output=True)
    nm = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm, "library is not instrumented"
    runner = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import mixture_experts_ffn_expert_amd as moe
        moe._LIB_PATH = {str(lib)!r}
        import pytest
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                              {os.path.join(ROOT, "tests", "test_abi.py")!r}]))
    """)
    r = subprocess.run([sys.executable, "-c", runner], capture_output=True, text=True,
                       env=_env(toolchain), cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert r.returncode == 0, out[-3000:]
    assert " passed" in r.stdout, out[-2000:]
