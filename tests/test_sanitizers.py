"""Host sanitizers (no GPU): the library's host code with the kernels' index
arithmetic run through the CPU emulator, and the oracle, each built with
AddressSanitizer and UndefinedBehaviorSanitizer (g++/gcc, host code only)
and run over tagged round trips, both modes and layouts, several launch
shapes and the validation paths."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_re_layout_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
       "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert res.returncode == 0 and res.stdout.strip().startswith("OK"), res.stdout[-3000:] + res.stderr[-3000:]


def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "emu_sanitize")
    subprocess.run(["g++", "-std=c++17", "-DBASP_HD="] + SAN +
                   ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "launch.cpp"),
                    os.path.join(ROOT, "tests", "emu", "kernel_emu.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "emu_sanitize.cpp"), "-o", exe], check=True)
    run(exe)


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11"] + SAN +
                   [os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize.c"), "-o", exe], check=True)
    run(exe)
