"""CPU checks of the library's host code and device code objects.

1. The C-ABI's argument checks, step packing and block sequencing (api.cpp) built for
   the host with the address and undefined-behaviour sanitizers, linked with launcher
   stand-ins that record each launch (tests/host/), and run.
2. No atomic operation anywhere: the M-0002 record's threat model rules out atomic
   functions, and its limitations name atomic de-quantisation as residual
   nondeterminism.  Checked in the kernel sources (comments stripped) and in the
   disassembly of the gfx950 code objects built into libbi.so here.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_deterministic_amd", "csrc")
LIB = os.path.join(ROOT, "invariant_deterministic_amd", "libbi.so")
LLVM = "/opt/rocm/llvm/bin"


def test_api_checks_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "api_check")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *san,
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "host", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "host", "api_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "api_check ok" in r.stdout


def _strip_comments(src: str) -> str:
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return re.sub(r'"(\\.|[^"\\])*"', '""', src)


def test_no_atomics_in_sources():
    names = [f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h"))]
    assert len(names) >= 8
    hits = []
    for n in names:
        code = _strip_comments(open(os.path.join(CSRC, n)).read())
        for m in re.finditer(r"\w*atomic\w*", code, flags=re.I):
            hits.append((n, m.group(0)))
    assert not hits, hits


VECTOR_ATOMIC = re.compile(r"\b(global|buffer|flat)_atomic_\w+")
LDS_ATOMIC = re.compile(r"\bds_(add|sub|rsub|inc|dec|min|max|and|or|xor|mskor|wrxchg|cmpst|cmpswap|condxchg)\w*")


def test_no_atomic_instructions_in_code_objects(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libbi.so not built")
    if not (os.path.exists(f"{LLVM}/clang-offload-bundler") and os.path.exists(f"{LLVM}/llvm-objdump")):
        pytest.skip("ROCm LLVM tools not available")
    fat = tmp_path / "fatbin.bin"
    # objcopy rewrites the file it reads when no output is named: work on a copy, never on
    # the library a test process may have mapped
    lib_copy = tmp_path / "libbi_copy.so"
    shutil.copyfile(LIB, lib_copy)
    subprocess.run(["objcopy", f"--dump-section=.hip_fatbin={fat}", str(lib_copy)], check=True, capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    assert len(starts) >= 8  # one bundle per translation unit
    n_lines = 0
    for i, s in enumerate(starts):
        part = tmp_path / f"b{i}.bin"
        part.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"co{i}.o"
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--input={part}", f"--output={co}", "--unbundle"], check=True, capture_output=True)
        dis = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(co)], check=True, capture_output=True,
                             text=True).stdout
        n_lines += dis.count("\n")
        bad = [l.strip() for l in dis.splitlines() if VECTOR_ATOMIC.search(l) or LDS_ATOMIC.search(l)]
        assert not bad, bad[:5]
    assert n_lines > 10000
