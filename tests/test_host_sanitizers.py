"""The library's host code (argument checks, layouts, the packer, the dispatch
rules) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven
by tests/sanitize_driver.c, on the CPU.

Only the host side of each source is compiled again, with the sanitizers
(every sanitizer flag applies to the host compilation alone); each host
object refers to its device code by one symbol, which is bound to the device
code of the regular build (the .hip_fatbin section of its object, copied out
and wrapped under that symbol), so no device code is compiled twice.  No GPU
is touched.  The driver hands the library buffers of exactly the documented
sizes, so any read or write past them, any misaligned access, signed overflow
or invalid shift on these paths stops the run with a report."""
import os
import runpy
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.conftest import ROOT

HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# host-only sanitizer flags, each behind -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({res.returncode}):\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
@pytest.mark.timeout(600)
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    pkg = os.path.join(ROOT, "compressed_output_head_amd")
    build = runpy.run_path(os.path.join(pkg, "build.py"))
    regular = [os.path.join(pkg, "_build", os.path.splitext(s)[0] + ".o") for s in build["SOURCES"]]
    if not all(os.path.exists(o) for o in regular):
        build["build"]()
    flags = [f for f in build["FLAGS"] if f not in ("-shared", "-O3")] + ["-O1", "-g", "--cuda-host-only"]
    csrc = os.path.join(pkg, "csrc")
    names = [os.path.splitext(s)[0] for s in build["SOURCES"]]
    objs = [str(tmp_path / (n + ".o")) for n in names]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, *SAN, "-c", os.path.join(csrc, so[0]), "-o", so[1]]),
                    zip(build["SOURCES"], objs)))
    # each host object's device code: the regular object's .hip_fatbin under the symbol it expects
    fb_objs = []
    for n, obj, reg in zip(names, objs, regular):
        sym = [ln.split()[-1] for ln in _run(["nm", obj]).stdout.splitlines()
               if ln.split()[-1].startswith("__hip_fatbin_") and ln.split()[0] == "U"]
        if not sym:
            continue
        fb = str(tmp_path / (n + ".fatbin"))
        _run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", reg, fb])
        asm = tmp_path / (n + "_fatbin.s")
        asm.write_text(f'\t.section .hip_fatbin,"a",@progbits\n\t.p2align 12\n\t.globl {sym[0]}\n'
                       f'{sym[0]}:\n\t.incbin "{fb}"\n')
        fb_objs.append(str(tmp_path / (n + "_fatbin.o")))
        _run([CLANG, "-c", str(asm), "-o", fb_objs[-1]])
    lib = str(tmp_path / "libarchead_san.so")
    _run([HIPCC, "-shared", "-fPIC", *SAN, *objs, *fb_objs, *build["LINK_LIBS"], "-o", lib])
    exe = str(tmp_path / "sanitize_driver")
    _run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize_driver.c"),
          "-L", str(tmp_path), "-larchead_san", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert "0 failures" in res.stdout
