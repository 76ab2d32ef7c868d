"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer builds (no GPU needed): the CPU
oracle run on small shapes of every dtype, and the C-ABI argument validation, which must
reject or accept every call before any HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "oracle/moe_oracle.c", os.path.join(SAN, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.stdout.count(": ok") == 6, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None
                    or not os.path.exists(HIPCC), reason="needs gcc, g++ and hipcc")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    from mixture_experts_layer_softmax_amd import build

    build.build()  # the objects of the kernels that validation never launches
    objs = []
    for src in ("api.hip", "probe.hip"):  # the host code that runs: instrumented
        obj = str(tmp_path / (src + ".san.o"))
        _run([HIPCC] + build.FLAGS + ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                                      "-Xarch_host", "-fsanitize=undefined",
                                      "-c", os.path.join(build.CSRC, src), "-o", obj])
        objs.append(obj)
    for src in build.sources():
        if os.path.basename(src) not in ("api.hip", "probe.hip"):
            objs.append(os.path.join(build.BUILD, os.path.basename(src) + ".o"))
    drv = str(tmp_path / "abi_driver.o")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-I", "include", "-c",
          os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run(["g++", "-fsanitize=address,undefined", drv] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi validation: ok" in r.stdout, r.stdout
