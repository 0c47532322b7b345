"""The C ABI used from C alone: tests/c_abi_smoke.c is compiled as C11 with gcc against
include/lite_attn.h and linked against liblite_attn.so (no Python, torch or HIP compiler in
between). On the CPU it must compile and link; on the GPU it must run a short chain and pass its
own checks (finite outputs inside the range of V, a non-decreasing skip count, bit-identical
reruns, argument errors reported, and the scheduled and refresh entry points reproducing the
plain chain bit for bit, and the calibration entries agreeing with a replay of the schedule
they choose)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "temporally_sparse_attention_amd")
SRC = os.path.join(ROOT, "tests", "c_abi_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(os.path.join(LIBDIR, "liblite_attn.so")):
        pytest.fail("liblite_attn.so is not built (run python -m temporally_sparse_attention_amd.build)")
    exe = str(tmp_path / "c_abi_smoke")
    cmd = [gcc, "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", exe,
           f"-L{LIBDIR}", "-llite_attn", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_c_program_compiles_and_links_as_c11(tmp_path):
    _build(tmp_path)


@pytest.mark.gpu
def test_c_program_runs_a_chain(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "c abi smoke ok" in r.stdout
