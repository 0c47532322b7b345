"""The C-ABI library: it loads without a GPU, exports what include/lite_attn.h declares, and
its host-side validation returns the documented status codes (no device call is made)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import temporally_sparse_attention_amd as tsa
from temporally_sparse_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lite_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lite_attn_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                        text=True).stdout
    exported = set(re.findall(r" T (lite_attn_\w+)", nm))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c_and_cpp(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "lite_attn.h"\nint main(void){ lite_attn_config c = {0};'
                   ' (void)c; return (int)sizeof(lite_attn_t) == 0; }\n')
    for compiler, flags in (("gcc", ["-std=c99"]), ("g++", ["-x", "c++", "-std=c++17"])):
        r = subprocess.run([compiler, *flags, "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                            "-c", str(src), "-o", str(tmp_path / "use.o")], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr


def test_config_struct_layout_matches_c(tmp_path):
    src = tmp_path / "off.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lite_attn.h"\n'
                   'int main(void){ printf("%zu %zu %zu %zu\\n", sizeof(lite_attn_config),'
                   ' offsetof(lite_attn_config, softmax_scale), offsetof(lite_attn_config, dense_prefix),'
                   ' offsetof(lite_attn_config, stride_b)); printf("%zu %zu %d\\n",'
                   ' offsetof(lite_attn_config, options), offsetof(lite_attn_config, reserved),'
                   ' (int)LITE_ATTN_OPT_IN_STEP_SKIP); return 0; }\n')
    exe = tmp_path / "off"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()
    c = binding.LiteAttnConfig
    assert [int(x) for x in got] == [ctypes.sizeof(c), c.softmax_scale.offset,
                                     c.dense_prefix.offset, c.stride_b.offset, c.options.offset,
                                     c.reserved.offset, binding.OPT_IN_STEP_SKIP]


def _status(fn):
    try:
        fn()
    except tsa.LiteAttnError as e:
        return e.status
    return binding.OK


def test_create_validation():
    ok = lambda **kw: (lambda: tsa.lite_attn_create(1, 2, 1000, 128, **kw))
    assert _status(ok()) == binding.OK
    assert _status(ok(dtype="fp32", tile_q=64)) == binding.OK
    assert _status(lambda: tsa.lite_attn_create(1, 2, 1000, 96)) == binding.ERR_UNSUPPORTED
    assert _status(ok(tile_k=128)) == binding.ERR_UNSUPPORTED
    assert _status(ok(tile_q=32)) == binding.ERR_UNSUPPORTED
    assert _status(lambda: tsa.lite_attn_create(-1, 2, 1000, 128)) == binding.ERR_INVALID_ARG
    assert _status(ok(dense_prefix=1001)) == binding.ERR_INVALID_ARG
    assert _status(ok(dense_prefix=-1)) == binding.ERR_INVALID_ARG
    assert _status(ok(strides=(0, 0, 100))) == binding.ERR_INVALID_ARG     # not a multiple of 8
    assert _status(ok(strides=(0, 0, 64))) == binding.ERR_INVALID_ARG      # < head_dim
    assert _status(lambda: tsa.lite_attn_create(1, 1, 140000, 64, tile_q=128)) == binding.ERR_UNSUPPORTED
    assert _status(ok(in_step_skip=True)) == binding.OK
    assert _status(ok(in_step_skip=True, dtype="fp32", tile_q=64)) == binding.OK
    for field, value in (("options", 2), ("options", 0x80000001), ("reserved", 1)):
        bad = tsa.make_config(1, 2, 1000, 128)
        setattr(bad, field, value)
        assert _status(lambda: tsa.lite_attn_create(0, 0, 0, 0, config=bad)) == binding.ERR_INVALID_ARG
    cfg = tsa.make_config(1, 2, 1000, 128)
    cfg.abi_version = 99
    assert _status(lambda: tsa.lite_attn_create(0, 0, 0, 0, config=cfg)) == binding.ERR_INVALID_ARG
    lib = binding.library()
    assert lib.lite_attn_create(None, None) == binding.ERR_INVALID_ARG
    assert "NULL" in tsa.lite_attn_last_error()


def test_geometry_and_mask_bytes():
    h = tsa.lite_attn_create(2, 3, 75600, 128, tile_q=128)
    assert tsa.lite_attn_mask_geometry(h) == (591, 1182, 37)
    assert tsa.lite_attn_mask_bytes(h) == 2 * 3 * 591 * 37 * 4
    e = tsa.lite_attn_create(0, 3, 100, 64)
    assert tsa.lite_attn_mask_bytes(e) == 0
    assert binding.library().lite_attn_mask_bytes(None) == 0


def test_step_host_validation_makes_no_device_call():
    h = tsa.lite_attn_create(1, 1, 100, 64, tile_q=64)
    lib = binding.library()
    p = ctypes.c_void_p(4096)
    ms = ctypes.c_void_p(4096)
    st = lambda *a: lib.lite_attn_step(h.ptr, *a)
    assert st(None, p, p, ctypes.c_void_p(8192), ms, ctypes.c_float(-1.0), 0, None) == binding.ERR_INVALID_ARG
    assert st(p, p, p, ctypes.c_void_p(8192), ms, ctypes.c_float(0.5), 0, None) == binding.ERR_INVALID_ARG
    assert st(p, p, p, ctypes.c_void_p(8192), ms, ctypes.c_float(math.nan), 0, None) == binding.ERR_INVALID_ARG
    assert st(p, p, p, ctypes.c_void_p(8192), ms, ctypes.c_float(-1.0), -1, None) == binding.ERR_INVALID_ARG
    assert st(p, p, p, ctypes.c_void_p(8200), ms, ctypes.c_float(-1.0), 0, None) == binding.ERR_INVALID_ARG
    assert st(p, p, p, p, ms, ctypes.c_float(-1.0), 0, None) == binding.ERR_INVALID_ARG  # out aliases
    assert lib.lite_attn_step(None, p, p, p, p, ms, ctypes.c_float(-1.0), 0, None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_reset_mask(h.ptr, None, None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_mask_popcount(h.ptr, ms, None, None) == binding.ERR_INVALID_ARG
    sc = lambda ws, *a: lib.lite_attn_step_scheduled(h.ptr, p, p, p, ctypes.c_void_p(8192), ms,
                                                    ctypes.c_float(-1.0), 0, ws, None)
    assert sc(None) == binding.ERR_INVALID_ARG                          # no workspace
    assert sc(ctypes.c_void_p(4096 + 128)) == binding.ERR_INVALID_ARG    # not 256-byte aligned
    assert lib.lite_attn_step_scheduled(h.ptr, p, p, p, ctypes.c_void_p(8192), ms,
                                        ctypes.c_float(0.5), 0, p, None) == binding.ERR_INVALID_ARG
    rf = lambda stats, delta: lib.lite_attn_step_refresh(h.ptr, p, p, p, ctypes.c_void_p(8192), ms,
                                                         stats, ctypes.c_float(delta),
                                                         ctypes.c_float(-1.0), 0, None)
    assert rf(None, 1.0) == binding.ERR_INVALID_ARG                     # no tile_stats
    assert rf(ctypes.c_void_p(4098), 1.0) == binding.ERR_INVALID_ARG    # misaligned
    assert rf(p, -1.0) == binding.ERR_INVALID_ARG                       # negative delta
    assert rf(p, math.nan) == binding.ERR_INVALID_ARG                   # NaN delta
    n = 1 * 1 * 2   # B * H * Tq for N = 100, tile_q = 64
    assert tsa.lite_attn_workspace_bytes(h) >= 6 * n and tsa.lite_attn_workspace_bytes(h) % 256 == 0
    assert lib.lite_attn_workspace_bytes(None) == 0
    # an empty problem is a no-op that needs no pointers
    e = tsa.lite_attn_create(1, 0, 100, 64, tile_q=64)
    assert lib.lite_attn_step(e.ptr, None, None, None, None, None, ctypes.c_float(-1.0), 0, None) == binding.OK
    assert lib.lite_attn_reset_mask(e.ptr, None, None) == binding.OK


def test_status_strings():
    for code in range(5):
        assert tsa.lite_attn_status_string(code)
    assert tsa.lite_attn_status_string(77) == "unknown status"


def test_error_budget_schedule():
    s = tsa.ErrorBudgetSchedule.linear(10, -14.0, -8.0)
    assert s[0] == -14.0 and s[9] == -8.0 and len(s) == 10
    tsa.ErrorBudgetSchedule([-math.inf, -12, -10, -9])
    with pytest.raises(ValueError):
        tsa.ErrorBudgetSchedule([-8, -10])       # tightens later
    with pytest.raises(ValueError):
        tsa.ErrorBudgetSchedule([0.5])


def test_create_rejects_strides_that_overlap_out_rows():
    """out is written through the strides it shares with q, k and v: a stride set under which two
    (b, h, n) rows land on the same memory would be a silent write race."""
    B, H, N, D = 2, 3, 1000, 64
    mk = lambda strides, b=B, h=H: (lambda: tsa.lite_attn_create(b, h, N, D, tile_q=64,
                                                                  strides=strides))
    assert _status(mk((H * N * D, N * D, D))) == binding.OK                  # contiguous
    assert _status(mk((H * N * 3 * D, N * 3 * D, 3 * D))) == binding.OK      # packed QKV view
    assert _status(mk((N * H * D, D, H * D))) == binding.OK                  # [B][N][H][D]
    assert _status(mk((0, N * D, D))) == binding.ERR_INVALID_ARG             # batches share rows
    assert _status(mk((H * N * D, 0, D))) == binding.ERR_INVALID_ARG         # heads share rows
    assert _status(mk((H * N * D, N * D - 8, D))) == binding.ERR_INVALID_ARG  # heads overlap
    assert _status(mk((N * D, N * D, D))) == binding.ERR_INVALID_ARG         # b and h collide
    assert _status(mk((0, 0, D), b=1, h=1)) == binding.OK                    # one head: no overlap
    assert _status(mk((8, 0, D), b=1, h=1)) == binding.OK


def test_last_launch_before_any_step():
    import threading
    got = []
    th = threading.Thread(target=lambda: got.append(tsa.lite_attn_last_launch()))
    th.start()
    th.join()
    assert got == [(0, -1)]


def test_static_workspace_entry_point_rejects_large_problems_without_a_device_call():
    lib = binding.library()
    p = ctypes.c_void_p(4096)
    small = tsa.lite_attn_create(1, 2, 1000, 128)
    assert tsa.lite_attn_workspace_bytes(small) <= 1 << 20
    big = tsa.lite_attn_create(200, 8, 131072, 64, tile_q=128)      # 1.6M query tiles
    assert tsa.lite_attn_workspace_bytes(big) > 1 << 20
    st = lambda h, eps=-1.0: lib.lite_attn_step_scheduled_static(h.ptr, p, p, p,
                                                                 ctypes.c_void_p(8192), p,
                                                                 ctypes.c_float(eps), 0, None)
    assert st(big) == binding.ERR_UNSUPPORTED
    assert "static workspace" in tsa.lite_attn_last_error()
    assert lib.lite_attn_step_scheduled_static(None, p, p, p, p, p, ctypes.c_float(-1.0), 0,
                                               None) == binding.ERR_INVALID_ARG
    empty = tsa.lite_attn_create(1, 0, 100, 64, tile_q=64)
    assert lib.lite_attn_step_scheduled_static(empty.ptr, None, None, None, None, None,
                                               ctypes.c_float(-1.0), 0, None) == binding.OK


def test_create_rejects_heads_spanning_2_gib_in_bf16():
    """The bf16 kernels address a head's rows through a 32-bit buffer offset."""
    n, d = 131072, 128
    ok = tsa.make_config(1, 1, n, d, strides=(0, 0, 8192))       # 2 GiB - 16 KiB + 256 B
    assert _status(lambda: tsa.lite_attn_create(0, 0, 0, 0, config=ok)) == binding.OK
    big = tsa.make_config(1, 1, n, d, strides=(0, 0, 8200))
    assert _status(lambda: tsa.lite_attn_create(0, 0, 0, 0, config=big)) == binding.ERR_UNSUPPORTED
    f32 = tsa.make_config(1, 1, n, d, strides=(0, 0, 8200), dtype="fp32")
    assert _status(lambda: tsa.lite_attn_create(0, 0, 0, 0, config=f32)) == binding.OK


def test_calibration_entries_validate_on_the_host_without_a_device_call():
    lib = binding.library()
    h = tsa.lite_attn_create(1, 2, 1000, 128, tile_q=128)
    p = ctypes.c_void_p(4096)
    # workspace: four outputs (1 * 2 * 1000 * 128 bf16, contiguous), two masks, one result word
    out_bytes = (2 * 1000 * 128 * 2 + 255) // 256 * 256
    mask_bytes = (tsa.lite_attn_mask_bytes(h) + 255) // 256 * 256
    assert tsa.lite_attn_calibrate_workspace_bytes(h) == 4 * out_bytes + 2 * mask_bytes + 256
    assert lib.lite_attn_calibrate_workspace_bytes(None) == 0
    # output_max_abs_diff
    assert lib.lite_attn_output_max_abs_diff(None, p, p, p, None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_output_max_abs_diff(h.ptr, p, p, None, None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_output_max_abs_diff(h.ptr, p, p, ctypes.c_void_p(4098),
                                             None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_output_max_abs_diff(h.ptr, None, p, p, None) == binding.ERR_INVALID_ARG
    assert lib.lite_attn_output_max_abs_diff(h.ptr, ctypes.c_void_p(4104), p, p,
                                             None) == binding.ERR_INVALID_ARG
    # calibrate: every argument check comes before the first device call
    steps = 3
    ptrs = (ctypes.c_void_p * steps)(*([4096] * steps))
    fl = ctypes.c_float * steps

    def cal(budgets=(0.1, 0.1, 0.1), cands=(-4.0, -8.0), n=None, handle=h, nsteps=steps,
            q=ptrs, out=True):
        c = (ctypes.c_float * max(1, len(cands)))(*cands)
        le, er = fl(), fl()
        return lib.lite_attn_calibrate(handle.ptr if handle else None, q, ptrs, ptrs, nsteps,
                                       fl(*budgets), c, len(cands) if n is None else n,
                                       le if out else None, er, p, None)

    assert cal(handle=None) == binding.ERR_INVALID_ARG
    assert cal(nsteps=-1) == binding.ERR_INVALID_ARG
    assert cal(q=None) == binding.ERR_INVALID_ARG
    assert cal(out=False) == binding.ERR_INVALID_ARG
    assert cal(n=-1) == binding.ERR_INVALID_ARG
    assert cal(budgets=(0.1, math.nan, 0.1)) == binding.ERR_INVALID_ARG
    assert cal(cands=(-4.0, 0.5)) == binding.ERR_INVALID_ARG
    assert "candidate" in tsa.lite_attn_last_error()
    assert cal(cands=(math.nan,)) == binding.ERR_INVALID_ARG
    assert cal(nsteps=0) == binding.OK                                  # nothing to do
    # an empty problem needs no workspace and no device: every error is 0, so each step takes
    # the loosest candidate whose budget 0 meets, and the last step repeats its predecessor
    e = tsa.lite_attn_create(1, 0, 100, 64, tile_q=64)
    assert tsa.lite_attn_calibrate_workspace_bytes(e) == 256
    le, er = fl(), fl()
    c = (ctypes.c_float * 3)(-8.0, -2.0, -8.0)
    assert lib.lite_attn_calibrate(e.ptr, ptrs, ptrs, ptrs, steps, fl(1.0, -1.0, 1.0), c, 3, le,
                                   er, None, None) == binding.OK
    assert list(le) == [-math.inf, -2.0, -2.0] and list(er) == [0.0] * 3
