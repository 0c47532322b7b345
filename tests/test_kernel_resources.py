"""Resource use of the attention kernels as the compiler reports it (CPU: hipcc cross-compiles
gfx950). The bf16 kernels are tuned for two workgroups per compute unit with no register
spills in the tile loop: a spill there halves the rate, and more LDS or registers halve the
occupancy. This test pins those properties so that a change that breaks them fails here rather
than only on the device."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "temporally_sparse_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _remarks(tmp_path):
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "lite_attn_kernels.hip"), "-o", str(tmp_path / "k.o"),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:(.*)\[-Rpass", line)
        if cur and m:
            text = re.sub(r"^.*?:\d+:\d+:", "", m.group(1))   # a leading source location, if any
            m2 = re.match(r"\s*([A-Za-z ]+?)(?: \[[^\]]+\])?: (\d+)\s*$", text)
            if m2:
                kernels[cur][m2.group(1).strip()] = int(m2.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_bf16_kernels_fit_two_workgroups_per_cu_without_spills(tmp_path):
    k = _remarks(tmp_path)
    bf16 = {n: v for n, v in k.items() if "lite_attn_fwd_bf16" in n}
    assert len(bf16) == 8, sorted(k)            # D 64/128 x tile_q 64/128 x in-step skip
    for name, v in bf16.items():
        # At most a couple of values spilled once per tile, outside the tile loop (the queue
        # driver holds its loop state across the tile); the tile loop itself is checked for
        # scratch traffic below.
        assert 0 <= v.get("VGPRs Spill", -1) <= 2, (name, v)
        assert v.get("Occupancy", 0) >= 1, (name, v)
        assert v.get("LDS Size", 1 << 30) <= 80 * 1024, (name, v)   # two per 160 KiB CU
        if "ILi4E" in name:                      # tile_q 128: four waves, two workgroups per CU
            assert v.get("Occupancy", 0) >= 2, (name, v)


@pytest.fixture(scope="module")
def tile_loops(tmp_path_factory):
    """The tile loop of every out-of-line tile driver, as assembly lines: the stretch between two
    workgroup barriers that holds the most MFMAs. The tile runs inside two drivers (one tile;
    tiles from the queue) per head dim, tile_q and variant, whose code the kernels' remarks do
    not describe, so their assembly is read."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "lite_attn_kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    asm = out.read_text()
    loops = {}
    for m in re.finditer(r"^(_ZN\w*bf16_tiles?I\w*):", asm, re.M):
        body = asm[m.start():asm.index(".Lfunc_end", m.start())].split("\n")
        bars = [i for i, l in enumerate(body) if "s_barrier" in l]
        assert len(bars) >= 2, m.group(1)
        spans = [(sum("v_mfma" in l for l in body[a:b]), a, b) for a, b in zip(bars, bars[1:])]
        mfmas, a, b = max(spans)
        if mfmas:                 # a driver that calls the one-tile driver holds no tile loop
            loops[m.group(1)] = body[a:b]
    # 2 drivers x 2 head dims x 2 tile_q x plain / in-step, less the queue drivers at D = 128 and
    # tile_q 64, which call the one-tile driver per tile
    assert len(loops) == 14, sorted(loops)
    return loops


def test_tile_loop_has_no_scratch_traffic(tile_loops):
    """For tile_q 128 the tile loop must not touch scratch memory (the saves of callee-saved
    registers at a driver's entry and exit lie outside it). tile_q 64 runs one wave per SIMD at
    256 VGPRs and may spill a few values."""
    for name, loop in tile_loops.items():
        scratch = sum("scratch_" in l for l in loop)
        limit = 0 if "ILi4E" in name else 12
        assert scratch <= limit, (name, scratch)


def test_tile_loop_interleaves_mfma_with_vector_work(tile_loops):
    """The software pipeline of the plain step: while the S^T MFMAs of one tile run (phase A),
    the wave computes the exponentials of the previous tile, and while the PV MFMAs run (phase
    B), the scaling and row maxima of the next. Scheduling groups pin that interleave; when the
    compiler drops them (as it did once after an unrelated change to the tile's inputs), the
    MFMAs of a phase issue back to back and the vector work trails them, which costs far more
    than any parity test notices. At most two MFMAs of each phase may lack vector instructions
    before the next MFMA (the first and last PV MFMAs at D = 64 do)."""
    checked = 0
    for name, loop in tile_loops.items():
        if "Lb0E" not in name:      # the in-step variant masks the ragged tile between phases
            continue
        d = int(re.search(r"ILi(\d+)E", name).group(1))
        seq = []
        for line in loop:
            t = line.split()
            if not t or t[0].startswith((";", ".")):
                continue
            if "v_mfma" in t[0]:
                seq.append("M")
            elif t[0].startswith("v_"):
                seq.append("v")
        marks = [i for i, c in enumerate(seq) if c == "M"]
        per_phase = d // 8
        assert len(marks) >= 2 * per_phase, (name, len(marks))
        for phase in range(2):
            idx = marks[phase * per_phase:(phase + 1) * per_phase]
            bare = sum("v" not in seq[a + 1:b] for a, b in zip(idx, idx[1:]))
            assert bare <= 2, (name, "phase A" if phase == 0 else "phase B", bare,
                               "".join(seq[idx[0]:idx[-1] + 1]))
        checked += 1
    assert checked == 7
