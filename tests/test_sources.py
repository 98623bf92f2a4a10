"""Static checks on the HIP sources (CPU only).

clang lowers ``__builtin_bit_cast(T, v.y)`` on an ext_vector_type element by
reading from the vector's base address, i.e. it returns the bits of ``v.x``.
Kernels therefore only pass plain scalars or whole vectors to it (helpers such
as ``unpack_f16x2`` take the element by value). This test keeps that rule.
"""
import glob
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gated_delta_rule_87_amd", "csrc")

# __builtin_bit_cast(type, <expr ending in .x/.y/.z/.w or [i] of a vector>)
_ELEMENT_ARG = re.compile(r"__builtin_bit_cast\s*\([^,()]+,\s*[A-Za-z_][\w\[\]\.]*\.(?:[xyzw]|s[0-9a-f])\s*\)")


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))


def test_sources_exist():
    names = {os.path.basename(p) for p in _sources()}
    assert {"kda_device.h", "kda_intra.hip", "kda_chain.hip", "kda_sched.hip", "kda_recurrent.hip"} <= names


def test_no_bit_cast_of_vector_element():
    bad = []
    for path in _sources():
        for n, line in enumerate(open(path), 1):
            if _ELEMENT_ARG.search(line):
                bad.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not bad, "bit_cast of a vector element (miscompiled by clang):\n" + "\n".join(bad)


def test_pattern_catches_the_bad_form():
    assert _ELEMENT_ARG.search("f32x2 a = conv(__builtin_bit_cast(f16x2, uh.y), f32x2);")
    assert _ELEMENT_ARG.search("__builtin_bit_cast(f16x2, R.ut[w][t].x)")
    assert not _ELEMENT_ARG.search("__builtin_bit_cast(f16x2, u)")
    assert not _ELEMENT_ARG.search("__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2))")


def _device_asm(source, tmp_path):
    import subprocess
    from gated_delta_rule_87_amd.build import FLAGS, HIPCC
    if not os.access(HIPCC, os.X_OK):
        import pytest
        pytest.skip("hipcc not available")
    out = tmp_path / "k.s"
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, source)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def test_chain_lds_dma_has_uniform_destination(tmp_path):
    """Every LDS DMA load of the chain kernel takes M0 (its LDS destination, one per
    wave) from scalar arithmetic, never from a per-lane value via v_readfirstlane, and
    no load sits in a waterfall loop. A lane-dependent branch around such a load once
    let the optimiser merge call sites and route lanes to the wrong LDS address."""
    lines = [ln.strip() for ln in _device_asm("kda_chain.hip", tmp_path)]
    loads = [i for i, ln in enumerate(lines) if ln.startswith("buffer_load_dwordx4") and ln.endswith("lds")]
    assert len(loads) >= 2 * 56
    rfl = {}
    for i, ln in enumerate(lines):
        m = re.match(r"v_readfirstlane_b32 (s\d+),", ln)
        if m:
            rfl[m.group(1)] = i
        m = re.match(r"s_mov_b32 m0, (s\d+)$", ln)
        if m and m.group(1) in rfl and i - rfl[m.group(1)] < 8:
            raise AssertionError(f"M0 set from v_readfirstlane at asm line {i}: {ln}")
    for i, ln in enumerate(lines):
        if ln.startswith("s_xor_b64 exec, exec"):
            raise AssertionError(f"waterfall loop (s_xor_b64 exec) at asm line {i}")


def test_no_kernel_uses_scratch(tmp_path):
    """Every kernel keeps its working set in registers and LDS: no VGPR spills and no
    private (scratch) segment. A cross-lane read evaluated under a lane condition (for
    example a DPP broadcast inside one arm of ?:) once turned into divergent branches
    and about a thousand spilled registers."""
    bad = []
    for src in ("kda_intra.hip", "kda_chain.hip", "kda_sched.hip", "kda_recurrent.hip"):
        text = "\n".join(_device_asm(src, tmp_path))
        names = re.findall(r"\.name:\s+(\S+)", text)
        spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
        priv = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
        assert spills and len(spills) == len(priv)
        for i, (sp, pr) in enumerate(zip(spills, priv)):
            if sp or pr:
                bad.append(f"{src}: kernel {i} ({names[i] if i < len(names) else '?'}): {sp} spills, {pr} B scratch")
    assert not bad, "\n".join(bad)
