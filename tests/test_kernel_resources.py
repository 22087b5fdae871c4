"""Build-time guard: no kernel of the library uses scratch memory.

The fused step must keep the gradient tile on chip (FORGE explainer, §2 Method, core
mechanism: the tile is consumed in registers and discarded, never written to device
memory). A register spill is private scratch memory in HBM, so every kernel in
optimizer_gemm_amd/csrc is compiled for gfx950 with the release flags and the
compiler's resource-usage remarks (the session's host-checking build, whose device code
is the release build's), and each must report ScratchSize 0 and no spilled vector
registers. The per-configuration register and LDS figures are printed (pytest -s) for
the record.
"""
import re

import pytest

KEYS = {"vgpr": r"VGPRs", "agpr": r"AGPRs", "vspill": r"VGPRs Spill", "sspill": r"SGPRs Spill",
        "scratch": r"ScratchSize \[bytes/lane\]", "lds": r"LDS Size \[bytes/block\]",
        "occupancy": r"Occupancy \[waves/SIMD\]"}


def _parse(stderr):
    kernels = {}
    for block in stderr.split("remark: Function Name: ")[1:]:
        name = block.split()[0]
        vals = {}
        for k, pat in KEYS.items():
            m = re.search(pat + r": (\d+)", block)
            vals[k] = int(m.group(1)) if m else None
        kernels[name] = vals
    return kernels


def _config_tag(name):
    """GEMM core kernels: tile configuration and epilogue from the mangled template arguments."""
    m = re.search(r"GCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)ELi(\d)ELi(\d)ELi(\d)ELi(\d)", name)
    if not m:
        return None
    bm, bn, bk, wm, wn, btr, occ, nst, ks, inp = m.groups()
    e = re.search(r"EEELi(\d)ELi(\d)ELi(\d)ELb(\d)E", name)
    epi = {"0": "dW store", "1": "fused step", "2": "dgrad"}[e.group(1)] if e else "?"
    return f"{bm}x{bn} BK{bk} {int(wm) * int(wn) * int(ks)} waves occ{occ} k-split{ks} {'fp8' if inp == '1' else 'bf16'}: {epi}"


@pytest.fixture(scope="module")
def resources(host_checked_build):
    _, _, stderr = host_checked_build
    out = {}
    for text in stderr.values():
        out.update(_parse(text))
    return out


def test_no_kernel_uses_scratch(resources):
    fused = [n for n in resources if "gemm_kernel" in n and re.search(r"EEELi1E", n)]
    assert len(fused) >= 400, f"expected every fused-step instantiation, found {len(fused)}"
    bad = {n: v for n, v in resources.items() if v["scratch"] != 0 or v["vspill"] != 0}
    assert not bad, "kernels with scratch or spilled VGPRs:\n" + "\n".join(
        f"  {_config_tag(n) or n}: {v}" for n, v in sorted(bad.items())[:20])


def test_resource_table(resources):
    """Per tile configuration and epilogue: the largest register and LDS figures over its
    instantiations (optimizers, moment formats, rounding)."""
    table = {}
    for n, v in resources.items():
        tag = _config_tag(n)
        if tag is None:
            continue
        t = table.setdefault(tag, {"n": 0, "vgpr": 0, "agpr": 0, "lds": 0, "occupancy": 99})
        t["n"] += 1
        t["vgpr"] = max(t["vgpr"], v["vgpr"] or 0)
        t["agpr"] = max(t["agpr"], v["agpr"] or 0)
        t["lds"] = max(t["lds"], v["lds"] or 0)
        t["occupancy"] = min(t["occupancy"], v["occupancy"] or 0)
    assert table
    for tag, t in sorted(table.items()):
        print(f"[resources] {tag}: {t['n']} kernels, VGPR <= {t['vgpr']}, AGPR <= {t['agpr']}, "
              f"LDS <= {t['lds']} B, occupancy >= {t['occupancy']} waves/SIMD")
