"""Register, spill and occupancy guards on the kernels of the last build.

The build records the compiler's per-kernel resource report
(_build/kernel_resources.json).  The kernels are designed around an occupancy
and a register budget; a change that pushes one of them into scratch spills
still computes the right values, so the parity tests would not notice it, but
it runs several times slower.  These checks catch that on the CPU.
"""
import json
import os
import re

import pytest

from denoiser_attention_amd import build as B

MFMA = re.compile(r"attn_mfma_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")


def _resources():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("no build here yet (run the build first)")
    newest_src = max(os.path.getmtime(os.path.join(B.CSRC, s)) for s in B.SOURCES + B.PROBE_SOURCES)
    if os.path.getmtime(B.RESOURCES) < newest_src:
        pytest.fail("a kernel source changed after the last build: rebuild before testing")
    with open(B.RESOURCES) as f:
        return json.load(f)


def _kernels(res, src):
    assert src in res, f"no resource report for {src}"
    assert res[src], f"empty resource report for {src}"
    return res[src]


def test_every_source_reported():
    res = _resources()
    for src in B.SOURCES + B.PROBE_SOURCES:
        if src.endswith(".hip"):
            _kernels(res, src)


def test_attention_mfma_budget():
    """32-row waves: no spill, two waves per SIMD (the pipeline pairs a wave's
    softmax with the other wave's MFMAs).  64-row waves (opt-in): one wave per
    SIMD and at most a few spilled registers."""
    ks = _kernels(_resources(), "attn_mfma.hip")
    seen = {1: 0, 2: 0}
    for name, r in ks.items():
        m = MFMA.search(name)
        assert m, name
        D, NS, KG, RB, RG = map(int, m.groups())
        seen[RB] += 1
        if RB == 1:
            assert r["vgpr_spill"] == 0 and r["scratch_bytes"] == 0, (name, r)
            assert r["waves_per_simd"] >= 2, (name, r)
            assert r["vgprs"] + r["agprs"] <= 256, (name, r)
        else:
            assert D == 128 and KG == 1, name
            assert r["vgpr_spill"] <= 4 and r["scratch_bytes"] <= 16, (name, r)
    assert seen[1] > 0 and seen[2] > 0


def test_no_spills_elsewhere():
    res = _resources()
    for src in ("attn_shuffle.hip", "unmask.hip", "lmhead.hip", "probes.hip"):
        for name, r in _kernels(res, src).items():
            assert r["vgpr_spill"] == 0 and r["scratch_bytes"] == 0, (src, name, r)


def test_streaming_kernels_occupancy():
    """The vocabulary pass hides HBM latency with many waves in flight."""
    ks = _kernels(_resources(), "unmask.hip")
    vr = {n: r for n, r in ks.items() if "vocab_reduce_kernel" in n}
    assert vr
    for name, r in vr.items():
        assert r["waves_per_simd"] >= 7, (name, r)


def test_lmhead_stats_budget():
    ks = _kernels(_resources(), "lmhead.hip")
    st = [r for n, r in ks.items() if "lmhead_stats_kernel" in n]
    assert len(st) == 1
    assert st[0]["waves_per_simd"] >= 2 and st[0]["lds_bytes"] <= 160 * 1024, st[0]


def test_parse_resources_on_sample():
    text = (
        "x.hip:1:1: remark: Function Name: kern [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs: 74 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n"
        "x.hip:1:1: remark:     LDS Size [bytes/block]: 12424 [-Rpass-analysis=kernel-resource-usage]\n"
    )
    assert B.parse_resources(text) == {
        "kern": {"vgprs": 74, "scratch_bytes": 8, "vgpr_spill": 3, "lds_bytes": 12424}}


# --- Hazards the compiler cannot see through inline asm ---------------------
#
# The direct-to-LDS loads are written as inline asm.  On gfx950 a vector
# instruction that writes a scalar register (v_readlane of a spilled scalar,
# v_readfirstlane, a compare into an SGPR pair) needs 5 wait states before a
# memory instruction reads that register; the compiler inserts them for the
# instructions it generates, not for the operands of an asm statement.  A load
# that reads its scalar base too early takes a stale address.  Every such load
# in the built assembly must be at least 5 wait states (s_nop N counts N + 1)
# after any vector write of its scalar operands, in program order.

def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dma_hazards(asm_text):
    ins = []
    for raw in asm_text.splitlines():
        t = raw.strip()
        if not t or t.startswith((";", ".")) or re.match(r"^[\w.$]+:", t):
            continue
        ins.append(t)
    found = []
    for k, t in enumerate(ins):
        if not t.startswith("global_load_lds"):
            continue
        regs = set()
        for tok in t.replace(",", " ").split()[1:]:
            regs |= _sgprs(tok)
        ws, b = 0, k - 1
        while b >= 0 and ws < 5:
            prev = ins[b]
            if prev.startswith("v_"):
                ops = prev.replace(",", " ").split()
                if len(ops) > 1 and _sgprs(ops[1]) & regs:
                    found.append((prev, ws, t))
                    break
            m = re.match(r"s_nop\s+(\d+)", prev)
            ws += int(m.group(1)) + 1 if m else 1
            b -= 1
    return found


def test_dma_hazard_check_catches_a_planted_case():
    bad = "v_readlane_b32 s17, v246, 42\n\ts_mov_b32 m0, s5\n\tglobal_load_lds_dwordx4 v2, s[16:17]\n"
    good = "v_readlane_b32 s17, v246, 42\n\ts_nop 4\n\tglobal_load_lds_dwordx4 v2, s[16:17]\n"
    other = "v_readlane_b32 s20, v246, 42\n\tglobal_load_lds_dwordx4 v2, s[16:17]\n"
    assert len(dma_hazards(bad)) == 1
    assert dma_hazards(good) == [] and dma_hazards(other) == []


def test_no_scalar_base_hazard_before_lds_dma():
    _resources()   # the freshness check of the last build
    for src in B.SOURCES + B.PROBE_SOURCES:
        if not src.endswith(".hip"):
            continue
        path = B.device_asm(src)
        assert os.path.exists(path), f"no device assembly for {src}: rebuild"
        found = dma_hazards(open(path).read())
        assert not found, f"{src}: {found[:3]}"
