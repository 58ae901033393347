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
