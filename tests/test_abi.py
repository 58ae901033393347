"""The C ABI on the host: the library loads, exports every entry point the
header declares, and rejects invalid arguments before touching HIP.  None of
these tests launches a kernel."""
import ctypes
import os
import re

import pytest
import torch

import denoiser_attention_amd as tt
from denoiser_attention_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tt.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libtt.so not built (python -m denoiser_attention_amd.build)")

FAKE = 0x1000   # never dereferenced: every call below fails validation first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert "tt_block_attn" in names and "tt_unmask_step" in names
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    exported = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    ours = sorted(set(re.findall(r"\bT (tt_\w+)", exported)))
    assert ours == names, "library exports must equal the header's declarations"


def test_status_strings_and_version():
    assert tt.status_string(0) == "TT_OK"
    assert "EINVAL" in tt.status_string(1)
    assert "unknown" in tt.status_string(99)
    assert tt.version() == "0.1.0"


def attn_call(**kw):
    a = dict(q=FAKE, k_ctx=FAKE, v_ctx=FAKE, prefix_len=64, k_blk=FAKE, v_blk=FAKE, block_len=16,
             hq=4, hkv=1, d=64, scale=0.125, out=FAKE, batch=1, pcap=64, dtype=B.TT_FP32,
             odt=B.TT_FP32, ws=None, wsb=0, stream=None, opts=None)
    a.update(kw)
    opts = None if a["opts"] is None else ctypes.byref(B.AttnOpts(*a["opts"]))
    return tt.lib().tt_block_attn_ex(a["q"], a["k_ctx"], a["v_ctx"], a["prefix_len"], a["k_blk"],
                                     a["v_blk"], a["block_len"], a["hq"], a["hkv"], a["d"],
                                     a["scale"], a["out"], a["batch"], a["pcap"], a["dtype"],
                                     a["odt"], a["ws"], a["wsb"], a["stream"], opts)


@pytest.mark.parametrize("kw", [
    dict(q=None), dict(k_blk=None), dict(v_blk=None), dict(out=None),
    dict(k_ctx=None), dict(v_ctx=None),
    dict(batch=-1), dict(block_len=-1), dict(prefix_len=-1), dict(hq=0), dict(hkv=0),
    dict(hq=6, hkv=4), dict(pcap=10), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(scale=3e38), dict(scale=-3e38),
    dict(dtype=7), dict(odt=7), dict(dtype=B.TT_FP32, odt=B.TT_BF16),
    dict(opts=(9, 0, 0)), dict(opts=(0, -1, 0)), dict(opts=(0, 0, 3)), dict(opts=(0, 0, -1)),
    dict(opts=(0, 0, 0, 48)), dict(opts=(0, 0, 0, -32)),
    dict(opts=(0, 0, 0, 0, 6)), dict(opts=(0, 0, 0, 0, -8)),
    # bf16 with a split that needs a workspace, none given
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, hq=32, hkv=2, d=128, prefix_len=2048, pcap=2048,
         block_len=32, batch=8, opts=(B.TT_ATTN_MFMA, 4, 0)),
])
def test_attn_rejects_invalid(kw):
    assert attn_call(**kw) == B.TT_EINVAL


@pytest.mark.parametrize("kw", [
    dict(d=96), dict(d=32), dict(opts=(B.TT_ATTN_MFMA, 0, 0)),         # fp32 on MFMA
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=256, opts=(B.TT_ATTN_MFMA, 0, 0)),
    # 64-row waves: head_dim 128 and one wave group only
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=64, opts=(B.TT_ATTN_MFMA, 0, 0, 64)),
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=128, opts=(B.TT_ATTN_MFMA, 0, 2, 64)),
    # eight waves on one K/V stream: head_dim 128, one wave group, 32-row waves only
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=64, opts=(B.TT_ATTN_MFMA, 0, 0, 0, 8)),
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=128, opts=(B.TT_ATTN_MFMA, 0, 2, 0, 8)),
    dict(dtype=B.TT_BF16, odt=B.TT_BF16, d=128, opts=(B.TT_ATTN_MFMA, 0, 0, 64, 8)),
])
def test_attn_unsupported(kw):
    assert attn_call(**kw) == B.TT_EUNSUPPORTED


def test_attn_empty_is_noop():
    assert attn_call(batch=0, q=None, out=None) == B.TT_OK
    assert attn_call(block_len=0, q=None, out=None) == B.TT_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
def test_attn_valid_call_without_device_reports_enodev():
    assert attn_call(ws=FAKE, wsb=1 << 24) == B.TT_ENODEV
    assert tt.lib().tt_unmask_step(FAKE, FAKE, 4, FAKE, FAKE, 1, 16, 1000, None, None, FAKE,
                                   1 << 20, None) == B.TT_ENODEV


def test_attn_workspace_query():
    # MFMA plan for the decode geometry splits the prefix and needs a workspace.
    n = tt.attn_workspace_bytes(8, 2048, 32, 32, 2, 128, torch.bfloat16)
    assert n > 0 and n % 256 == 0
    assert tt.attn_workspace_bytes(16, 1024, 256, 32, 2, 128, torch.bfloat16) == 0
    assert tt.attn_workspace_bytes(8, 2048, 32, 32, 2, 128, torch.bfloat16, kv_splits=1) == 0
    with pytest.raises(ValueError):
        tt.attn_workspace_bytes(1, 10, 4, 6, 4, 64, torch.float32)


def _attn_splits(batch, prefix_len, block_len, n_q_heads=32, n_kv_heads=2, head_dim=128):
    """Key splits of the launch plan, read back from the workspace size
    (splits x rows x (D + 1) fp32 partials, each part rounded up to 256 B)."""
    ws = tt.attn_workspace_bytes(batch, prefix_len, block_len, n_q_heads, n_kv_heads, head_dim,
                                 torch.bfloat16)
    if ws == 0:
        return 1
    rows = batch * n_q_heads * block_len
    up = lambda x: (x + 255) // 256 * 256
    for s in range(2, 4096):
        if up(s * rows * head_dim * 4) + up(s * rows * 4) == ws:
            return s
    raise AssertionError(f"workspace size {ws} matches no split count")


@pytest.mark.parametrize("shape,splits", [
    # B, P, L at 32 q / 2 kv heads, D = 128.  Long blocks with at least one
    # wave of query tiles per CU: no splits.
    ((16, 1024, 256), 1), ((4, 16128, 256), 1), ((64, 4096, 64), 1),
    # Decode geometry: one 4-wave group per workgroup and about one workgroup
    # per CU of key splits (65 tiles of 32 keys: 4 splits of 17 tiles at L32,
    # 8 at L16; at L1 the 16 requested splits of 5 tiles leave 13 non-empty).
    ((8, 2048, 32), 4), ((8, 2048, 16), 8), ((8, 2048, 1), 13),
    # Single-token blocks: query tiles filling 3/4 to all of the CUs once take
    # two key groups and no split; 128 tiles take two key splits.
    ((96, 2048, 1), 1), ((128, 2048, 1), 1), ((64, 4096, 1), 2),
])
def test_attn_launch_plan_splits(shape, splits):
    # Guards the tuned launch plans against an unintended change of the rules.
    assert _attn_splits(*shape) == splits


def unmask_call(**kw):
    a = dict(logits=FAKE, mask=FAKE, k=4, tokens=FAKE, mask_out=FAKE, batch=1, L=16, V=1000,
             conf=None, pred=None, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return tt.lib().tt_unmask_step(a["logits"], a["mask"], a["k"], a["tokens"], a["mask_out"],
                                   a["batch"], a["L"], a["V"], a["conf"], a["pred"], a["ws"],
                                   a["wsb"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(logits=None), dict(mask=None), dict(tokens=None), dict(mask_out=None), dict(k=-1),
    dict(batch=-1), dict(L=-1), dict(V=0), dict(ws=None), dict(wsb=16),
])
def test_unmask_rejects_invalid(kw):
    assert unmask_call(**kw) == B.TT_EINVAL


def test_unmask_limits_and_empty():
    assert unmask_call(L=1025) == B.TT_EUNSUPPORTED
    assert unmask_call(batch=0, logits=None, ws=None, wsb=0) == B.TT_OK
    assert tt.unmask_workspace_bytes(8, 32, 131072) == 8 * 32 * 16 * 16
    assert tt.unmask_workspace_bytes(1, 16, 1000) == 256
    with pytest.raises(ValueError):
        tt.unmask_workspace_bytes(1, 16, 0)


def test_unmask_halves_validate():
    lib = tt.lib()
    assert lib.tt_unmask_reduce(None, FAKE, 1, 16, 1000, FAKE, 1 << 20, None) == B.TT_EINVAL
    assert lib.tt_unmask_commit(FAKE, -2, FAKE, FAKE, 1, 16, 1000, None, None, FAKE, 1 << 20,
                                None) == B.TT_EINVAL
    assert lib.tt_unmask_commit(FAKE, 2, None, FAKE, 1, 16, 1000, None, None, FAKE, 1 << 20,
                                None) == B.TT_EINVAL


def varlen_call(**kw):
    a = dict(q=FAKE, k_ctx=FAKE, v_ctx=FAKE, lens=FAKE, pmax=64, k_blk=FAKE, v_blk=FAKE, L=16,
             hq=4, hkv=1, d=64, scale=0.125, out=FAKE, batch=1, pcap=64, dtype=B.TT_FP32,
             odt=B.TT_FP32, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return tt.lib().tt_block_attn_varlen(a["q"], a["k_ctx"], a["v_ctx"], a["lens"], a["pmax"],
                                         a["k_blk"], a["v_blk"], a["L"], a["hq"], a["hkv"], a["d"],
                                         a["scale"], a["out"], a["batch"], a["pcap"], a["dtype"],
                                         a["odt"], a["ws"], a["wsb"], None, None)


@pytest.mark.parametrize("kw", [dict(lens=None), dict(pmax=-1), dict(pmax=65), dict(q=None),
                                dict(hq=3, hkv=2), dict(scale=float("nan"))])
def test_varlen_rejects_invalid(kw):
    assert varlen_call(**kw) == B.TT_EINVAL


def test_varlen_empty_batch_and_workspace_query():
    assert varlen_call(batch=0, lens=None) == B.TT_OK
    assert tt.attn_workspace_bytes(8, 2048, 32, 32, 2, 128, torch.bfloat16) >= 0


def multiblock_call(**kw):
    a = dict(q=FAKE, k_ctx=FAKE, v_ctx=FAKE, kn=FAKE, vn=FAKE, S=16, N=4, hq=4, hkv=1, d=64,
             scale=0.125, out=FAKE, batch=1, cap=48, dtype=B.TT_FP32, odt=B.TT_FP32, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return tt.lib().tt_block_attn_multiblock(a["q"], a["k_ctx"], a["v_ctx"], a["kn"], a["vn"],
                                             a["S"], a["N"], a["hq"], a["hkv"], a["d"], a["scale"],
                                             a["out"], a["batch"], a["cap"], a["dtype"], a["odt"],
                                             a["ws"], a["wsb"], None, None)


@pytest.mark.parametrize("kw", [dict(cap=47), dict(kn=None), dict(vn=None), dict(out=None),
                                dict(k_ctx=None), dict(N=-1), dict(S=-2), dict(hq=0),
                                dict(dtype=B.TT_FP32, odt=B.TT_BF16)])
def test_multiblock_rejects_invalid(kw):
    assert multiblock_call(**kw) == B.TT_EINVAL


def test_multiblock_empty_and_workspace_query():
    assert multiblock_call(N=0, q=None, kn=None, vn=None, out=None, cap=0) == B.TT_OK
    assert multiblock_call(batch=0) == B.TT_OK
    assert multiblock_call(S=0) == B.TT_OK
    n = tt.attn_multiblock_workspace_bytes(1, 256, 32, 32, 2, 128, torch.bfloat16)
    assert n >= 0
    with pytest.raises(ValueError):
        tt.attn_multiblock_workspace_bytes(1, -1, 4, 32, 2, 128, torch.bfloat16)


SELECT_BAD = [
    dict(mode="top_k", k=-1),
    dict(mode="leftmost", k=-3),
    dict(mode="threshold", gamma=float("nan"), steps_left=2),
    dict(mode="threshold", gamma=float("inf"), steps_left=2),
    dict(mode="threshold", gamma=0.8, steps_left=0),
    dict(mode="schedule", step=0, n_steps=4),
    dict(mode="schedule", step=5, n_steps=4),
    dict(mode="schedule", step=1, n_steps=0),
]


@pytest.mark.parametrize("kw", SELECT_BAD, ids=[str(k) for k in SELECT_BAD])
def test_select_rules_validate(kw):
    lib = tt.lib()
    sel = tt.select_rule(**kw)
    assert lib.tt_unmask_step_ex(FAKE, FAKE, ctypes.byref(sel), FAKE, FAKE, 1, 16, 1000, None,
                                 None, FAKE, 1 << 20, None) == B.TT_EINVAL
    assert lib.tt_unmask_commit_ex(FAKE, ctypes.byref(sel), FAKE, FAKE, 1, 16, 1000, None, None,
                                   FAKE, 1 << 20, None) == B.TT_EINVAL


def test_select_rule_struct_and_unknown_mode():
    lib = tt.lib()
    bad = B.Select(9, 1, 0.0, 1, 1, 1)
    assert lib.tt_unmask_step_ex(FAKE, FAKE, ctypes.byref(bad), FAKE, FAKE, 1, 16, 1000, None,
                                 None, FAKE, 1 << 20, None) == B.TT_EINVAL
    assert lib.tt_unmask_step_ex(FAKE, FAKE, None, FAKE, FAKE, 1, 16, 1000, None, None, FAKE,
                                 1 << 20, None) == B.TT_EINVAL
    # Empty batch with a valid rule: nothing to do.
    ok = tt.select_rule("threshold", gamma=0.8, steps_left=3)
    assert lib.tt_unmask_step_ex(None, FAKE, ctypes.byref(ok), None, None, 0, 16, 1000, None, None,
                                 None, 0, None) == B.TT_OK
    assert ctypes.sizeof(B.Select) == 24
    with pytest.raises(ValueError):
        tt.select_rule("greedy")


def lmhead_call(**kw):
    a = dict(h=FAKE, w=FAKE, m=FAKE, sel=tt.select_rule("top_k", k=2), tok=FAKE, mo=FAKE, B=2,
             L=16, V=1000, d=64, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    sel = None if a["sel"] is None else ctypes.byref(a["sel"])
    return tt.lib().tt_lmhead_unmask_step(a["h"], a["w"], a["m"], sel, a["tok"], a["mo"], a["B"],
                                          a["L"], a["V"], a["d"], None, None, a["ws"], a["wsb"],
                                          None)


@pytest.mark.parametrize("kw,status", [
    (dict(h=None), B.TT_EINVAL), (dict(w=None), B.TT_EINVAL), (dict(m=None), B.TT_EINVAL),
    (dict(tok=None), B.TT_EINVAL), (dict(mo=None), B.TT_EINVAL), (dict(sel=None), B.TT_EINVAL),
    (dict(ws=None), B.TT_EINVAL), (dict(wsb=100), B.TT_EINVAL), (dict(d=0), B.TT_EINVAL),
    (dict(V=0), B.TT_EINVAL), (dict(d=48), B.TT_EUNSUPPORTED), (dict(L=1025), B.TT_EUNSUPPORTED),
    (dict(B=1 << 16, L=1024, d=4096), B.TT_EUNSUPPORTED),
    (dict(sel=tt.select_rule("threshold", gamma=0.5, steps_left=0)), B.TT_EINVAL),
])
def test_lmhead_rejects_invalid(kw, status):
    assert lmhead_call(**kw) == status


def test_lmhead_empty_and_workspace():
    assert lmhead_call(B=0, h=None, w=None, m=None, tok=None, mo=None, ws=None, wsb=0) == B.TT_OK
    n = tt.lmhead_unmask_workspace_bytes(8, 32, 131072, 2688)
    # per-slice partials + merged partials + row list + count, each 256-byte aligned
    assert n == 256 * 512 * 16 + 256 * 16 + 1024 + 256
    with pytest.raises(ValueError):
        tt.lmhead_unmask_workspace_bytes(8, 32, 131072, 100)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        B.lib()


@pytest.mark.parametrize("field", ["q", "k_ctx", "v_ctx", "k_blk", "v_blk", "out"])
def test_attn_rejects_misaligned_tensor(field):
    # 16-byte tile loads and stores from every tensor's base: an offset view
    # is refused before anything is enqueued.
    assert attn_call(**{field: FAKE + 8}, ws=FAKE, wsb=1 << 24) == B.TT_EINVAL
    assert attn_call(**{field: FAKE + 2}, dtype=B.TT_BF16, odt=B.TT_BF16, ws=FAKE,
                     wsb=1 << 24) == B.TT_EINVAL


def test_attn_rejects_misaligned_workspace_and_lengths():
    decode = dict(dtype=B.TT_BF16, odt=B.TT_BF16, hq=32, hkv=2, d=128, prefix_len=2048,
                  pcap=2048, block_len=32, batch=8)
    assert attn_call(**decode, ws=FAKE + 4, wsb=1 << 26) == B.TT_EINVAL
    assert varlen_call(lens=FAKE + 2) == B.TT_EINVAL


@pytest.mark.parametrize("kw", [dict(h=FAKE + 2), dict(w=FAKE + 8), dict(ws=FAKE + 4)])
def test_lmhead_rejects_misaligned(kw):
    assert lmhead_call(**kw) == B.TT_EINVAL


def noalloc_call(**kw):
    a = dict(logits=FAKE, mask=FAKE, k=4, tokens=FAKE, mask_out=FAKE, batch=1, L=16, V=1000,
             conf=None, pred=None, stream=None)
    a.update(kw)
    return tt.lib().tt_unmask_step_noalloc(a["logits"], a["mask"], a["k"], a["tokens"],
                                           a["mask_out"], a["batch"], a["L"], a["V"], a["conf"],
                                           a["pred"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), B.TT_EINVAL), (dict(mask=None), B.TT_EINVAL),
    (dict(tokens=None), B.TT_EINVAL), (dict(mask_out=None), B.TT_EINVAL),
    (dict(k=-1), B.TT_EINVAL), (dict(V=0), B.TT_EINVAL), (dict(L=1025), B.TT_EUNSUPPORTED),
    # partials beyond the static scratch: 64 x 1024 positions x 32 chunks x 16 B = 32 MiB
    (dict(batch=64, L=1024, V=131072), B.TT_EUNSUPPORTED),
    (dict(batch=0, logits=None), B.TT_OK),
])
def test_noalloc_validates_before_any_device_call(kw, status):
    assert noalloc_call(**kw) == status


def test_noalloc_scratch_limit_matches_workspace_query():
    # The largest calls that fit: the workspace query's bytes <= 8 MiB.
    assert tt.unmask_workspace_bytes(128, 128, 131072) == B.NOALLOC_SCRATCH_BYTES
    assert noalloc_call(batch=129, L=128, V=131072) == B.TT_EUNSUPPORTED


@pytest.mark.skipif(torch.cuda.is_available(), reason="needs a host without a GPU")
def test_noalloc_without_device_reports_enodev():
    assert noalloc_call() == B.TT_ENODEV


PROBE_LIB = os.path.join(os.path.dirname(B.LIB_PATH), "libtt_probes.so")
PROBE_HEADER = os.path.join(ROOT, "include", "tt_probes.h")


@pytest.mark.skipif(not os.path.exists(PROBE_LIB), reason="libtt_probes.so not built")
def test_probe_library_exports_and_validates():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tt_probe_[a-z0-9_]+)\s*\(", text)))
    exported = os.popen(f"nm -D --defined-only {PROBE_LIB}").read()
    assert sorted(set(re.findall(r"\bT (tt_\w+)", exported))) == names
    lib = ctypes.CDLL(PROBE_LIB)
    lib.tt_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.tt_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.tt_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.tt_probe_mfma_bf16_flops.restype = ctypes.c_double
    assert lib.tt_probe_hbm_read(FAKE, 1000, FAKE, None) == 1        # not a multiple of 16 KB
    assert lib.tt_probe_hbm_read(FAKE + 4, 1 << 14, FAKE, None) == 1  # misaligned
    assert lib.tt_probe_hbm_read(None, 1 << 14, FAKE, None) == 1
    assert lib.tt_probe_mfma_bf16(0, 16, 1, FAKE, None) == 1
    assert lib.tt_probe_mfma_bf16(4, 0, 1, FAKE, None) == 1
    assert lib.tt_probe_mfma_bf16(4, 10, 0, FAKE, None) == 1         # not a multiple of 4
    assert lib.tt_probe_mfma_bf16_flops(512, 4096) == 512 * 16 * 4096 * 2 * 32 * 32 * 16
