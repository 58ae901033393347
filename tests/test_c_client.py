"""The C ABI from a plain C99 program (tests/c/tt_c_client.c, built by the
package build with gcc against include/tt.h and libtt.so, no Python in the
loop): the header compiles as C; the host-side calls and the argument checks
answer as they do through the Python binding; on the GPU, one denoising step
run from C (tt_block_attn, then tt_unmask_step) matches the oracle."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from denoiser_attention_amd import build as Bd
from denoiser_attention_amd import synth
from helpers import check_attn, check_unmask, oracle_attn, say

TT_EINVAL = 1


def _client():
    if not os.path.exists(Bd.C_CLIENT):
        pytest.skip("no build here yet (run the build first)")
    return Bd.C_CLIENT


def test_header_compiles_as_c99(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "h.c"
    src.write_text('#include "tt.h"\nint main(void) { return tt_version() == 0; }\n')
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", Bd.INCLUDE, "-I", os.path.join(rocm, "include"), "-fsyntax-only",
                        str(src)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_host_calls_from_c():
    import torch

    import denoiser_attention_amd as tt

    r = subprocess.run([_client(), "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert got["version"] == tt.version()
    assert got["status_ok"] == "TT_OK"
    assert got["status_einval"].startswith("TT_EINVAL")
    assert int(got["attn_ws_decode"]) == tt.attn_workspace_bytes(8, 2048, 32, 32, 2, 128,
                                                                 torch.bfloat16)
    assert int(got["attn_ws_highbatch"]) == tt.attn_workspace_bytes(64, 4096, 64, 32, 2, 128,
                                                                    torch.bfloat16)
    assert got["attn_ws_bad_heads"] == "1"
    assert int(got["unmask_ws_decode"]) == tt.unmask_workspace_bytes(8, 32, 131072)
    for key in ("attn_bad_heads", "attn_prefix_over_cap", "attn_null_out", "unmask_negative_k",
                "unmask_short_workspace"):
        assert int(got[key]) == TT_EINVAL, key


@pytest.mark.gpu
@pytest.mark.parametrize("P", [100, 0])
def test_step_from_c_matches_oracle(tmp_path, P):
    """GQA 4:1 bf16 attention over a ragged prefix and block (3 + 1 query row
    tiles' worth of packed rows, a ragged last key tile), then the unmask of a
    random mask over a 5000-word vocabulary; the GPU is used by the C child
    process only."""
    client = _client()
    cfg = synth.get_config("decode_b8_p2048_l32").with_(
        batch=2, n_q_heads=8, n_kv_heads=2, prefix_len=P, block_len=24, vocab=5000)
    B, Hq, Hkv, L, D, V, k = 2, 8, 2, 24, 128, 5000, cfg.k
    inp = synth.attn_inputs(cfg, seed=21, prefix_cap=P)
    x = synth.logits(cfg, seed=21, step=0)
    rng = np.random.default_rng(21)
    mask = (rng.random((B, L)) < 0.8).astype(np.uint8)
    tokens0 = np.full((B, L), 7, np.int32)
    with open(tmp_path / "shape.txt", "w") as f:
        f.write(f"{B} {Hq} {Hkv} {L} {P} {D} {k} {V} {inp['scale']!r}\n")
    for name in ("q", "k_ctx", "v_ctx", "k_blk", "v_blk"):
        np.ascontiguousarray(inp[name]).astype(np.uint16).tofile(tmp_path / f"{name}.bin")
    np.ascontiguousarray(x, dtype=np.float32).tofile(tmp_path / "logits.bin")
    mask.tofile(tmp_path / "mask.bin")
    tokens0.tofile(tmp_path / "tokens.bin")

    say(f"C client step: B{B} Hq{Hq} Hkv{Hkv} L{L} P{P} D{D} V{V} k{k}")
    r = subprocess.run([client, "gpu", str(tmp_path)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    out = np.fromfile(tmp_path / "out.bin", np.uint16).reshape(B, Hq, L, D)
    check_attn(oracle.decode_bf16(out), oracle_attn(inp), "bf16", True, f"C client P={P}")
    got = dict(tokens=np.fromfile(tmp_path / "tokens_out.bin", np.int32).reshape(B, L),
               mask_out=np.fromfile(tmp_path / "mask_out.bin", np.uint8).reshape(B, L),
               conf=np.fromfile(tmp_path / "conf.bin", np.float32).reshape(B, L),
               pred=np.fromfile(tmp_path / "pred.bin", np.int32).reshape(B, L))
    ref = oracle.unmask_step(x, mask, k)
    check_unmask(got, ref, mask, k, tokens0, f"C client unmask P={P}")
