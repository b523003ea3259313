"""The host-side dispatch log: with FLEXATTN_LOG set (to anything but "" or
"0") every entry point that can launch work prints one line on stderr when it
returns, naming its arguments, the kernels it launched and its status; unset
or "0", nothing. Each case runs in a child process, since the library reads
the variable once per process.

The CPU cases pass fake, never-dereferenced addresses that fail validation
(no launch) and are skipped where a GPU is visible; the GPU case runs one
small forward, a split decode step and a backward and checks the kernel names
the log reports."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

REJECTED = r"""
import attention_tiled_attn_amd as fa
A = 0x10000
print(fa.flexattn_fwd(A, A, A, A, A, 1, 2, 2, 128, 128, 96, 0.125, 0, 0, check=False))
print(fa.flexattn_fwd(None, A, A, A, A, 1, 2, 2, 128, 128, 64, 0.125, 1, 0, check=False))
print(fa.flexattn_decode(A, A, A, A, A, 1, 2, 2, 1, 128, 64, 0.125, 0, 0, None, None, 0, A, 0, check=False))
print(fa.flexattn_bwd(A, A, A, A, A, A, A, A, A, A, 1, 3, 2, 128, 128, 64, 0.125, 0, 0, check=False))
print(fa.flexattn_build_block_mask(17, None, 1, 256, 256, A, 64, fa.BlockMask(), check=False))
print(fa.flexattn_block_mask_bytes(1, 256, 256, 1))
"""


def _child(script: str, value: str | None, timeout: int = 300) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.pop("FLEXATTN_LOG", None)
    if value is not None:
        env["FLEXATTN_LOG"] = value
    return subprocess.run([sys.executable, "-c", script], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _log_lines(stderr: str) -> list[str]:
    return [ln for ln in stderr.splitlines() if ln.startswith("[flexattn] ")]


@pytest.fixture(scope="module")
def cpu_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation cases run only without a GPU")
    from attention_tiled_attn_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libflexattn.so is not built (python -m attention_tiled_attn_amd.build)")


def test_log_lines_for_rejected_calls(cpu_only):
    from attention_tiled_attn_amd import _lib
    r = _child(REJECTED, "1")
    assert r.returncode == 0, r.stderr[-3000:]
    codes = [int(x) for x in r.stdout.split()]
    assert codes[:5] == [_lib.ERR_UNSUPPORTED, _lib.ERR_NULLPTR, _lib.ERR_ARG, _lib.ERR_SHAPE,
                         _lib.ERR_UNSUPPORTED]
    lines = _log_lines(r.stderr)
    # one line per call of a launching entry point; the size query logs nothing
    assert [ln.split("(")[0] for ln in lines] == [
        "[flexattn] flexattn_fwd", "[flexattn] flexattn_fwd", "[flexattn] flexattn_decode",
        "[flexattn] flexattn_bwd", "[flexattn] flexattn_build_block_mask"]
    for ln, code in zip(lines, codes):
        assert ln.endswith(f"-> no launch -> {code} ({_lib.lib().flexattn_strerror(code).decode()})"), ln
    assert "B=1 H=2 Hkv=2 Sq=128 Skv=128 D=96 bf16 scale=0.125 mask=0x0 mod=0 block_mask=none" in lines[0]
    assert "mask=0x1" in lines[1]
    assert "splits=0" in lines[2]
    assert "H=3 Hkv=2" in lines[3]
    assert "mask=0x11 B=1 Sq=256 Skv=256 bytes=64" in lines[4]


@pytest.mark.parametrize("value", [None, "", "0"])
def test_log_off(cpu_only, value):
    r = _child(REJECTED, value)
    assert r.returncode == 0, r.stderr[-3000:]
    assert _log_lines(r.stderr) == []


LAUNCHES = r"""
import torch, attention_tiled_attn_amd as fa
print("[case] dispatch log: forward B1 H2 S256 D128, causal; decode split 4; backward", flush=True)
g = torch.Generator(device="cuda").manual_seed(7)
q, k, v = (torch.randn(1, 2, 256, 128, generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(3))
out, lse = fa.attention(q, k, v, block_mask=None)
out, lse = fa.attention(q, k, v, fa.Variant(causal=True))
qd = torch.randn(1, 2, 1, 128, generator=g, device="cuda", dtype=torch.bfloat16)
fa.decode(qd, k, v, splits=4, block_mask=None)
dq, dk, dv = fa.attention_backward(q, k, v, out, lse, torch.ones_like(out), fa.Variant(causal=True))
torch.cuda.synchronize()
print("done", flush=True)
"""


@pytest.mark.gpu
def test_log_names_launched_kernels():
    r = _child(LAUNCHES, "1", timeout=240)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    lines = _log_lines(r.stderr)
    print("\n".join(lines))
    ok = "-> 0 (success)"
    fwd = [ln for ln in lines if ln.startswith("[flexattn] flexattn_fwd(")]
    assert len(fwd) == 2 and all(ln.endswith(ok) for ln in fwd)
    assert "attn_fwd_pp_kernel<128, 0, false, 0> grid 8 x 512 splits 1" in fwd[0]
    assert "block_mask=none" in fwd[0] and "block_mask=given" in fwd[1]
    bm = [ln for ln in lines if ln.startswith("[flexattn] flexattn_build_block_mask(")]
    assert len(bm) == 2 and all("block_mask_kernel grid 1 x 1 x 64" in ln and ln.endswith(ok) for ln in bm)
    dec = [ln for ln in lines if ln.startswith("[flexattn] flexattn_decode(")]
    assert len(dec) == 1 and dec[0].endswith(ok)
    assert re.search(r"attn_fwd_pp_kernel<128, 0, false, 2> grid \d+ x 512 splits 4; "
                     r"attn_decode_merge_kernel grid \d+ x 256", dec[0]), dec[0]
    bwd = [ln for ln in lines if ln.startswith("[flexattn] flexattn_bwd(")]
    assert len(bwd) == 1 and bwd[0].endswith(ok)
    assert re.search(r"attn_bwd_dq_kernel<128, 0, false> grid \d+ x 256; "
                     r"attn_bwd_dkdv2_kernel<128, 0, false> grid \d+ x 512", bwd[0]), bwd[0]
