"""The inline-asm MFMAs of the attention kernels keep their wait states in the generated
code (CPU: compiles k_attn.hip for gfx950 with the library's flags and checks the
assembly), and the checker itself flags the cases it is meant to find."""
import os
import subprocess

import pytest

from asm_hazards import check

KERNELS = {
    "bf16": "_ZN4lact21k_attn_bf16_d128_dualENS_8AttnArgsE",  # lact::k_attn_bf16_d128_dual(AttnArgs)
    "f8v": "_ZN4lact20k_attn_f8v_d128_dualENS_8AttnArgsE",    # lact::k_attn_f8v_d128_dual(AttnArgs)
}

SNIPPET = """{name}:
\tv_mov_b32 v1, 0
{nops}\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[10:25], v[0:3], a[0:3], v[10:25]
\t;;#ASMEND
{nops2}\tv_add_f32_e32 v30, v12, v12
\ts_endpgm
"""


def test_checker_flags_close_operand_write_and_result_read():
    text = SNIPPET.format(name="k", nops="", nops2="")
    issues = check(text, "k")
    assert any(i.startswith("PRE 0: v_mov_b32 v1") for i in issues)
    assert any(i.startswith("POST 0:") and "v_add_f32" in i for i in issues)


def test_checker_accepts_separated_instructions():
    text = SNIPPET.format(name="k", nops="\ts_nop 7\n", nops2="\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n")
    assert check(text, "k") == []


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    from compressed_kv_causal_amd import build as B
    out = tmp_path_factory.mktemp("asm") / "k_attn.s"
    cmd = ([B.HIPCC] + B.COMMON + ["--offload-device-only", "-S", "-o", str(out),
                                   os.path.join(B.CSRC, "k_attn.hip")])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
@pytest.mark.parametrize("which", sorted(KERNELS))
def test_dual_kernel_inline_asm_mfma_hazards(kernel_asm, which):
    kernel = KERNELS[which]
    text = kernel_asm
    assert kernel + ":" in text
    body = text[text.index(kernel + ":"):]
    body = body[:body.index("s_endpgm")]
    assert body.count(";;#ASMSTART") > 0 and "v_mfma" in body
    issues = check(text, kernel)
    assert issues == [], "\n".join(issues[:20])
