"""No kernel of the library chains one bf16 MFMA shape's result into the other
shape's accumulator too soon (the hazard tests/mfma_hazard.py describes): every
HIP source is compiled to gfx950 assembly and scanned.  The checker itself is
checked on the probe tests/hip/mfma_chain.hip, whose two direct chains it must
find.  CPU only (hipcc cross-compiles)."""
import os
import subprocess

import pytest

from mfma_hazard import find_chains

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_81_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-S",
         "--cuda-device-only"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _asm(src, tmp_path):
    # the library's own per-source flags (its scheduler choices), so that the
    # assembly scanned is the assembly that ships
    from gated_delta_rule_81_amd.build import SOURCE_FLAGS
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    extra = SOURCE_FLAGS.get(os.path.basename(src), [])
    subprocess.run([HIPCC, *FLAGS, *extra, src, "-o", out], check=True, capture_output=True)
    return open(out).read()


def test_checker_finds_the_probe_chains(tmp_path):
    chains = find_chains(_asm(os.path.join(ROOT, "tests", "hip", "mfma_chain.hip"), tmp_path))
    pairs = {(a, b) for _, _, a, b, _ in chains}
    assert ("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16") in pairs
    assert ("v_mfma_f32_16x16x16_bf16", "v_mfma_f32_16x16x32_bf16") in pairs
    assert len(chains) == 2  # the padded chain is not reported


@pytest.mark.parametrize("src", ["kda_chunk.hip", "kda_bwd.hip", "kda_bwd_chain.hip", "kda_decode.hip",
                                 "kda_seq.hip", "kda_segment.hip"])
def test_library_has_no_short_mixed_mfma_chains(src, tmp_path):
    chains = find_chains(_asm(os.path.join(CSRC, src), tmp_path))
    assert not chains, chains[:5]


def _dot_without_wait_states(asm):
    """Each v_dot2c_f32_bf16 (written as inline assembly, which the compiler's
    hazard recognizer does not see) not followed directly by an s_nop of at
    least three wait states."""
    lines = [ln.split(";")[0].strip() for ln in asm.splitlines()]
    lines = [ln for ln in lines if ln and not ln.startswith((".", "//"))]
    bad = []
    for i, ln in enumerate(lines):
        if ln.startswith("v_dot2c_f32_bf16"):
            nxt = lines[i + 1] if i + 1 < len(lines) else ""
            ok = nxt.startswith("s_nop") and int(nxt.split()[1], 0) >= 2
            if not ok:
                bad.append((i, ln, nxt))
    return bad


def test_checker_finds_a_dot_without_wait_states():
    asm = "v_dot2c_f32_bf16 v1, v2, v3\nv_add_f32_e32 v4, v1, v1\nv_dot2c_f32_bf16 v1, v2, v3\ns_nop 3\n"
    bad = _dot_without_wait_states(asm)
    assert len(bad) == 1 and bad[0][2].startswith("v_add")


@pytest.mark.parametrize("src", ["kda_bwd.hip"])
def test_inline_dot_products_carry_their_wait_states(src, tmp_path):
    """Another VALU instruction reading a dot product's result needs three wait
    states; the library's inline v_dot2c_f32_bf16 provides them itself (with a
    scheduler that puts the consumer right behind it, the row sums of the
    gradient kernel read stale values otherwise)."""
    asm = _asm(os.path.join(CSRC, src), tmp_path)
    assert "v_dot2c_f32_bf16" in asm
    assert not _dot_without_wait_states(asm)
