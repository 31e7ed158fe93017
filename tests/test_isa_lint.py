"""Compile each kernel source to gfx950 assembly and check two codegen hazards seen with this
toolchain:

- a scalar conditional select (s_cselect) whose condition code was last written by a
  non-compare instruction while the actual comparison went to VCC (v_cmp) in between. That
  pattern silently returned a wrong mask in the top-k kernel; the source now avoids the form
  that produced it;
- private (scratch) memory. Register blocks copied through HIP's vector structs can stay in
  private memory instead of registers; every scratch access is then a vector-memory
  operation that the kernels' counted waits also wait for (the prefill scorer lost about
  a fifth of its time to this). No kernel here needs private memory.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asm(src, out_dir):
    from sparse_attention_indexer_fp4_amd import build as B

    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [B.HIPCC, "-S", "--cuda-device-only", src, "-o", out] + B.FLAGS
    subprocess.run(cmd, check=True, capture_output=True)
    return out


SCC_WRITER = re.compile(r"^\s+(s_cmp\w*|s_(and|or|xor|andn2|orn2|nand|nor|xnor|not)_b\d+|s_(add|sub|addc|subb)_[ui]32|"
                        r"s_(min|max)_\w+|s_(lshl|lshr|ashr)\w*|s_bfe\w*|s_abs\w*|s_bitcmp\w*|"
                        r"s_\w+_saveexec\w*|s_mul_i32|s_absdiff\w*|s_bcnt\w*|s_quadmask\w*|s_wqm\w*)\b")


def suspicious_selects(asm_text):
    lines = asm_text.split("\n")
    hits = []
    for i, line in enumerate(lines):
        if not re.match(r"^\s+s_cselect", line):
            continue
        j = i - 1
        while j >= 0 and not SCC_WRITER.match(lines[j]) and not re.match(r"^\S", lines[j]):
            j -= 1
        if j < 0 or re.match(r"^\S", lines[j]):
            continue  # condition code comes from another block
        between = lines[j + 1:i]
        # a compare, or a uniform lane-mask condition turned into SCC by ANDing it with exec,
        # is the select's intended condition
        intended = lines[j].strip().startswith("s_cmp") or re.match(r"^\s+s_and_b(32|64) [^,]+, [^,]+, exec", lines[j])
        if not intended and any(x.strip().startswith("v_cmp") for x in between):
            hits.append((i, lines[j].strip(), line.strip()))
    return hits


def test_lint_flags_the_known_bad_pattern():
    bad = "\n".join(["\ts_lshr_b32 s4, -1, s30", "\ts_not_b32 s31, s4", "\tv_cmp_eq_u32_e32 vcc, v8, v7",
                     "\ts_cselect_b32 s29, -1, s31"])
    good = "\n".join(["\tv_cmp_eq_u32_e32 vcc, v8, v7", "\ts_cmp_eq_u32 s4, s5", "\ts_cselect_b32 s29, -1, s31"])
    mask = "\n".join(["\ts_and_b64 s[0:1], s[20:21], exec", "\tv_cmp_lt_i32_e32 vcc, v3, v4",
                      "\ts_cselect_b32 s0, s4, 0"])
    # selects read the condition code without writing it: a chain of them after one compare
    chain = "\n".join(["\ts_cmp_eq_u32 s27, 0", "\ts_cselect_b32 s54, s10, s11", "\tv_cmp_lt_i32_e32 vcc, v21, v22",
                       "\ts_cselect_b32 s55, s48, s23"])
    assert suspicious_selects(bad) and not suspicious_selects(good) and not suspicious_selects(mask)
    assert not suspicious_selects(chain)


@pytest.fixture(scope="module")
def kernel_asm():
    from sparse_attention_indexer_fp4_amd import build as B

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES if s != "errors.hip"]
    with tempfile.TemporaryDirectory() as d, concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
        outs = list(ex.map(lambda s: _asm(s, d), srcs))
        return {os.path.basename(src): open(out).read() for src, out in zip(srcs, outs)}


def test_kernels_have_no_stale_condition_selects(kernel_asm):
    for name, text in kernel_asm.items():
        hits = suspicious_selects(text)
        assert not hits, f"{name}: {hits[:3]}"


def scratch_users(asm_text):
    """Kernels whose private segment is not empty: (name, bytes) from the kernel descriptors."""
    out = []
    for m in re.finditer(r"^\s*\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm_text, re.M | re.S):
        size = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
        if size and int(size.group(1)) != 0:
            out.append((m.group(1), int(size.group(1))))
    return out


def test_lint_finds_private_segments():
    text = "\n".join(["\t.amdhsa_kernel k0", "\t\t.amdhsa_private_segment_fixed_size 0", "\t.end_amdhsa_kernel",
                      "\t.amdhsa_kernel k1", "\t\t.amdhsa_private_segment_fixed_size 192", "\t.end_amdhsa_kernel"])
    assert scratch_users(text) == [("k1", 192)]


def test_kernels_use_no_scratch(kernel_asm):
    for name, text in kernel_asm.items():
        assert ".amdhsa_kernel" in text, name
        users = scratch_users(text)
        assert not users, f"{name}: {users[:3]}"
