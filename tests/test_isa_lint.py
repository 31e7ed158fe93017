"""Compile each kernel source to gfx950 assembly and check a codegen hazard seen with this
toolchain: a scalar conditional select (s_cselect) whose condition code was last written by
a non-compare instruction while the actual comparison went to VCC (v_cmp) in between. That
pattern silently returned a wrong mask in the top-k kernel; the source now avoids the form
that produced it, and this test keeps any kernel from reintroducing it."""
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
                        r"s_(min|max)_\w+|s_(lshl|lshr|ashr)\w*|s_bfe\w*|s_abs\w*|s_bitcmp\w*|s_cselect\w*|"
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
    assert suspicious_selects(bad) and not suspicious_selects(good) and not suspicious_selects(mask)


def test_kernels_have_no_stale_condition_selects():
    from sparse_attention_indexer_fp4_amd import build as B

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES if s != "errors.hip"]
    with tempfile.TemporaryDirectory() as d, concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
        outs = list(ex.map(lambda s: _asm(s, d), srcs))
        for src, out in zip(srcs, outs):
            hits = suspicious_selects(open(out).read())
            assert not hits, f"{os.path.basename(src)}: {hits[:3]}"
