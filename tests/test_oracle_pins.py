"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself:
hand-worked codes and scores (tests/golden), an exhaustive cross-check of the element
rounding against an independently written threshold encoder, the pages' description of
the scale plane as a 16x4 transpose, a brute-force unpaged scorer, exact integer dot
products, invariances (power-of-two scaling, page permutation), padding rows that read no
key, a brute-force top-k, and the coverage of the work schedules.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _parse_value(tok):
    tok = tok.strip()
    if "^" in tok:
        if "*" in tok:
            a, p = tok.split("*")
            return float(a) * 2.0 ** int(p.split("^")[1])
        return 2.0 ** int(tok.split("^")[1])
    return float(tok)


def _block_bits(values):
    v = np.zeros(32, np.float32)
    v[: len(values)] = values
    bits = W.bf16_bits(v)
    # every golden value must be exact in bf16, or the fixture is wrong
    assert np.array_equal(W.bf16_to_f32(bits), v), values
    return bits


def _vec_bits(values):
    v = np.zeros(128, np.float32)
    v[: len(values)] = values
    bits = W.bf16_bits(v)
    assert np.array_equal(W.bf16_to_f32(bits), v)
    return bits


# ---------------------------------------------------------------------------- encodings

def test_golden_blocks_codes_scales_and_packing():
    cases = list(_lines("mx_blocks.txt"))
    assert len(cases) >= 8
    for line in cases:
        vals_s, scale_s, codes_s, packed_s = [p.strip() for p in line.split(";")]
        vals = [_parse_value(t) for t in vals_s.split(",")]
        bits = _block_bits(vals)
        scale, codes = oracle.mx_encode_blocks(bits[None, :])
        assert scale[0] == int(scale_s, 16), line
        want = [int(c, 16) for c in codes_s.split()]
        assert list(codes[0, : len(want)]) == want, line
        assert not codes[0, len(want):].any() or all(c in (0, 8) for c in codes[0, len(want):])
        # packing through the cache writer: key = this block in group 0, zeros elsewhere
        key = np.zeros((1, 128), np.uint16)
        key[0, :32] = bits
        kp = np.zeros((1, 64, 64), np.uint8)
        ks = np.zeros((1, 4, 64), np.uint8)
        oracle.quant_and_cache(key, np.array([5], np.int64), kp, ks)
        want_packed = [int(b, 16) for b in packed_s.split()]
        assert list(kp[0, 5, : len(want_packed)]) == want_packed, line
        assert ks[0, 0, oracle.scale_slot(5)] == int(scale_s, 16)


def _bf16_floor_log2(bits):
    """floor(log2|v|) of nonzero finite bf16 patterns, read off the exponent field."""
    bits = bits.astype(np.int64)
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    out = e - 127
    sub = e == 0
    if sub.any():
        msb = np.floor(np.log2(np.maximum(m[sub], 1))).astype(np.int64)  # m < 128: exact
        out[sub] = msb - 133
    return out


def _threshold_code(x):
    """E2M1 magnitude code from decision thresholds (ties go to the even code)."""
    x = np.asarray(x, np.float64)
    c = np.full(x.shape, 7, np.int64)
    c[x <= 5.0] = 6
    c[x < 3.5] = 5
    c[x <= 2.5] = 4
    c[x < 1.75] = 3
    c[x <= 1.25] = 2
    c[x < 0.75] = 1
    c[x <= 0.25] = 0
    return c


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e = (b.astype(np.int64) >> 7) & 0xFF
    return b[e != 0xFF]


def test_exhaustive_element_rounding_self_scaled():
    """Every finite bf16 value alone in a block: its own amax fixes the scale, so the
    rescaled magnitude lands in [4, 8) and exercises codes 6/7, the 5.0 tie and saturation."""
    bits = _all_finite_bf16()
    blocks = np.zeros((bits.size, 32), np.uint16)
    blocks[:, 0] = bits
    scale, codes = oracle.mx_encode_blocks(blocks)
    v = W.bf16_to_f32(bits).astype(np.float64)
    nz = v != 0
    fl = np.zeros(bits.size, np.int64)
    fl[nz] = _bf16_floor_log2(bits[nz])
    e = np.clip(fl - 2, -127, 127)
    e[~nz] = -127
    assert np.array_equal(scale.astype(np.int64), e + 127)
    x = np.abs(v) / np.exp2(e.astype(np.float64))
    want = _threshold_code(x) | np.where(np.signbit(v), 8, 0)
    assert np.array_equal(codes[:, 0].astype(np.int64), want)
    assert not codes[:, 1:].any()
    # unclamped blocks: the rescaled amax sits in [4, 8) -- the "largest exponent 2" rule
    ok = nz & (fl - 2 >= -127)
    assert ((x[ok] >= 4.0) & (x[ok] < 8.0)).all()


@pytest.mark.parametrize("e", range(-10, 11))
def test_exhaustive_element_rounding_fixed_scale(e):
    """Block [2^(e+2), v] for every bf16 v with |v| < 2^(e+2): scale exponent e, and the
    element code of v is its nearest grid point below 4 (ties at 0.25 .. 3.5)."""
    bits = _all_finite_bf16()
    v = W.bf16_to_f32(bits).astype(np.float64)
    A = 2.0 ** (e + 2)
    sel = np.abs(v) < A
    bits, v = bits[sel], v[sel]
    blocks = np.zeros((bits.size, 32), np.uint16)
    blocks[:, 0] = W.bf16_bits(np.full(bits.size, A, np.float32))
    blocks[:, 1] = bits
    scale, codes = oracle.mx_encode_blocks(blocks)
    assert (scale == e + 127).all()
    assert (codes[:, 0] == 6).all()  # the amax element itself is 4 * 2^e
    want = _threshold_code(np.abs(v) / 2.0 ** e) | np.where(np.signbit(v), 8, 0)
    assert np.array_equal(codes[:, 1].astype(np.int64), want)


def test_value_tables():
    for c in range(16):
        mag = E2M1[c & 7]
        assert oracle.e2m1_value(c) == (-mag if c & 8 else mag)
    for b in (0, 1, 126, 127, 128, 254):
        assert oracle.e8m0_value(b) == 2.0 ** (b - 127)


# ---------------------------------------------------------------------------- swizzle

def test_scale_slots_golden_and_transpose():
    pairs = [tuple(int(t) for t in line.split()) for line in _lines("scale_slots.txt")]
    for pos, slot in pairs:
        assert oracle.scale_slot(pos) == slot
    slots = np.array([oracle.scale_slot(p) for p in range(64)])
    assert sorted(slots) == list(range(64))  # a permutation of the 64 slots
    # "16x4 transpose": positions laid out as 4 rows of 16 land as the transposed 16x4
    grid = np.empty(64, np.int64)
    grid[slots] = np.arange(64)
    assert np.array_equal(grid.reshape(16, 4), np.arange(64).reshape(4, 16).T)


def test_writer_places_scales_by_slot_and_keys_flat():
    """Key at position p gets a distinct amax 2^(p-20); its four scale bytes must land in
    slot(p) of each group plane and its packed bytes in flat row p."""
    keys = np.zeros((64, 128), np.float32)
    for p in range(64):
        for g in range(4):
            keys[p, 32 * g] = 2.0 ** (p - 20 + g)
            keys[p, 32 * g + 1] = -(2.0 ** (p - 20 + g))
    kp = np.zeros((2, 64, 64), np.uint8)
    ks = np.zeros((2, 4, 64), np.uint8)
    oracle.quant_and_cache(W.bf16_bits(keys), np.arange(64, 128, dtype=np.int64), kp, ks)
    assert not kp[0].any() and not ks[0].any()
    for p in range(64):
        for g in range(4):
            assert ks[1, g, (p % 16) * 4 + p // 16] == 127 + (p - 20 + g) - 2
            assert kp[1, p, 16 * g] == 0x6 | (0xE << 4)
    # a slot < 0 is skipped; untouched bytes keep their poison
    kp2 = np.full((1, 64, 64), 0xA5, np.uint8)
    ks2 = np.full((1, 4, 64), 0x5A, np.uint8)
    oracle.quant_and_cache(W.bf16_bits(keys[:2]), np.array([-1, 3], np.int64), kp2, ks2)
    assert (kp2[0, 0] == 0xA5).all() and not (kp2[0, 3] == 0xA5).all()
    assert (np.delete(kp2[0], 3, axis=0) == 0xA5).all()
    touched = {(g, oracle.scale_slot(3)) for g in range(4)}
    for g in range(4):
        for s in range(64):
            if (g, s) not in touched:
                assert ks2[0, g, s] == 0x5A


# ---------------------------------------------------------------------------- scores

def _one_row_case(qvals, kvals, w, heads=1):
    q = np.zeros((1, heads, 128), np.uint16)
    q[0, 0] = _vec_bits(qvals)
    qp, qs = oracle.quant_q(q)
    kp = np.zeros((1, 64, 64), np.uint8)
    ks = np.zeros((1, 4, 64), np.uint8)
    oracle.quant_and_cache(_vec_bits(kvals)[None, :], np.array([0], np.int64), kp, ks)
    wv = np.zeros((1, heads), np.float32)
    wv[0, 0] = w
    s, reads = oracle.score(qp, qs, wv, np.array([0], np.int32), np.array([1], np.int32), kp, ks,
                            np.array([[0]], np.int32))
    return s[0, 0], reads[0]


def test_worked_dots():
    n = 0
    for line in _lines("worked_dots.txt"):
        qs, ks, w, want = [p.strip() for p in line.split(";")]
        qv = [_parse_value(t) for t in qs.split(",")]
        kv = [_parse_value(t) for t in ks.split(",")]
        got, reads = _one_row_case(qv, kv, float(w))
        assert got == float(want), line
        assert reads == 1
        n += 1
    assert n == 3


def _exact_dot(qp, qs, kp, ks, page, pos, row, h):
    """Per-head dot from the codes in exact rational arithmetic (independent of dequant)."""
    total = Fraction(0)
    for g in range(4):
        sq = int(qs[row, h, g]) - 127
        sk = int(ks[page, g, (pos % 16) * 4 + pos // 16]) - 127
        acc = Fraction(0)
        for i in range(32):
            d = 32 * g + i
            bq = int(qp[row, h, d // 2])
            bk = int(kp[page, pos, d // 2])
            cq = (bq >> 4) if d % 2 else (bq & 0xF)
            ck = (bk >> 4) if d % 2 else (bk & 0xF)
            vq = Fraction(E2M1[cq & 7]).limit_denominator() * (-1 if cq & 8 else 1)
            vk = Fraction(E2M1[ck & 7]).limit_denominator() * (-1 if ck & 8 else 1)
            acc += vq * vk
        total += acc * Fraction(2) ** (sq + sk)
    return total


def test_single_head_scores_equal_exact_rational_dots():
    case = W.decode_case([130], heads=1, topk=8, seed=3)
    qp, qs = oracle.quant_q(case.q)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    w = np.ones((1, 1), np.float32)
    rs, rl = oracle.decode_geometry(case.ctx)
    s, _ = oracle.score(qp, qs, w, rs, rl, kp, ks, case.block_table)
    npos = 0
    for j in range(130):
        page = case.block_table[0, j // 64]
        exact = _exact_dot(qp, qs, kp, ks, page, j % 64, 0, 0)
        want = max(exact, Fraction(0))
        assert Fraction(s[0, j]) == want, j
        npos += exact > 0
    assert 20 < npos < 110  # both signs occur, so ReLU is exercised


def _dense_scores(q_codes, q_scales, w, k_codes, k_scales):
    """Unpaged brute force: dequantize from the encoder's codes in numpy, then score with
    an explicit head loop (same summation order over heads, exact per-head dots)."""
    grid = np.array(E2M1)

    def deq(codes, scales):  # codes [..., 4, 32], scales [..., 4]
        v = grid[codes & 7] * np.where(codes & 8, -1.0, 1.0)
        return (v * np.exp2(scales.astype(np.float64) - 127)[..., None]).reshape(*codes.shape[:-2], 128)

    qd = deq(q_codes, q_scales)  # [H, 128]
    kd = deq(k_codes, k_scales)  # [n, 128]
    s = np.zeros(kd.shape[0])
    for h in range(qd.shape[0]):
        dot = kd @ qd[h]
        s = s + np.float64(w[h]) * np.maximum(dot, 0.0)
    return s


@pytest.mark.parametrize("sens", [False, True])
def test_paged_equals_unpaged_bruteforce(sens):
    case = W.decode_config("decode_tiny", swizzle_sensitive=sens)
    qp, qs = oracle.quant_q(case.q)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    rs, rl = oracle.decode_geometry(case.ctx)
    s, reads = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table)
    assert list(reads) == list(case.ctx)
    off = 0
    for b in range(case.batch):
        L = int(case.ctx[b])
        kbits = case.keys[off:off + L]
        off += L
        ksc, kcodes = oracle.mx_encode_blocks(kbits.reshape(-1, 32))
        qsc, qcodes = oracle.mx_encode_blocks(case.q[b].reshape(-1, 32))
        dense = _dense_scores(qcodes.reshape(-1, 4, 32), qsc.reshape(-1, 4), case.w[b],
                              kcodes.reshape(L, 4, 32), ksc.reshape(L, 4))
        # per-head dots are exact in fp64 for these inputs, and heads are summed in the
        # same order, so the two must agree bit for bit
        assert np.array_equal(s[b, :L], dense), b
        assert np.isnan(s[b, L:]).all()


def test_swizzle_sensitive_keys_change_scores_if_scales_are_read_flat():
    """With per-token power-of-two scaling, reading a key's scale from the flat row instead
    of its slot gives different scores (what went wrong in the pages' second review
    finding); the pinned oracle does not."""
    case = W.decode_config("decode_tiny", swizzle_sensitive=True)
    qp, qs = oracle.quant_q(case.q)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    rs, rl = oracle.decode_geometry(case.ctx)
    s, _ = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table)
    # un-swizzle the plane so a flat read is wrong: move slot(p) -> p
    flat = np.empty_like(ks)
    for p in range(64):
        flat[:, :, p] = ks[:, :, oracle.scale_slot(p)]
    s_wrong, _ = oracle.score(qp, qs, case.w, rs, rl, kp, flat, case.block_table)
    L = int(case.ctx[0])
    assert np.mean(s_wrong[0, :L] != s[0, :L]) > 0.5


def test_power_of_two_query_scaling_scales_scores_exactly():
    case = W.decode_config("decode_tiny")
    qp, qs = oracle.quant_q(case.q)
    q2 = W.bf16_bits(W.bf16_to_f32(case.q) * 2.0)
    qp2, qs2 = oracle.quant_q(q2)
    assert np.array_equal(qp, qp2) and np.array_equal(qs2.astype(int), qs.astype(int) + 1)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    rs, rl = oracle.decode_geometry(case.ctx)
    s, _ = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table)
    s2, _ = oracle.score(qp2, qs2, case.w, rs, rl, kp, ks, case.block_table)
    m = ~np.isnan(s)
    assert np.array_equal(s2[m], 2.0 * s[m])


def test_page_permutation_invariance():
    case = W.decode_config("decode_tiny")
    qp, qs = oracle.quant_q(case.q)
    rs, rl = oracle.decode_geometry(case.ctx)

    def run(bt, slots, n_pages):
        kp = np.zeros((n_pages, 64, 64), np.uint8)
        ks = np.zeros((n_pages, 4, 64), np.uint8)
        oracle.quant_and_cache(case.keys, slots, kp, ks)
        return oracle.score(qp, qs, case.w, rs, rl, kp, ks, bt)[0]

    base = run(case.block_table, case.slots, case.n_pages)
    perm = np.random.default_rng(7).permutation(case.n_pages + 5).astype(np.int32)
    bt2 = np.where(case.block_table >= 0, perm[np.maximum(case.block_table, 0)], -1).astype(np.int32)
    slots2 = perm[case.slots // 64].astype(np.int64) * 64 + case.slots % 64
    other = run(bt2, slots2, case.n_pages + 5)
    assert np.array_equal(np.isnan(base), np.isnan(other))
    assert np.array_equal(base[~np.isnan(base)], other[~np.isnan(other)])


# ---------------------------------------------------------------------------- geometry

def test_decode_geometry_staggers_speculative_rows():
    rs, rl = oracle.decode_geometry(np.array([10, 300], np.int32), next_n=3)
    assert list(rs) == [0, 0, 0, 1, 1, 1]
    assert list(rl) == [8, 9, 10, 298, 299, 300]


def test_padding_rows_read_no_key():
    case = W.prefill_config("prefill_tiny")
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    for st in case.steps:
        k, sl = W.step_keys(case, st)
        oracle.quant_and_cache(k, sl, kp, ks)
        rs, rl = oracle.prefill_geometry(st.cu_rows, st.start_pos, st.n_rows_padded)
        assert st.n_rows_padded > st.n_rows  # every tiny step carries padding rows
        pad = np.arange(st.n_rows_padded) >= st.n_rows
        assert (rl[pad] == 0).all() and (rs[pad] == len(st.req_ids) - 1).all()
        qp, qs = oracle.quant_q(st.q)
        bt = W.step_block_table(case, st)
        s, reads = oracle.score(qp, qs, st.w, rs, rl, kp, ks, bt, ld=int(case.lengths.max()))
        assert (reads[pad] == 0).all()
        assert np.array_equal(reads[~pad], rl[~pad].astype(np.int64))
        assert np.isnan(s[pad]).all()
        top = oracle.topk(s, rl, case.topk)
        assert (top[pad] == -1).all()
        # causal rows: row r of request i sees exactly positions [0, start + r - first]
        for i in range(len(st.req_ids)):
            for r in range(st.cu_rows[i], st.cu_rows[i + 1]):
                assert rl[r] == st.start_pos[i] + (r - st.cu_rows[i]) + 1


# ---------------------------------------------------------------------------- top-k

def _bruteforce_topk(s, L, k):
    """k rounds of argmax over the row, the lowest column winning a tie."""
    taken = np.zeros(L, bool)
    out = []
    for _ in range(min(k, L)):
        best = -1
        for j in range(L):
            if not taken[j] and (best < 0 or s[j] > s[best]):
                best = j
        taken[best] = True
        out.append(best)
    return out + [-1] * (k - len(out))


def test_topk_matches_bruteforce():
    case = W.decode_config("decode_tiny")
    qp, qs = oracle.quant_q(case.q)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    rs, rl = oracle.decode_geometry(case.ctx)
    s, _ = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table)
    top = oracle.topk(s, rl, case.topk)
    for r in range(case.rows):
        assert list(top[r]) == _bruteforce_topk(s[r], int(rl[r]), case.topk)


def test_topk_ties_short_rows_and_bounds():
    s = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 9.0, 9.0, 0.0],
                  [5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0, 5.0],
                  [0.0, -1.0, 7.0, np.nan, np.nan, np.nan, np.nan, np.nan]])
    rl = np.array([6, 8, 3], np.int32)
    top = oracle.topk(s, rl, 4)
    assert list(top[0]) == [5, 1, 2, 4]      # 9 past the row end is never seen
    assert list(top[1]) == [0, 1, 2, 3]      # all tied: lowest columns
    assert list(top[2]) == [2, 0, 1, -1]     # short row keeps every key, padded with -1
    for r in range(3):
        assert list(top[r]) == _bruteforce_topk(s[r], int(rl[r]), 4)


# ---------------------------------------------------------------------------- schedules

def _check_partition(unit_begin, n_items, n_units):
    ub = np.asarray(unit_begin, np.int64)
    assert ub[0] == 0 and ub[n_units] == n_items
    assert (np.diff(ub) >= 0).all()
    sizes = np.diff(ub)
    assert sizes.max() - sizes.min() <= 1  # an even split


@pytest.mark.parametrize("ctx,units", [([300, 512], 512), ([4096], 512), ([0, 65, 64, 1, 0], 7),
                                       ([131072] * 8, 512), ([5] * 600, 512)])
def test_decode_schedule_covers_every_page_once(ctx, units):
    ctx = np.array(ctx, np.int32)
    sch = oracle.decode_schedule(ctx, units)
    pages = (ctx.astype(np.int64) + 63) // 64
    assert list(sch["cum_pages"]) == [0] + list(np.cumsum(pages))
    n_items = int(pages.sum())
    _check_partition(sch["unit_begin"], n_items, units)
    covered = np.zeros(n_items, np.int64)
    for u in range(units):
        a, b = sch["unit_begin"][u], sch["unit_begin"][u + 1]
        covered[a:b] += 1
        seq = sch["unit_seq"][u]
        if a < n_items:
            assert sch["cum_pages"][seq] <= a < sch["cum_pages"][seq + 1]
        else:
            assert seq == len(ctx)
    assert (covered == 1).all()


def _ints(field):
    return [int(t) for t in field.split()]


def test_schedules_and_geometry_golden():
    """Hand-worked decode schedules and prefill geometry/tiles (tests/golden/schedules.txt)."""
    n_dec = n_pre = 0
    for line in _lines("schedules.txt"):
        f = [t.strip() for t in line.split(";")]
        if f[0] == "decode":
            ctx = np.array(_ints(f[1]), np.int32)
            sch = oracle.decode_schedule(ctx, int(f[2]))
            assert list(sch["cum_pages"]) == _ints(f[3])
            assert list(sch["unit_begin"]) == _ints(f[4])
            assert list(sch["unit_seq"]) == _ints(f[5])
            n_dec += 1
        else:
            cu, sp = np.array(_ints(f[1]), np.int32), np.array(_ints(f[2]), np.int32)
            npad, units = int(f[3]), int(f[4])
            rs, rl = oracle.prefill_geometry(cu, sp, npad)
            assert list(rs) == _ints(f[5]) and list(rl) == _ints(f[6])
            sch = oracle.prefill_schedule(cu, sp, npad, 8, units)
            assert [list(t) for t in sch["tiles"]] == [_ints(t) for t in f[7].split(",")]
            assert list(sch["cum_items"]) == _ints(f[8])
            assert list(sch["unit_begin"]) == _ints(f[9])
            assert list(sch["unit_tile"]) == _ints(f[10])
            n_pre += 1
    assert n_dec >= 4 and n_pre >= 2


@pytest.mark.parametrize("which", ["prefill_tiny", "prefill_tiny_mbt", "prefill_4req", "prefill_4req_mbt512"])
@pytest.mark.parametrize("tile_rows", [8, 16])
def test_prefill_schedule_covers_rows_and_pages_once(which, tile_rows):
    case = W.prefill_config(which, heads=4)
    TR = tile_rows
    for st in case.steps:
        units = 4096 if which.startswith("prefill_4req") else 13
        sch = oracle.prefill_schedule(st.cu_rows, st.start_pos, st.n_rows_padded, TR, units)
        rs, rl = oracle.prefill_geometry(st.cu_rows, st.start_pos, st.n_rows_padded)
        tiles = sch["tiles"]
        # every row in exactly one tile; tiles inside one group, aligned to its start
        seen = np.zeros(st.n_rows_padded, np.int64)
        R = len(st.req_ids)
        for r0, nr, req, npg in tiles:
            seen[r0:r0 + nr] += 1
            assert 1 <= nr <= TR
            first = st.cu_rows[req]
            end = st.n_rows_padded if req == R - 1 else st.cu_rows[req + 1]
            assert first <= r0 and r0 + nr <= end and (r0 - first) % TR == 0
            assert (rs[r0:r0 + nr] == req).all()
            assert npg == (int(rl[r0:r0 + nr].max()) + 63) // 64
        assert (seen == 1).all()
        n_items = int(sch["cum_items"][-1])
        assert n_items == int(tiles[:, 3].sum())
        _check_partition(sch["unit_begin"], n_items, units)
        # (row, page) coverage: every page a valid row needs is covered exactly once
        need = np.zeros((st.n_rows_padded, (int(rl.max()) + 63) // 64 + 1), np.int64)
        for u in range(units):
            for it in range(sch["unit_begin"][u], sch["unit_begin"][u + 1]):
                t = int(np.searchsorted(sch["cum_items"], it, side="right") - 1)
                if it == sch["unit_begin"][u]:
                    assert t == sch["unit_tile"][u]
                r0, nr, req, npg = tiles[t]
                p = it - sch["cum_items"][t]
                for r in range(r0, r0 + nr):
                    if p * 64 < rl[r]:
                        need[r, p] += 1
        for r in range(st.n_rows_padded):
            npg = (int(rl[r]) + 63) // 64
            assert (need[r, :npg] == 1).all() and not need[r, npg:].any()


# ---------------------------------------------------------------------------- candidate merge

def _shard_candidates(s, n, W, k):
    """Split columns [0, n) of a row by pages over W shards (page p on shard p % W), take
    each shard's oracle top-k in its local column order, and map it back to global columns;
    returns (scores, indices) of the W*k candidates (-1 = empty)."""
    sc = np.zeros(W * k)
    ix = np.full(W * k, -1, np.int32)
    cols = np.arange(n)
    for sh in range(W):
        g = cols[(cols // 64) % W == sh]  # global columns of the shard, ascending
        if g.size == 0:
            continue
        top = oracle.topk(s[g][None, :], np.array([g.size], np.int32), k)[0]
        m = top >= 0
        sc[sh * k: sh * k + m.sum()] = s[g[top[m]]]
        ix[sh * k: sh * k + m.sum()] = g[top[m]]
    return sc, ix


@pytest.mark.parametrize("W", [2, 4, 8])
def test_topk_merge_of_shard_topks_equals_the_unsharded_topk(W):
    """Context parallelism is exact: merging the shards' local top-k candidates gives the
    unsharded top-k, order and tie-break included (ties cross shard boundaries here)."""
    rng = np.random.default_rng(W)
    k = 50
    for n in [1, 49, 50, 64, 65, 300, 1000, 2047]:
        for kind in range(3):
            if kind == 0:
                s = rng.standard_normal(n)
            elif kind == 1:
                s = rng.integers(-3, 4, n).astype(np.float64)  # heavy ties
            else:
                s = np.full(n, 2.5)  # one value
            want = oracle.topk(s[None, :], np.array([n], np.int32), k)[0]
            sc, ix = _shard_candidates(s, n, W, k)
            got = oracle.topk_merge(sc[None, :], ix[None, :], k)[0]
            assert np.array_equal(got, want), (W, n, kind)


def test_topk_merge_skips_empty_slots_and_pads():
    sc = np.array([[5.0, 9.0, 1.0, 9.0, 7.0, 0.0], [1.0, 2.0, 3.0, 4.0, 5.0, 6.0]])
    ix = np.array([[10, -1, 3, 7, -1, 2], [-1, -1, -1, -1, -1, -1]], np.int32)
    got = oracle.topk_merge(sc, ix, 4)
    # valid: (5,10) (1,3) (9,7) (0,2): by score desc -> 7, 10, 3, 2
    assert got[0].tolist() == [7, 10, 3, 2]
    assert got[1].tolist() == [-1, -1, -1, -1]
    got = oracle.topk_merge(sc[:1], ix[:1], 6)
    assert got[0].tolist() == [7, 10, 3, 2, -1, -1]
    # equal scores: the smaller index first
    got = oracle.topk_merge(np.array([[1.0, 1.0, 1.0]]), np.array([[8, 3, 5]], np.int32), 2)
    assert got[0].tolist() == [3, 5]


# ---------------------------------------------------------------------------- fused writer (R12-R15)

def test_bf16_round_matches_torch_on_fp32_values():
    """On values that are exactly fp32, rounding to bf16 is torch's own fp32 -> bf16 conversion
    (nearest, ties to even), subnormals and ties included."""
    import torch

    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]                 # finite
    ties = (rng.integers(0, 2**16, 5000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    sub = rng.integers(0, 2**23, 5000, dtype=np.uint32)             # subnormal fp32
    allb = np.concatenate([bits, ties, sub, [0, 0x80000000, 0x7F7FFFFF]]).astype(np.uint32)
    f = allb.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_bf16_round_is_a_single_rounding():
    """A double just above a bf16 tie rounds up; rounding through fp32 first would see the tie and
    go to even."""
    assert int(oracle.bf16_round(1.0 + 2.0**-8 + 2.0**-30)) == 0x3F81
    assert int(oracle.bf16_round(1.0 + 2.0**-8)) == 0x3F80             # the tie itself: even
    assert int(oracle.bf16_round(-(1.0 + 3 * 2.0**-8))) == 0xBF82
    assert int(oracle.bf16_round(2.0**-133 * 0.5)) == 0                 # half the least step: even (zero)
    assert int(oracle.bf16_round(2.0**-133 * 0.75)) == 1
    assert int(oracle.bf16_round(3.4e38)) == 0x7F80                     # past the largest finite: inf


def test_layer_norm_closed_form():
    x = np.arange(128, dtype=np.float64)
    mean, var = 63.5, (128**2 - 1) / 12.0                               # of 0..n-1
    eps = np.float32(1e-6)
    ones, zeros = np.ones(128, np.float32), np.zeros(128, np.float32)
    y = oracle.layer_norm(x, ones, zeros, eps)
    want = (x - mean) / np.sqrt(var + float(eps))
    assert np.allclose(y, want, rtol=1e-14, atol=1e-14)
    g = np.linspace(-2, 2, 128).astype(np.float32)
    b = np.linspace(1, -1, 128).astype(np.float32)
    y2 = oracle.layer_norm(x, g, b, eps)
    assert np.allclose(y2, want * g.astype(np.float64) + b.astype(np.float64), rtol=1e-13, atol=1e-13)
    # invariants for random input: zero mean, variance var / (var + eps)
    r = np.random.default_rng(2).standard_normal(128) * 3 + 5
    y3 = oracle.layer_norm(r, ones, zeros, np.float32(0.5))
    v = r.var()
    assert abs(y3.mean()) < 1e-13 and abs(y3.var() - v / (v + 0.5)) < 1e-12


@pytest.mark.parametrize("rope_dim", [64, 32, 128])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_is_complex_multiplication(rope_dim, interleaved):
    """Each rotated pair (a, b) is (a + ib) * exp(i theta); elements past rope_dim are untouched."""
    rng = np.random.default_rng(rope_dim + interleaved)
    half = rope_dim // 2
    theta = rng.uniform(-np.pi, np.pi, half)
    cs = np.concatenate([np.cos(theta), np.sin(theta)]).astype(np.float32)
    x = rng.standard_normal(128)
    y = oracle.rope(x, cs, rope_dim, interleaved)
    ia = np.arange(half) * 2 if interleaved else np.arange(half)
    ib = ia + 1 if interleaved else ia + half
    z = (x[ia] + 1j * x[ib]) * (cs[:half].astype(np.float64) + 1j * cs[half:].astype(np.float64))
    assert np.allclose(y[ia], z.real, rtol=0, atol=1e-14) and np.allclose(y[ib], z.imag, rtol=0, atol=1e-14)
    assert np.array_equal(y[rope_dim:], x[rope_dim:])
    # angle 0 is the identity; a quarter turn maps (a, b) to (-b, a)
    ident = np.concatenate([np.ones(half), np.zeros(half)]).astype(np.float32)
    assert np.array_equal(oracle.rope(x, ident, rope_dim, interleaved), x)
    quarter = np.concatenate([np.zeros(half), np.ones(half)]).astype(np.float32)
    yq = oracle.rope(x, quarter, rope_dim, interleaved)
    assert np.array_equal(yq[ia], -x[ib]) and np.array_equal(yq[ib], x[ia])


def _writer_inputs(n_tok, H, seed, rope_dim=64):
    rng = np.random.default_rng(seed)
    k = W.normal_bf16(rng, (n_tok, 128))
    q = W.normal_bf16(rng, (n_tok, H, 128))
    w = rng.standard_normal((n_tok, H)).astype(np.float32)
    max_pos = 4096
    inv = 10000.0 ** (-np.arange(rope_dim // 2) * 2.0 / max(rope_dim, 1))
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    cs = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    pos = rng.integers(0, max_pos, n_tok).astype(np.int64)
    return k, q, w, cs, pos


def test_fused_writer_without_norm_and_rope_is_the_plain_writer():
    n_tok, H = 40, 16
    k, q, w, cs, pos = _writer_inputs(n_tok, H, 1)
    slots = np.arange(n_tok, dtype=np.int64) * 3
    slots[5] = -1
    kp0, ks0 = np.zeros((4, 64, 64), np.uint8), np.zeros((4, 4, 64), np.uint8)
    kp1, ks1 = kp0.copy(), ks0.copy()
    oracle.quant_and_cache(k, slots, kp0, ks0)
    qp0, qs0 = oracle.quant_q(q)
    o = oracle.norm_rope_quant_and_cache(k, pos, None, 0, False, None, None, 0.0, slots, kp1, ks1, q, w, 0.25,
                                         all_q=True)
    assert o["err"] == 0
    assert np.array_equal(kp0, kp1) and np.array_equal(ks0, ks1)
    assert np.array_equal(o["qp"], qp0) and np.array_equal(o["qs"], qs0)
    assert np.array_equal(o["w_mqa"], (w.astype(np.float64) * 0.25).astype(np.float32))


def test_fused_writer_skips_and_flags_rows():
    """slot < 0: no key, and (unless all_q) the zero query and zero weights; a position outside the
    table: the whole row is skipped and flagged 16; a slot past the pool: the key is skipped and
    flagged 32, the query is written."""
    n_tok, H = 6, 16
    k, q, w, cs, pos = _writer_inputs(n_tok, H, 2)
    slots = np.array([0, -1, 5, 7, 64 * 4 + 3, 9], np.int64)
    pos[3] = 4096                                                       # one past the table
    g = np.ones(128, np.float32)
    kp, ks = np.zeros((4, 64, 64), np.uint8), np.zeros((4, 4, 64), np.uint8)
    o = oracle.norm_rope_quant_and_cache(k, pos, cs, 64, False, g, None, 1e-6, slots, kp, ks, q, w, 1.0)
    assert o["err"] == 16 | 32
    zq, zs = oracle.quant_q(np.zeros((1, H, 128), np.uint16))
    for t in (1, 3):
        assert np.array_equal(o["qp"][t], zq[0]) and np.array_equal(o["qs"][t], zs[0])
        assert not o["w_mqa"][t].any() and np.isnan(o["q_pre"][t]).all() and np.isnan(o["k_pre"][t]).all()
    assert np.isnan(o["k_pre"][4]).all() and not np.isnan(o["q_pre"][4]).any() and o["w_mqa"][4].any()
    assert not kp[0, 7].any()                                           # row 3's slot stayed empty
    o2 = oracle.norm_rope_quant_and_cache(k, pos, cs, 64, False, g, None, 1e-6, slots, kp.copy(), ks.copy(), q, w,
                                          1.0, all_q=True)
    assert not np.isnan(o2["q_pre"][1]).any() and o2["w_mqa"][1].any()  # all_q computes slot < 0 rows
    assert np.isnan(o2["q_pre"][3]).all()                               # but not a bad position


@pytest.mark.parametrize("interleaved", [False, True])
def test_fused_writer_dequantizes_to_the_normalized_rotated_vector(interleaved):
    """Decoding what the fused writer stored gives the normalized, rotated vector within the MXFP4
    error bound (half a grid step of each block's scale, plus bf16 rounding)."""
    n_tok, H = 24, 16
    k, q, w, cs, pos = _writer_inputs(n_tok, H, 3)
    rng = np.random.default_rng(4)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    b = rng.uniform(-0.2, 0.2, 128).astype(np.float32)
    slots = np.arange(n_tok, dtype=np.int64)
    kp, ks = np.zeros((1, 64, 64), np.uint8), np.zeros((1, 4, 64), np.uint8)
    o = oracle.norm_rope_quant_and_cache(k, pos, cs, 64, interleaved, g, b, 1e-6, slots, kp, ks, q, w, 1.0)
    kf = k.astype(np.uint32) << 16
    for t in range(n_tok):
        x = kf[t].view(np.float32).astype(np.float64)
        xn = (x - x.mean()) / np.sqrt(x.var() + np.float64(np.float32(1e-6))) * g + b
        c, sn = cs[pos[t], :32].astype(np.float64), cs[pos[t], 32:].astype(np.float64)
        ia = np.arange(32) * 2 if interleaved else np.arange(32)
        ib = ia + 1 if interleaved else ia + 32
        z = (xn[ia] + 1j * xn[ib]) * (c + 1j * sn)
        want = xn.copy()
        want[ia], want[ib] = z.real, z.imag
        assert np.allclose(o["k_pre"][t], want, rtol=1e-9, atol=1e-9)
        got = oracle.dequant_key(kp, ks, 0, t)
        for blk in range(4):
            sl = slice(32 * blk, 32 * blk + 32)
            step = 2.0 ** (int(ks[0, blk, oracle.scale_slot(t)]) - 127)   # E2M1 grid step at 1 is 0.5 * scale
            bound = np.maximum(0.25 * step, 1.0 * step) + np.abs(want[sl]) * 2.0**-8
            assert (np.abs(got[sl] - np.clip(want[sl], -6 * step, 6 * step)) <= bound).all()


# ---------------------------------------------------------------------------- MXFP8 comparator (R16)

def test_e4m3_values_match_torch():
    import torch

    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(got[~np.isnan(got)], want[~np.isnan(want)])


def test_mx8_element_rounding_matches_torch_at_unit_scale():
    """Every bf16 value of magnitude in [2^-12, 448], in blocks anchored by 256 (scale 2^0): the
    codes are torch's fp32 -> float8_e4m3fn conversion (nearest, ties to even)."""
    import torch

    mags = []
    for e in range(-12, 9):
        for m in range(128):
            v = (1 + m / 128) * 2.0**e
            if v <= 448:
                mags.append(v)
    vals = np.array(mags + [-v for v in mags], np.float32)
    vals = np.concatenate([vals, np.zeros((-len(vals)) % 31, np.float32)])
    blocks = vals.reshape(-1, 31)
    blocks = np.concatenate([np.full((blocks.shape[0], 1), 256.0, np.float32), blocks], axis=1)
    bits = W.bf16_bits(blocks)
    assert np.array_equal(W.bf16_to_f32(bits), blocks)  # all exact in bf16
    scale, codes = oracle.mx8_encode_blocks(bits)
    assert (scale == 127).all()
    want = torch.from_numpy(blocks.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want)


def test_mx8_scale_rule_and_saturation():
    def enc(vals):
        b = W.bf16_bits(np.asarray(vals, np.float32).reshape(1, 32))
        return oracle.mx8_encode_blocks(b)

    s, c = enc([1.0] + [0.0] * 31)           # amax 1: 2^(0 - 8), 1.0 -> 256 = 0x78
    assert s[0] == 127 - 8 and c[0, 0] == 0x78
    s, c = enc([448.0, 500.0] + [0.0] * 30)  # amax 500: scale 2^0, 500 saturates to 448
    assert s[0] == 127 and c[0, 0] == 0x7E and c[0, 1] == 0x7E
    s, c = enc([0.0] * 32)
    assert s[0] == 0 and not c.any()
    s, c = enc([-3.0e-39] + [0.0] * 31)      # the smallest scales clamp at 2^-127
    assert s[0] == 0


def test_fp8_scores_equal_fp4_scores_on_fp4_representable_data():
    """E4M3 holds every E2M1 value, so data already on an MXFP4 grid passes through MXFP8
    unchanged: the FP8 score equals the FP4 score exactly (an FP4-pinned quantity)."""
    case = W.decode_case([300, 130], heads=16, topk=32, seed=12)
    kp4 = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks4 = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp4, ks4)
    qp4, qs4 = oracle.quant_q(case.q)
    # bf16 images of the FP4-quantized vectors (exact: FP4 values times powers of two)
    keys_q = np.zeros_like(case.keys)
    for t, s in enumerate(case.slots):
        keys_q[t] = W.bf16_bits(oracle.dequant_key(kp4, ks4, s // 64, s % 64).astype(np.float32))
    q_q = np.zeros_like(case.q)
    for r in range(case.rows):
        for h in range(case.heads):
            q_q[r, h] = W.bf16_bits(oracle.dequant_q(qp4, qs4, r, h).astype(np.float32))
    kp8 = np.zeros((case.n_pages, 64, 128), np.uint8)
    ks8 = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant8_and_cache(keys_q, case.slots, kp8, ks8)
    qp8, qs8 = oracle.quant8_q(q_q)
    rs, rl = oracle.decode_geometry(case.ctx)
    s4, _ = oracle.score(qp4, qs4, case.w, rs, rl, kp4, ks4, case.block_table)
    s8, _ = oracle.score8(qp8, qs8, case.w, rs, rl, kp8, ks8, case.block_table)
    assert np.array_equal(np.isnan(s4), np.isnan(s8))
    assert np.array_equal(s4[~np.isnan(s4)], s8[~np.isnan(s8)])
    for t, s in enumerate(case.slots[:50]):  # and the keys decode to the same values
        assert np.array_equal(oracle.dequant8_key(kp8, ks8, s // 64, s % 64),
                              oracle.dequant_key(kp4, ks4, s // 64, s % 64))


# ---------------------------------------------------------------------------- planted mistakes

def test_parity_checks_catch_planted_mistakes():
    """The checks the GPU parity tests apply reject outputs with a planted mistake (planted in
    the oracle's own outputs, on the CPU): a row scored one key too far or one key short (an
    off-by-one context), a padding row that reads keys, and top-k lists with a shifted index,
    an index past the row or a duplicate. The unmodified outputs pass."""
    from helpers import check_logits, check_topk

    def rejects(f):
        try:
            f()
        except AssertionError:
            return True
        return False

    # decode: an off-by-one context either way
    case = W.decode_config("decode_tiny")
    qp, qs = oracle.quant_q(case.q)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    rs, rl = oracle.decode_geometry(case.ctx)
    ld = case.block_table.shape[1] * 64
    s, _ = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table, ld=ld)
    assert not rejects(lambda: check_logits(s, s, rl))
    rl_long, rl_short = rl.copy(), rl - 1
    rl_long[0] += 1  # (row 0 has room in its last page and in the logits row)
    assert rl[0] % 64 != 0 and rl[0] < ld
    s_long, _ = oracle.score(qp, qs, case.w, rs, rl_long, kp, ks, case.block_table, ld=ld)
    s_short, _ = oracle.score(qp, qs, case.w, rs, rl_short, kp, ks, case.block_table, ld=ld)
    assert rejects(lambda: check_logits(s_long, s, rl))
    assert rejects(lambda: check_logits(s_short, s, rl))
    # top-k: a shifted index, an index past the row, a duplicate
    k = case.topk
    top = oracle.topk(s, rl, k)
    assert not rejects(lambda: check_topk(top, top, s, rl, k))
    r = int(np.argmax(rl))
    n = min(k, int(rl[r]))
    order = np.argsort(-s[r, :int(rl[r])], kind="stable")
    out_of_set = int(order[-1])  # the row's smallest score, far from the k-th
    bad = top.copy()
    bad[r, 0] = out_of_set
    assert rejects(lambda: check_topk(bad, top, s, rl, k))
    bad = top.copy()
    bad[r, n - 1] = int(rl[r])
    assert rejects(lambda: check_topk(bad, top, s, rl, k))
    bad = top.copy()
    bad[r, 1] = bad[r, 0]
    assert rejects(lambda: check_topk(bad, top, s, rl, k))
    # prefill: a padding row scored as if it saw keys
    pc = W.prefill_config("prefill_tiny")
    kp = np.zeros((pc.n_pages, 64, 64), np.uint8)
    ks = np.zeros((pc.n_pages, 4, 64), np.uint8)
    st = pc.steps[0]
    k_, sl = W.step_keys(pc, st)
    oracle.quant_and_cache(k_, sl, kp, ks)
    rs, rl = oracle.prefill_geometry(st.cu_rows, st.start_pos, st.n_rows_padded)
    qp, qs = oracle.quant_q(st.q)
    bt = W.step_block_table(pc, st)
    ld = int(pc.lengths.max())
    s, _ = oracle.score(qp, qs, st.w, rs, rl, kp, ks, bt, ld=ld)
    assert not rejects(lambda: check_logits(s, s, rl))
    pad = int(st.n_rows)  # the first padding row
    assert rl[pad] == 0
    rl_read = rl.copy()
    rl_read[pad] = 5
    s_read, _ = oracle.score(qp, qs, st.w, rs, rl_read, kp, ks, bt, ld=ld)
    assert rejects(lambda: check_logits(s_read, s, rl))
