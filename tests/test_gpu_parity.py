"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs. Bit-exact for bytes, schedules and indices; 1e-3 relative for logits; top-k sets
equal up to near-ties of the k-th score (see helpers.py)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import (bf16_tensor, check_logits, check_topk, dev, gpu_decode, gpu_prefill_step, oracle_decode,
                     oracle_prefill_step, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ifp4():
    import sparse_attention_indexer_fp4_amd as m

    return m


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------- cache write

@pytest.mark.parametrize("sens", [False, True])
def test_cache_and_query_bytes_exact(ifp4, sens):
    case = W.decode_config("decode_tiny", swizzle_sensitive=sens)
    _say(f"decode_tiny swizzle_sensitive={sens}")
    g = gpu_decode(case, run_topk=False)
    o = oracle_decode(case, scores=False)
    assert np.array_equal(g["kp"].cpu().numpy(), o["kp"])
    assert np.array_equal(g["ks"].cpu().numpy(), o["ks"])
    assert np.array_equal(g["qp"].cpu().numpy(), o["qp"])
    assert np.array_equal(g["qs"].cpu().numpy(), o["qs"])


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b.astype(np.int64) >> 7) & 0xFF) != 0xFF]


def test_quantizer_exhaustive_bf16(ifp4):
    """Every finite bf16 value alone in its block, in a random block mix, and under fixed
    block scales 2^e (e = -10..10 and the extremes -127..-121, 100, 125, where bf16
    subnormals can reach nonzero codes and the scale leaves the normal floats), through the
    query arm: bytes equal the oracle's."""
    bits = _all_finite_bf16()
    rng = np.random.default_rng(11)
    vecs = []
    alone = np.zeros((bits.size, 32), np.uint16)
    alone[:, 0] = bits
    vecs.append(alone.reshape(-1, 128))
    vecs.append(rng.permutation(np.concatenate([bits, bits[: (-bits.size) % 128]])).reshape(-1, 128))
    for e in list(range(-10, 11)) + [-127, -126, -125, -124, -123, -122, -121, 100, 125]:
        v = W.bf16_to_f32(bits).astype(np.float64)
        sel = bits[np.abs(v) < 2.0 ** (e + 2)]
        blk = np.zeros((sel.size, 32), np.uint16)
        blk[:, 0] = W.bf16_bits(np.full(sel.size, 2.0 ** (e + 2), np.float32))
        blk[:, 1] = sel
        blk = np.concatenate([blk, np.zeros(((-sel.size) % 4, 32), np.uint16)])
        vecs.append(blk.reshape(-1, 128))
    q = np.concatenate(vecs)[:, None, :]  # [rows, 1 head, 128]
    _say(f"exhaustive quantizer rows={q.shape[0]}")
    qp = torch.empty((q.shape[0], 1, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((q.shape[0], 1, 4), dtype=torch.uint8, device=dev())
    kp = torch.zeros((1, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((1, 4, 64), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(None, None, kp, ks, bf16_tensor(q), qp, qs)
    oqp, oqs = oracle.quant_q(q)
    assert np.array_equal(qs.cpu().numpy(), oqs)
    assert np.array_equal(qp.cpu().numpy(), oqp)


def test_writer_skips_negative_and_out_of_pool_slots(ifp4):
    keys = W.normal_bf16(np.random.default_rng(5), (6, 128))
    slots = np.array([-1, 3, 64 * 2, -5, 64 * 2 + 70, 127], np.int64)  # page 2 does not exist
    kp = torch.full((2, 64, 64), 0xA5, dtype=torch.uint8, device=dev())
    ks = torch.full((2, 4, 64), 0x5A, dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(keys), to_dev(slots), kp, ks)
    okp = np.full((2, 64, 64), 0xA5, np.uint8)
    oks = np.full((2, 4, 64), 0x5A, np.uint8)
    ok = slots < 128
    oracle.quant_and_cache(keys[ok], slots[ok], okp, oks)
    assert np.array_equal(kp.cpu().numpy(), okp)
    assert np.array_equal(ks.cpu().numpy(), oks)


# ---------------------------------------------------------------------------- schedules

@pytest.mark.parametrize("ctx,units,next_n", [([300, 512], 512, 1), ([4096], 512, 1), ([0, 65, 64, 1, 0], 7, 1),
                                              ([131072] * 8, 512, 1), ([5] * 3000, 512, 1), ([200, 77], 64, 3)])
def test_decode_schedule_exact(ifp4, ctx, units, next_n):
    ctx = np.array(ctx, np.int32)
    sched = torch.full((ifp4.indexer_fp4_decode_sched_bytes(len(ctx), next_n, units),), 0xEE, dtype=torch.uint8,
                       device=dev())
    row_len = torch.empty(len(ctx) * next_n, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_decode_schedule(to_dev(ctx), next_n, units, sched, row_len)
    got = ifp4.read_decode_schedule(sched, len(ctx), units)
    want = oracle.decode_schedule(ctx, units)
    for key in ("cum_pages", "unit_begin", "unit_seq"):
        assert np.array_equal(got[key], want[key]), key
    # the library's private per-unit fields (the first item's page in its sequence and the
    # items left in that sequence) must agree with the oracle's prefix sums
    cum, ub, us = want["cum_pages"], want["unit_begin"], want["unit_seq"]
    for u in range(units):
        b = us[u]
        if b < len(ctx):
            assert got["unit_page"][u] == ub[u] - cum[b] and got["unit_run"][u] == cum[b + 1] - ub[u], u
        else:
            assert got["unit_page"][u] == 0 and got["unit_run"][u] == 0, u
    assert got["header"][1] == 0
    _, rl = oracle.decode_geometry(ctx, next_n)
    assert np.array_equal(row_len.cpu().numpy(), rl)


@pytest.mark.parametrize("which", ["prefill_tiny", "prefill_4req"])
@pytest.mark.parametrize("units", [13, 256, 4096])
def test_prefill_schedule_exact(ifp4, which, units):
    case = W.prefill_config(which, heads=16)
    TR = ifp4.TILE_ROWS
    for st in case.steps:
        R, NP = len(st.req_ids), st.n_rows_padded
        bt = W.step_block_table(case, st)
        bt_ld = bt.shape[1]
        sched = torch.full((ifp4.indexer_fp4_prefill_sched_bytes(R, NP, units, bt_ld),), 0xEE, dtype=torch.uint8,
                           device=dev())
        row_len = torch.empty(NP, dtype=torch.int32, device=dev())
        ifp4.indexer_fp4_prefill_schedule(to_dev(st.cu_rows), to_dev(st.start_pos), NP, units, to_dev(bt),
                                          case.n_pages, sched, row_len)
        got = ifp4.read_prefill_schedule(sched, R, NP, units, bt_ld)
        want = oracle.prefill_schedule(st.cu_rows, st.start_pos, NP, TR, units)
        assert got["header"][1] == 0
        for key in ("tiles", "cum_items", "unit_begin", "unit_tile"):
            assert np.array_equal(got[key], want[key]), key
        rs, rl = oracle.prefill_geometry(st.cu_rows, st.start_pos, NP)
        assert np.array_equal(row_len.cpu().numpy(), rl)
        # the library's own words, against the oracle's tiles, lengths and the block table:
        # valid rows, first position, first item of every tile; every item's physical page;
        # every unit's start record
        cum = want["cum_items"]
        for t, (r0, nr, req, pages) in enumerate(want["tiles"]):
            tw = got["tile_words"][t]
            nv = int((rl[r0:r0 + nr] > 0).sum())
            assert tw[2] == nv and tw[6] == cum[t], t
            if nv:
                assert tw[3] + 1 == rl[r0]
            for p in range(pages):
                assert got["item_phys"][cum[t] + p] == bt[req, p], (t, p)
        ub = want["unit_begin"]
        for u in range(units):
            rec = got["unit_records"][u]
            assert rec[0] == ub[u] and rec[1] == ub[u + 1] and rec[2] == want["unit_tile"][u], u
            if ub[u] < ub[u + 1]:
                assert np.array_equal(rec[4:12], got["tile_words"][rec[2]]), u
            for j in range(4):
                i = ub[u] + j
                assert rec[12 + j] == (got["item_phys"][i] if i < ub[u + 1] else -1), (u, j)


# ---------------------------------------------------------------------------- decode scores

DECODE_CASES = [
    dict(name="decode_tiny"),
    dict(name="decode_tiny", swizzle_sensitive=True),
    dict(name="h64_ragged", ctx=[1000, 64, 1, 129, 4095], heads=64, topk=256),
    dict(name="h32_small_k", ctx=[700, 70], heads=32, topk=16),
    dict(name="h128", ctx=[513, 2000], heads=128, topk=300),
    dict(name="next_n2", ctx=[300, 191], heads=64, topk=64, next_n=2),
    dict(name="next_n4", ctx=[520, 4], heads=16, topk=32, next_n=4),
]


@pytest.mark.parametrize("p", DECODE_CASES, ids=lambda p: p["name"] + ("_sens" if p.get("swizzle_sensitive") else ""))
@pytest.mark.parametrize("units", [512, 5])
def test_decode_scores_and_topk(ifp4, p, units):
    p = dict(p)
    name = p.pop("name")
    case = W.decode_config(name, **p) if name in W.DECODE_CONFIGS else W.decode_case(name=name, **p)
    _say(f"decode {name} ctx={list(case.ctx)} H={case.heads} next_n={case.next_n} units={units}")
    g = gpu_decode(case, units=units)
    o = oracle_decode(case)
    assert g["err"] == 0
    assert np.array_equal(g["row_len"].cpu().numpy(), o["row_len"])
    check_logits(g["logits"].cpu().numpy(), o["s"], o["row_len"])
    check_topk(g["top"].cpu().numpy(), o["top"], o["s"], o["row_len"], case.topk)


def test_topk_is_exact_on_the_same_logits(ifp4):
    """Selection itself is exact: on the GPU's own fp32 logits the GPU top-k equals the oracle's
    full sort (ties to the lower column), returned in ascending column order."""
    case = W.decode_case([3000, 4096, 2049, 100], heads=16, topk=2048, seed=9)
    g = gpu_decode(case)
    lg = g["logits"].cpu().numpy().astype(np.float64)
    rl = g["row_len"].cpu().numpy()
    want = oracle.topk(lg, rl, case.topk)
    top = g["top"].cpu().numpy()
    for r in range(case.rows):
        n = min(case.topk, int(rl[r]))
        assert list(top[r][:n]) == sorted(want[r][:n].tolist())
        assert (top[r][n:] == -1).all()


def test_topk_ties_and_signed_zero(ifp4):
    rng = np.random.default_rng(3)
    rows, n = 6, 5000
    lg = rng.integers(-3, 4, size=(rows, n)).astype(np.float32)  # heavy ties
    lg[1] = 0.0
    lg[1, ::2] = -0.0                                          # -0 ranks with +0
    lg[2] = rng.standard_normal(n).astype(np.float32)
    lg[3, :] = 7.0
    lg[4] = -np.abs(rng.standard_normal(n)).astype(np.float32)  # all negative
    rl = np.array([n, n, 2500, 4097, n, 10], np.int32)
    k = 2048
    t = to_dev(lg)
    top = torch.full((rows, k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk(t, to_dev(rl), n, k, top)
    want = oracle.topk(lg.astype(np.float64), rl, k)
    got = top.cpu().numpy()
    for r in range(rows):
        m = min(k, int(rl[r]))
        assert list(got[r][:m]) == sorted(want[r][:m].tolist()), r
        assert (got[r][m:] == -1).all()


@pytest.mark.parametrize("max_len", [16384, 6144])
@pytest.mark.parametrize("tile", [1, 150])
@pytest.mark.parametrize("k", [1, 16, 64, 2048])
def test_topk_short_rows_exact(ifp4, k, tile, max_len):
    """Short-row selection on ragged lengths around the per-wave column ranges (64-column
    steps, ranges clamped to the row, some empty) equals the oracle's full sort exactly; 14
    rows run on 512-thread workgroups, 2100 rows on 256-thread ones. Rows of at most 6144
    keys (max_len 6144) take the register-resident kernel, longer ones the LDS one."""
    rng = np.random.default_rng(11 + k)
    base = np.array([65, 70, 100, 129, 191, 255, 256, 257, 1000, 2049, 2050, 4097, 8191, 16384], np.int32)
    if max_len == 6144:
        base = np.array([65, 70, 100, 129, 191, 255, 256, 257, 1000, 1535, 1537, 2049, 4097, 6144], np.int32)
    lens = np.tile(base, tile)
    n = int(lens.max())
    lg = (rng.standard_normal((len(lens), n)) * 40 + 100).astype(np.float32)
    lg[3, :50] = lg[3, 60]  # a tie block inside the first range
    t = to_dev(lg)
    top = torch.full((len(lens), k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk(t, to_dev(lens), n, k, top)
    want = oracle.topk(lg.astype(np.float64), lens, k)
    got = top.cpu().numpy()
    for r in range(len(lens)):
        m = min(k, int(lens[r]))
        assert list(got[r][:m]) == sorted(want[r][:m].tolist()), (r, int(lens[r]))
        assert (got[r][m:] == -1).all()


def test_device_side_errors_flag_and_skip(ifp4):
    case = W.decode_config("decode_tiny")
    bt = case.block_table.copy()
    bt[0, 1] = 10_000   # outside the pool
    bt[1, 2] = -3
    case.block_table = bt
    g = gpu_decode(case, run_topk=False)
    assert g["err"] & ifp4.DEV_BAD_PAGE
    lg = g["logits"].cpu().numpy()
    assert np.isnan(lg[0, 64:128]).all() and np.isnan(lg[1, 128:192]).all()  # skipped, not faulted
    o = oracle_decode(W.decode_config("decode_tiny"))
    good = np.ones_like(lg, bool)
    good[0, 64:128] = False
    good[1, 128:192] = False
    for r in range(2):
        L = int(o["row_len"][r])
        m = good[r, :L]
        assert np.allclose(lg[r, :L][m], o["s"][r, :L][m], rtol=1e-3, atol=0)


def test_stale_or_zeroed_schedule_is_flagged(ifp4):
    """A schedule buffer that was never built (zero-filled) or was built for other sizes is
    not trusted: the scorers read only its header, flag INDEXER_FP4_DEV_BAD_SCHEDULE and
    score nothing (the logits keep their sentinel)."""
    case = W.decode_config("decode_tiny")
    g = gpu_decode(case, run_topk=False)
    units = g["units"]
    B = case.batch
    for fill in (0, 0xEE):
        sched = torch.full((ifp4.indexer_fp4_decode_sched_bytes(B, 1, units),), fill, dtype=torch.uint8, device=dev())
        sched.view(torch.int32)[1] = 0
        lg = torch.full_like(g["logits"], float("nan"))
        ifp4.indexer_fp4_score_decode(g["qp"], g["qs"], to_dev(case.w), g["kp"], g["ks"], to_dev(case.block_table), 1,
                                      sched, units, g["row_len"], lg)
        torch.cuda.synchronize()
        assert ifp4.sched_error(sched) == ifp4.DEV_BAD_SCHEDULE, fill
        assert torch.isnan(lg).all()
    # a schedule built for fewer units than the call names: header mismatch, nothing scored
    small = torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, 1, units), dtype=torch.uint8, device=dev())
    rl = torch.empty(B, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_decode_schedule(to_dev(case.ctx), 1, units // 2, small, rl)
    lg = torch.full_like(g["logits"], float("nan"))
    ifp4.indexer_fp4_score_decode(g["qp"], g["qs"], to_dev(case.w), g["kp"], g["ks"], to_dev(case.block_table), 1,
                                  small, units, rl, lg)
    torch.cuda.synchronize()
    assert ifp4.sched_error(small) == ifp4.DEV_BAD_SCHEDULE
    assert torch.isnan(lg).all()
    # prefill: a zeroed buffer
    pc = W.prefill_config("prefill_tiny", heads=16)
    st = pc.steps[0]
    NP, R, H = st.n_rows_padded, len(st.req_ids), pc.heads
    qp = torch.zeros((NP, H, 64), dtype=torch.uint8, device=dev())
    qs = torch.zeros((NP, H, 4), dtype=torch.uint8, device=dev())
    kp = torch.zeros((pc.n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((pc.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    bt = W.step_block_table(pc, st)
    pu = ifp4.PREFILL_UNITS
    psched = torch.zeros(ifp4.indexer_fp4_prefill_sched_bytes(R, NP, pu, bt.shape[1]), dtype=torch.uint8,
                         device=dev())
    plg = torch.full((NP, bt.shape[1] * 64), float("nan"), dtype=torch.float32, device=dev())
    ifp4.indexer_fp4_score_prefill(qp, qs, to_dev(st.w), kp, ks, R, bt.shape[1], psched, pu, NP, plg)
    torch.cuda.synchronize()
    assert ifp4.sched_error(psched) == ifp4.DEV_BAD_SCHEDULE
    assert torch.isnan(plg).all()


def test_prefill_device_side_errors_flag_and_skip(ifp4):
    """Prefill with block-table entries outside the pool: the schedule flags the step, the
    scorer skips exactly the pages those entries name (their columns keep the sentinel),
    nothing faults, and every other valid logit matches the oracle."""
    case = W.prefill_config("prefill_tiny", heads=16)
    kp = torch.zeros((case.n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((case.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    okp = np.zeros((case.n_pages, 64, 64), np.uint8)
    oks = np.zeros((case.n_pages, 4, 64), np.uint8)
    st0, st = case.steps[0], case.steps[1]  # the second step holds requests 0 and 2
    assert list(st.req_ids) == [0, 2]
    g0 = gpu_prefill_step(case, st0, kp, ks, run_topk=False)
    assert g0["err"] == 0
    oracle_prefill_step(case, st0, okp, oks, scores=False)
    o = oracle_prefill_step(case, st, okp, oks)
    # the step's own keys, then a schedule and the scorer over a corrupted table
    NP, R, H = st.n_rows_padded, len(st.req_ids), case.heads
    keys, slots = W.step_keys(case, st)
    qp = torch.empty((NP, H, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((NP, H, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(keys), to_dev(slots), kp, ks, bf16_tensor(st.q), qp, qs)
    bt = W.step_block_table(case, st).copy()
    bt[0, 1] = 10_000  # request 0, page 1: outside the pool
    bt[1, 0] = -3      # request 2, page 0
    units = ifp4.PREFILL_UNITS
    sched = torch.empty(ifp4.indexer_fp4_prefill_sched_bytes(R, NP, units, bt.shape[1]), dtype=torch.uint8,
                        device=dev())
    row_len = torch.empty(NP, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_prefill_schedule(to_dev(st.cu_rows), to_dev(st.start_pos), NP, units, to_dev(bt), case.n_pages,
                                      sched, row_len)
    ld = bt.shape[1] * 64
    logits = torch.full((NP, ld), float("nan"), dtype=torch.float32, device=dev())
    ifp4.indexer_fp4_score_prefill(qp, qs, to_dev(st.w), kp, ks, R, bt.shape[1], sched, units, NP, logits)
    torch.cuda.synchronize()
    assert ifp4.sched_error(sched) & ifp4.DEV_BAD_PAGE
    lg = logits.cpu().numpy().astype(np.float64)
    rl = o["row_len"]
    skipped = np.zeros_like(lg, bool)
    skipped[st.cu_rows[0]:st.cu_rows[1], 64:128] = True  # request 0's rows past 64 keys
    skipped[st.cu_rows[1]:st.cu_rows[2], 0:64] = True    # all of request 2's rows
    for r in range(NP):
        L = int(rl[r])
        if L == 0:
            continue
        sk = skipped[r, :L]
        assert np.isnan(lg[r, :L][sk]).all(), f"row {r}: a skipped page was written"
        ok = ~sk
        assert np.isfinite(lg[r, :L][ok]).all(), f"row {r}: a good page was not written"
        assert np.allclose(lg[r, :L][ok], o["s"][r, :L][ok], rtol=1e-3, atol=0), f"row {r}"
        assert np.isnan(lg[r, L:]).all()
    assert (rl[st.cu_rows[0]:st.cu_rows[1]] > 64).any()  # the case does reach page 1 of request 0


# ---------------------------------------------------------------------------- prefill scores

@pytest.mark.parametrize("which,heads,units", [("prefill_tiny", 16, 512), ("prefill_tiny", 64, 7),
                                               ("prefill_tiny", 64, 4096), ("prefill_tiny", 32, 13),
                                               ("prefill_tiny", 128, 512),
                                               ("prefill_tiny_mbt", 16, 13), ("prefill_tiny_mbt", 64, 512),
                                               ("prefill_4req", 64, 512),  # full size, as benched
                                               ("prefill_4req_mbt512", 64, 512)])
def test_prefill_scores_and_topk(ifp4, which, heads, units):
    case = W.prefill_config(which, heads=heads)
    kp = torch.zeros((case.n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((case.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    okp = np.zeros((case.n_pages, 64, 64), np.uint8)
    oks = np.zeros((case.n_pages, 4, 64), np.uint8)
    for si, st in enumerate(case.steps):
        _say(f"prefill {which} H={heads} units={units} step {si} rows={st.n_rows}/{st.n_rows_padded}")
        g = gpu_prefill_step(case, st, kp, ks, units=units)
        o = oracle_prefill_step(case, st, okp, oks)
        assert g["err"] == 0
        assert np.array_equal(kp.cpu().numpy(), okp) and np.array_equal(ks.cpu().numpy(), oks)
        assert np.array_equal(g["qp"].cpu().numpy(), o["qp"])
        assert np.array_equal(g["row_len"].cpu().numpy(), o["row_len"])
        check_logits(g["logits"].cpu().numpy(), o["s"], o["row_len"])
        check_topk(g["top"].cpu().numpy(), o["top"], o["s"], o["row_len"], case.topk)
        pad = np.arange(st.n_rows_padded) >= st.n_rows
        assert (g["top"].cpu().numpy()[pad] == -1).all()  # padding rows select nothing


# ---------------------------------------------------------------------------- full sizes

@pytest.mark.parametrize("name", ["decode_b1_4k", "decode_b8_128k", "decode_b16_128k", "decode_b8_256k"])
def test_full_size_decode(ifp4, name):
    case = W.decode_config(name)
    _say(f"full-size {name}: B={case.batch} ctx={int(case.ctx[0])}")
    g = gpu_decode(case)
    assert g["err"] == 0
    o = oracle_decode(case)
    assert np.array_equal(g["kp"].cpu().numpy(), o["kp"])
    assert np.array_equal(g["ks"].cpu().numpy(), o["ks"])
    check_logits(g["logits"].cpu().numpy(), o["s"], o["row_len"])
    check_topk(g["top"].cpu().numpy(), o["top"], o["s"], o["row_len"], case.topk)


def _order_hist(lg, n):
    """Per-row counts of the top 12 order-key bits of lg[r, :n[r]], in the device layout (bin b
    at word (b % 64) * 64 + b // 64)."""
    u = lg.view(np.uint32).copy()
    u[u == 0x80000000] = 0
    key = np.where(u >> 31 == 1, ~u, u | np.uint32(0x80000000))
    out = np.zeros((lg.shape[0], 4096), np.int64)
    b = np.arange(4096)
    for r in range(lg.shape[0]):
        h = np.bincount((key[r, : int(n[r])] >> 20).astype(np.int64), minlength=4096)
        out[r, (b % 64) * 64 + b // 64] = h
    return out


def test_topk_with_a_histogram_of_other_logits(ifp4):
    """A row histogram built from other logits (the interface allows it: a meaningless but
    in-bounds, -1-padded selection): histograms of far larger values (no key lies at or above
    the chosen bin: nothing is selected), of far smaller ones (every key lies above it: the
    lowest-column k are kept) and of a shuffled row's half (mixed counts). Every selection is
    valid (ascending distinct columns of the row, then -1), and the workspace and histograms
    serve a correct call afterwards."""
    n, k, rows = 131072, 2048, 4
    rng = np.random.default_rng(31)
    lg = rng.standard_normal((rows, n)).astype(np.float32)
    rl = np.array([n, n - 1, 70000, n], np.int32)
    other = np.stack([lg[0] + 1e4, lg[1] - 1e4, rng.permutation(lg[2])[:n] * 0.5, lg[3][::-1] * 3.0])
    hist = torch.from_numpy(_order_hist(other, rl).astype(np.uint32).view(np.int32)).to(dev())
    ws = torch.zeros(ifp4.indexer_topk_workspace_bytes(rows, n, k), dtype=torch.uint8, device=dev())
    top = torch.full((rows, k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk(to_dev(lg), to_dev(rl), n, k, top, ws, hist)
    torch.cuda.synchronize()
    got = top.cpu().numpy()
    for r in range(rows):
        sel = got[r][got[r] >= 0]
        m = len(sel)
        assert (got[r][m:] == -1).all(), f"row {r}: -1 only after the selection"
        assert (np.diff(sel) > 0).all() and (sel < rl[r]).all(), f"row {r}: ascending columns of the row"
    assert (got[0] == -1).all()                            # no key at or above the bin: nothing kept
    assert list(got[1]) == list(range(k))                  # every key above the bin: lowest columns
    assert int(torch.count_nonzero(hist).item()) == 0      # the histograms are left zeroed
    _topk_exact(ifp4, lg, rl, k, n, ws)                    # the same workspace, no histogram: exact


FUSED_CASES = [
    dict(name="long_ragged", ctx=[20000, 9000, 131, 2625], heads=64, topk=2048),
    dict(name="long_next_n2", ctx=[17000, 30000], heads=32, topk=2048, next_n=2),
    dict(name="long_next_n4", ctx=[40000, 16385], heads=16, topk=512, next_n=4),
    dict(name="short_rows", ctx=[300, 191], heads=64, topk=64, next_n=2),
    dict(name="h128_mixed", ctx=[64, 1, 20100, 640, 70000], heads=128, topk=2048),
]


@pytest.mark.parametrize("p", FUSED_CASES, ids=lambda p: p["name"])
@pytest.mark.parametrize("units", [512, 5, 37])
def test_fused_histogram(ifp4, p, units):
    """The scorer's histogram is exactly that of the logits it wrote (every row, including rows
    of sequences that start inside a unit), the top-k that takes it selects exactly what the
    top-k that builds its own selects, and it is left zero-filled."""
    p = dict(p)
    name = p.pop("name")
    case = W.decode_case(name=name, seed=units, **p)
    _say(f"fused {name} ctx={list(case.ctx)} H={case.heads} next_n={case.next_n} units={units}")
    a = gpu_decode(case, units=units)
    b = gpu_decode(case, units=units, fused=True)
    assert a["err"] == 0 and b["err"] == 0
    la, lb = a["logits"].cpu().numpy(), b["logits"].cpu().numpy()
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    rl = b["row_len"].cpu().numpy()
    assert np.array_equal(b["hist"].cpu().numpy().astype(np.int64), _order_hist(lb, rl))
    assert np.array_equal(a["top"].cpu().numpy(), b["top"].cpu().numpy())
    assert not b["row_hist"].any().item()


def test_fused_histogram_full_size(ifp4):
    case = W.decode_config("decode_b8_128k")
    _say(f"fused full-size: B={case.batch} ctx={int(case.ctx[0])}")
    a = gpu_decode(case)
    b = gpu_decode(case, fused=True)
    assert a["err"] == 0 and b["err"] == 0
    lb = b["logits"].cpu().numpy()
    assert np.array_equal(a["logits"].cpu().numpy().view(np.uint32), lb.view(np.uint32))
    assert np.array_equal(b["hist"].cpu().numpy().astype(np.int64), _order_hist(lb, b["row_len"].cpu().numpy()))
    assert np.array_equal(a["top"].cpu().numpy(), b["top"].cpu().numpy())
    assert not b["row_hist"].any().item()


# ---------------------------------------------------------------------------- long-row top-k

def _topk_exact(ifp4, lg, rl, k, max_len, ws=None, pad=0):
    rows, n = lg.shape
    # pad > 0 gives the rows a stride that is not a multiple of 4 floats
    t = to_dev(np.pad(lg, ((0, 0), (0, pad)))) if pad else to_dev(lg)
    top = torch.full((rows, k), -7, dtype=torch.int32, device=dev())
    if ws is None:
        ws = torch.zeros(max(ifp4.indexer_topk_workspace_bytes(rows, max_len, k), 16), dtype=torch.uint8,
                         device=dev())
    ifp4.indexer_topk(t, to_dev(rl), max_len, k, top, ws)
    got = top.cpu().numpy()
    want = oracle.topk(lg.astype(np.float64), np.minimum(rl, max_len).astype(np.int32), k)
    for r in range(rows):
        m = min(k, int(min(rl[r], max_len)))
        assert list(got[r][:m]) == sorted(want[r][:m].tolist()), f"row {r} len {rl[r]}"
        assert (got[r][m:] == -1).all(), f"row {r}: tail"
    return ws


@pytest.mark.parametrize("n,k", [(131072, 2048), (262144, 2048), (20000, 64), (50000, 10000)])
def test_topk_long_rows_exact(ifp4, n, k):
    rng = np.random.default_rng(n + k)
    rows = 8
    _say(f"long top-k n={n} k={k}")
    lg = rng.standard_normal((rows, n)).astype(np.float32)
    lg[1] = 3.0                                              # all ties
    lg[2] = rng.integers(-2, 3, n).astype(np.float32)        # heavy ties
    lg[3, ::3] = -0.0
    lg[3, 1::3] = 0.0                                        # signed zeros rank equal
    lg[4] = -np.abs(lg[4])                                   # all negative
    lg[5] = np.abs(lg[5]) * 1e-30                            # tiny magnitudes
    rl = np.array([n, n, n - 5, n - 4096 - 1, k, k + 1, 17, n + 100], np.int32)  # last row clamps to max_len
    ws = _topk_exact(ifp4, lg, rl, k, n)
    # the workspace is left ready for the next call: reuse it on different rows
    _topk_exact(ifp4, -lg[::-1].copy(), rl[::-1].copy(), k, n, ws)


def test_topk_long_rows_second_level_paths(ifp4):
    """Rows built so that the k-th key's digit-1 bin holds (a) a few thousand keys clustered in a
    few digit-2 bins, (b) exact ties at the threshold spread over every chunk, (c) far more
    candidates than one round of the emit kernel's reads covers (further rounds from the
    workspace); rows of odd stride."""
    n, k = 131072, 2048
    rng = np.random.default_rng(11)
    lg = rng.random((4, n)).astype(np.float32)
    idx = rng.permutation(n)[:6072]
    lg[0, idx] = 7.5 + 1e-4 * rng.random(6072)                          # (a) dense cluster at the top
    lg[1] = np.round(rng.standard_normal(n) * 64.0) / 64.0               # (b) ties everywhere
    lg[2, idx] = 7.5                                                     # (c) 6072 equal keys on top
    lg[2, rng.permutation(n)[:20000]] = 7.5
    lg[3] = rng.standard_normal(n)
    rl = np.array([n, n - 1, n, n - 333], np.int32)
    ws = _topk_exact(ifp4, lg, rl, k, n)
    _topk_exact(ifp4, lg[::-1].copy(), rl, k, n, ws)
    _topk_exact(ifp4, lg, rl, k, n, pad=1)


def test_topk_long_row_at_the_length_limit(ifp4):
    n, k = 1 << 20, 2048
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((2, n)).astype(np.float32)
    lg[1] = np.repeat(rng.standard_normal(n // 1024).astype(np.float32), 1024)  # blocks of ties
    _topk_exact(ifp4, lg, np.array([n, n - 1], np.int32), k, n)


def test_topk_workspace_shared_across_shapes(ifp4):
    """One workspace for calls of different shapes, never cleared: a call with more rows finds
    an earlier call's candidate lists where it builds its own digit-1 histograms, and every
    selection must still be exact. Fewer rows first, then more rows at other lengths, then
    fewer again."""
    rng = np.random.default_rng(5)
    calls = [(3, 40000, 2048), (16, 131072, 2048), (2, 262144, 512), (9, 20000, 64)]
    size = max(ifp4.indexer_topk_workspace_bytes(r, n, k) for r, n, k in calls)
    ws = torch.zeros(size, dtype=torch.uint8, device=dev())
    for rows, n, k in calls:
        _say(f"shared workspace: {rows} rows x {n} keys, k={k}")
        lg = rng.standard_normal((rows, n)).astype(np.float32)
        lg[0] = np.round(lg[0] * 8.0) / 8.0  # ties at the threshold
        rl = np.array([n - (i * 997) % (n // 2) for i in range(rows)], np.int32)
        _topk_exact(ifp4, lg, rl, k, n, ws)


@pytest.mark.parametrize("n,k", [(6144, 2048), (4213, 2048), (16000, 2048)])
def test_topk_crowded_threshold_bin(ifp4, n, k):
    """Rows whose k-th key sits in a crowded bin of the first histogram: thousands of keys in a
    tiny band (further 10-bit levels, then ranking), the band made of a few exact values
    (levels down to one value), exact ties straddling the cut across waves, and the k-th key
    equal to the row's minimum."""
    rng = np.random.default_rng(n + 7)
    rows = 6
    lg = (rng.standard_normal((rows, n)) * 30.0).astype(np.float32)
    band = rng.permutation(n)[:3000]
    lg[0, band] = 7.5 + 1e-4 * rng.random(3000)
    lg[1, band] = 7.5 + 1e-6 * rng.integers(0, 5, 3000)
    lg[2, :] = -1.0
    lg[2, rng.permutation(n)[:k // 2]] = 2.0   # the cut falls inside the ties at -1
    lg[3] = np.abs(lg[3]) + 1.0
    lg[3, rng.permutation(n)[:n - k + 10]] = 1.0  # the k-th key is the row minimum, tied
    lg[4, band] = np.float32(2.0 ** -126)       # a band near the smallest normal
    lg[5] = np.where(rng.random(n) < 0.5, 0.0, -0.0)
    rl = np.array([n, n - 1, n, n - 63, n - 64 * 7, n], np.int32)
    _topk_exact(ifp4, lg, rl, k, n)
    _topk_exact(ifp4, lg[::-1].copy(), rl, k, n)


@pytest.mark.parametrize("n,k", [(3000, 64), (16000, 2048), (131072, 2048)])
def test_topk_rows_sharing_leading_bits(ifp4, n, k):
    """Regression: rows whose keys all share their top bits (positive logits in a narrow band,
    as the scorer produces) once met a miscompiled select in the mask of the shared bits and
    selected nothing."""
    rng = np.random.default_rng(n)
    lg = np.stack([5.0 + 45.0 * rng.random(n), 1000.0 + rng.random(n), np.full(n, 7.5) + 1e-3 * rng.random(n),
                   -(5.0 + 45.0 * rng.random(n))]).astype(np.float32)
    rl = np.array([n, n - 1, n // 2 + k, n], np.int32)
    _topk_exact(ifp4, lg, rl, k, n)


# ---------------------------------------------------------------------------- graph replay

@pytest.mark.parametrize("fused", [False, True])
def test_graph_replay_bitwise_stable(ifp4, fused):
    """One decode step (schedule, key/query write, scorer, top-k) captured once at fixed
    addresses and replayed under four context-length vectors written in place: every replay
    equals an eager run of the same inputs bit for bit (the schedule is what lets a captured
    graph follow changing lengths), including the capture vector replayed again after the
    others. Eager work and synchronizations run between replays."""
    B, H, k, max_ctx, units = 4, 64, 2048, 20000, 64
    rng = np.random.default_rng(21)
    pages = -(-max_ctx // 64)
    n_pages = B * pages + 8
    bt_np = rng.permutation(n_pages)[:B * pages].astype(np.int32).reshape(B, pages)
    ld = pages * 64
    kp = torch.zeros((n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((n_pages, 4, 64), dtype=torch.uint8, device=dev())
    all_slots = (bt_np.astype(np.int64)[:, :, None] * 64 + np.arange(64)).reshape(B, -1)[:, :max_ctx]
    keys = torch.from_numpy(W.bf16_bits(rng.standard_normal((B * max_ctx, 128)).astype(np.float32)).view(np.int16))
    ifp4.indexer_fp4_quant_and_cache(keys.view(torch.bfloat16).to(dev()), to_dev(all_slots.reshape(-1).copy()), kp, ks)
    bt = to_dev(bt_np)
    ctx = torch.zeros(B, dtype=torch.int32, device=dev())
    slots = torch.zeros(B, dtype=torch.int64, device=dev())
    knew = torch.from_numpy(W.bf16_bits(rng.standard_normal((B, 128)).astype(np.float32)).view(np.int16)).view(
        torch.bfloat16).to(dev())
    q = torch.from_numpy(W.bf16_bits(rng.standard_normal((B, H, 128)).astype(np.float32)).view(np.int16)).view(
        torch.bfloat16).to(dev())
    w = to_dev(rng.random((B, H), dtype=np.float32))

    def buffers():
        return dict(sched=torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, 1, units), dtype=torch.uint8, device=dev()),
                    row_len=torch.empty(B, dtype=torch.int32, device=dev()),
                    qp=torch.empty((B, H, 64), dtype=torch.uint8, device=dev()),
                    qs=torch.empty((B, H, 4), dtype=torch.uint8, device=dev()),
                    logits=torch.full((B, ld), float("nan"), dtype=torch.float32, device=dev()),
                    top=torch.full((B, k), -7, dtype=torch.int32, device=dev()),
                    ws=torch.zeros(max(ifp4.indexer_topk_workspace_bytes(B, ld, k), 16), dtype=torch.uint8,
                                   device=dev()),
                    hist=ifp4.row_histogram(B, dev()) if fused else None)

    def step(o):
        ifp4.indexer_fp4_decode_schedule(ctx, 1, units, o["sched"], o["row_len"])
        ifp4.indexer_fp4_quant_and_cache(knew, slots, kp, ks, q, o["qp"], o["qs"])
        ifp4.indexer_fp4_score_decode(o["qp"], o["qs"], w, kp, ks, bt, 1, o["sched"], units, o["row_len"],
                                      o["logits"], o["hist"])
        ifp4.indexer_topk(o["logits"], o["row_len"], ld, k, o["top"], o["ws"], o["hist"])

    def set_ctx(c):
        ctx.copy_(to_dev(np.asarray(c, np.int32)))
        slots.copy_(to_dev(all_slots[np.arange(B), np.asarray(c) - 1].copy()))

    g_out, e_out = buffers(), buffers()
    set_ctx([4096, 100, 17000, 2049])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(g_out)  # warm-up on the capture stream
        with torch.cuda.graph(graph, stream=side):
            step(g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the capture batch, three others, then the capture batch again after them
    for c in ([4096, 100, 17000, 2049], [20000, 64, 1, 9000], [3000, 19999, 2048, 2047], [65, 12345, 20000, 300],
              [4096, 100, 17000, 2049]):
        _say(f"graph replay ctx={c}")
        set_ctx(c)
        e_out["logits"].fill_(float("nan"))
        g_out["logits"].fill_(float("nan"))
        step(e_out)  # eager, same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ifp4.sched_error(g_out["sched"]) == 0
        gl, el = g_out["logits"].cpu().numpy(), e_out["logits"].cpu().numpy()
        for r in range(B):
            n = int(c[r])
            assert np.array_equal(gl[r, :n].view(np.uint32), el[r, :n].view(np.uint32)), f"row {r}: logits differ"
            assert np.isnan(gl[r, n:]).all()
        assert np.array_equal(g_out["top"].cpu().numpy(), e_out["top"].cpu().numpy())
        assert np.array_equal(g_out["row_len"].cpu().numpy(), np.asarray(c, np.int32))
        if fused:
            assert not g_out["hist"].any().item() and not e_out["hist"].any().item()


def test_prefill_graph_replay_bitwise_stable(ifp4):
    """One prefill step (schedule, scorer, top-k) captured once at fixed addresses and replayed
    under four request layouts (row splits and chunk start positions written in place; the
    padded row count is fixed), then the first layout again: every replay equals an eager run
    of the same inputs bit for bit, padding rows select nothing, and the first layout's logits
    and top-k match the oracle. Eager work and synchronizations run between replays."""
    R, NP, H, k, units, lmax = 3, 48, 64, 512, 256, 4160
    rng = np.random.default_rng(33)
    pages = lmax // 64
    n_pages = R * pages + 5
    bt_np = rng.permutation(n_pages)[:R * pages].astype(np.int32).reshape(R, pages)
    ld = pages * 64
    slots = (bt_np.astype(np.int64)[:, :, None] * 64 + np.arange(64)).reshape(-1)
    keys = W.bf16_bits(rng.standard_normal((R * lmax, 128)).astype(np.float32))
    qb = W.bf16_bits(rng.standard_normal((NP, H, 128)).astype(np.float32))
    w_np = rng.random((NP, H), dtype=np.float32)
    kp = torch.zeros((n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((n_pages, 4, 64), dtype=torch.uint8, device=dev())
    qp = torch.empty((NP, H, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((NP, H, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(keys), to_dev(slots), kp, ks, bf16_tensor(qb), qp, qs)
    bt, w = to_dev(bt_np), to_dev(w_np)
    cu = torch.zeros(R + 1, dtype=torch.int32, device=dev())
    sp = torch.zeros(R, dtype=torch.int32, device=dev())

    def buffers():
        return dict(sched=torch.empty(ifp4.indexer_fp4_prefill_sched_bytes(R, NP, units, pages), dtype=torch.uint8,
                                      device=dev()),
                    row_len=torch.empty(NP, dtype=torch.int32, device=dev()),
                    logits=torch.full((NP, ld), float("nan"), dtype=torch.float32, device=dev()),
                    top=torch.full((NP, k), -7, dtype=torch.int32, device=dev()),
                    ws=torch.zeros(max(ifp4.indexer_topk_workspace_bytes(NP, ld, k), 16), dtype=torch.uint8,
                                   device=dev()))

    def step(o):
        ifp4.indexer_fp4_prefill_schedule(cu, sp, NP, units, bt, n_pages, o["sched"], o["row_len"])
        ifp4.indexer_fp4_score_prefill(qp, qs, w, kp, ks, R, pages, o["sched"], units, NP, o["logits"])
        ifp4.indexer_topk(o["logits"], o["row_len"], ld, k, o["top"], o["ws"])

    layouts = [([0, 16, 30, 45], [0, 500, 1000]), ([0, 40, 41, 48], [100, 0, 2000]), ([0, 1, 2, 3], [3000, 5, 64]),
               ([0, 8, 20, 44], [63, 4095, 4000]), ([0, 16, 30, 45], [0, 500, 1000])]

    def set_layout(lay):
        cu.copy_(to_dev(np.asarray(lay[0], np.int32)))
        sp.copy_(to_dev(np.asarray(lay[1], np.int32)))

    g_out, e_out = buffers(), buffers()
    set_layout(layouts[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(g_out)  # warm-up on the capture stream
        with torch.cuda.graph(graph, stream=side):
            step(g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, lay in enumerate(layouts):
        _say(f"prefill graph replay layout={lay}")
        set_layout(lay)
        e_out["logits"].fill_(float("nan"))
        g_out["logits"].fill_(float("nan"))
        step(e_out)  # eager, same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ifp4.sched_error(g_out["sched"]) == 0 and ifp4.sched_error(e_out["sched"]) == 0
        _, rl = oracle.prefill_geometry(np.asarray(lay[0], np.int32), np.asarray(lay[1], np.int32), NP)
        assert np.array_equal(g_out["row_len"].cpu().numpy(), rl)
        gl, el = g_out["logits"].cpu().numpy(), e_out["logits"].cpu().numpy()
        for r in range(NP):
            n = int(rl[r])
            assert np.array_equal(gl[r, :n].view(np.uint32), el[r, :n].view(np.uint32)), f"row {r}: logits differ"
            assert np.isnan(gl[r, n:]).all(), f"row {r}: written past its length {n}"
        gtop = g_out["top"].cpu().numpy()
        assert np.array_equal(gtop, e_out["top"].cpu().numpy())
        assert (gtop[lay[0][-1]:] == -1).all()  # padding rows select nothing
        if i == 0:
            okp = np.zeros((n_pages, 64, 64), np.uint8)
            oks = np.zeros((n_pages, 4, 64), np.uint8)
            oracle.quant_and_cache(keys, slots, okp, oks)
            oqp, oqs = oracle.quant_q(qb)
            rs, rl0 = oracle.prefill_geometry(np.asarray(lay[0], np.int32), np.asarray(lay[1], np.int32), NP)
            s0, _ = oracle.score(oqp, oqs, w_np, rs, rl0, okp, oks, bt_np, ld=ld)
            check_logits(gl, s0, rl0)
            check_topk(gtop, oracle.topk(s0, rl0, k), s0, rl0, k)


# ---------------------------------------------------------------------------- context parallelism

@pytest.mark.parametrize("rows,n_cand,k", [(8, 8192, 2048), (4, 16384, 2048), (6, 300, 64), (3, 100, 4096)])
def test_topk_merge_matches_oracle(ifp4, rows, n_cand, k):
    rng = np.random.default_rng(n_cand + k)
    sc = rng.standard_normal((rows, n_cand)).astype(np.float32)
    sc[1] = np.round(sc[1] * 4) / 4  # heavy ties
    sc[2] = 1.5                      # one value
    ix = rng.permutation(2 * rows * n_cand)[: rows * n_cand].reshape(rows, n_cand).astype(np.int32)
    ix[0, ::3] = -1                  # empty slots
    if rows > 3:
        ix[3, :] = -1                # no candidate at all
    _say(f"topk_merge rows={rows} n_cand={n_cand} k={k}")
    top = torch.full((rows, k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk_merge(to_dev(sc), to_dev(ix), k, top)
    got = top.cpu().numpy()
    want = oracle.topk_merge(sc.astype(np.float64), ix, k)
    for r in range(rows):
        m = int((want[r] >= 0).sum())
        assert list(got[r][:m]) == sorted(want[r][:m].tolist()), f"row {r}"
        assert (got[r][m:] == -1).all()


@pytest.mark.parametrize("mode", ["repeated", "wide"])
def test_topk_merge_index_ranges(ifp4, mode):
    """Indices that repeat (the ordering falls back from the LDS bitmap to the sort) and
    indices spread over [0, 2^31 - 1) (wider than the bitmap) merge as the oracle does."""
    rows, n_cand, k = 5, 3000, 256
    rng = np.random.default_rng(7 if mode == "repeated" else 8)
    sc = rng.standard_normal((rows, n_cand)).astype(np.float32)
    sc[1] = np.round(sc[1] * 4) / 4  # heavy ties
    hi = n_cand // 2 if mode == "repeated" else 2**31 - 1
    ix = rng.integers(0, hi, (rows, n_cand)).astype(np.int32)
    ix[2, ::5] = -1
    _say(f"topk_merge index mode={mode}")
    top = torch.full((rows, k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk_merge(to_dev(sc), to_dev(ix), k, top)
    got = top.cpu().numpy()
    want = oracle.topk_merge(sc.astype(np.float64), ix, k)
    for r in range(rows):
        m = int((want[r] >= 0).sum())
        assert list(got[r][:m]) == sorted(want[r][:m].tolist()), f"row {r}"
        assert (got[r][m:] == -1).all()


def test_context_parallel_decode_on_one_gpu(ifp4):
    """Context parallelism on one GPU's share: W = 4 page-interleaved shards of every
    sequence are scored by the scorer through their own block tables, each takes a local
    top-k, the candidates are exchanged (stubbed as a device gather) and merged: the result
    equals the unsharded decode top-k exactly."""
    Wn, k, units = 4, 2048, 512
    case = W.decode_case([20000, 9000, 131, 2049 + 64 * 9], heads=64, topk=k, seed=31)
    B = case.batch
    g = gpu_decode(case)  # unsharded: cache write, schedule, score, top-k
    kp, ks, qp, qs = g["kp"], g["ks"], g["qp"], g["qs"]
    wv = to_dev(case.w)
    bt = case.block_table
    pages = -(-case.ctx // 64)
    lw = -(-bt.shape[1] // Wn)  # local table width
    cand_s = torch.full((B, Wn * k), 0.0, dtype=torch.float32, device=dev())
    cand_i = torch.full((B, Wn * k), -1, dtype=torch.int32, device=dev())
    for s in range(Wn):
        lbt = np.full((B, lw), -1, np.int32)
        lctx = np.zeros(B, np.int32)
        for b in range(B):
            own = np.arange(s, pages[b], Wn)  # this shard's global pages of sequence b
            lbt[b, : own.size] = bt[b, own]
            lctx[b] = sum(min(64, int(case.ctx[b]) - 64 * int(p)) for p in own)
        _say(f"shard {s}: local ctx {lctx.tolist()}")
        lld = lw * 64
        sched = torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, 1, units), dtype=torch.uint8, device=dev())
        rl = torch.empty(B, dtype=torch.int32, device=dev())
        ifp4.indexer_fp4_decode_schedule(to_dev(lctx), 1, units, sched, rl)
        lg = torch.full((B, lld), float("nan"), dtype=torch.float32, device=dev())
        ifp4.indexer_fp4_score_decode(qp, qs, wv, kp, ks, to_dev(lbt), 1, sched, units, rl, lg)
        ltop = torch.full((B, k), -1, dtype=torch.int32, device=dev())
        ws = torch.zeros(max(ifp4.indexer_topk_workspace_bytes(B, lld, k), 16), dtype=torch.uint8, device=dev())
        ifp4.indexer_topk(lg, rl, lld, k, ltop, ws)
        assert ifp4.sched_error(sched) == 0
        # the exchange: scores and global columns of the local candidates
        li = ltop.long()
        ok = li >= 0
        sc = torch.gather(lg, 1, li.clamp(min=0))
        gi = ((li // 64) * Wn + s) * 64 + li % 64
        cand_s[:, s * k:(s + 1) * k] = torch.where(ok, sc, torch.zeros_like(sc))
        cand_i[:, s * k:(s + 1) * k] = torch.where(ok, gi, torch.full_like(gi, -1)).int()
    merged = torch.full((B, k), -7, dtype=torch.int32, device=dev())
    ifp4.indexer_topk_merge(cand_s, cand_i, k, merged)
    m = merged.cpu().numpy()
    assert np.array_equal(m, g["top"].cpu().numpy())
    # and against the oracle's full sort of its own fp64 scores, up to near-ties of the k-th
    o = oracle_decode(case)
    check_topk(m, o["top"], o["s"], o["row_len"], k)
