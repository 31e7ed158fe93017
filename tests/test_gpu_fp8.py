"""GPU parity of the FP8 comparator (MXFP8 writer and decode scorer) against the CPU oracle:
bytes exact, logits within 1e-3 relative, top-k sets equal up to near-ties of the k-th score."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import bf16_tensor, check_logits, check_topk, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ifp4():
    import sparse_attention_indexer_fp4_amd as m

    return m


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b.astype(np.int64) >> 7) & 0xFF) != 0xFF]


def test_fp8_quantizer_exhaustive_bf16(ifp4):
    """Every finite bf16 value alone in its block, in a random block mix, and under fixed block
    scales 2^e (e = -12..12, anchored by 2^(e+8)), through the query arm."""
    bits = _all_finite_bf16()
    rng = np.random.default_rng(12)
    vecs = []
    alone = np.zeros((bits.size, 32), np.uint16)
    alone[:, 0] = bits
    vecs.append(alone.reshape(-1, 128))
    vecs.append(rng.permutation(np.concatenate([bits, bits[: (-bits.size) % 128]])).reshape(-1, 128))
    for e in range(-12, 13):
        v = W.bf16_to_f32(bits).astype(np.float64)
        sel = bits[np.abs(v) < 2.0 ** (e + 8)]
        blk = np.zeros((sel.size, 32), np.uint16)
        blk[:, 0] = W.bf16_bits(np.full(sel.size, 2.0 ** (e + 8), np.float32))
        blk[:, 1] = sel
        blk = np.concatenate([blk, np.zeros(((-sel.size) % 4, 32), np.uint16)])
        vecs.append(blk.reshape(-1, 128))
    q = np.concatenate(vecs)[:, None, :]
    print(f"fp8 exhaustive quantizer rows={q.shape[0]}", flush=True)
    qp = torch.empty((q.shape[0], 1, 128), dtype=torch.uint8, device=dev())
    qs = torch.empty((q.shape[0], 1, 4), dtype=torch.uint8, device=dev())
    kp = torch.zeros((1, 64, 128), dtype=torch.uint8, device=dev())
    ks = torch.zeros((1, 4, 64), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp8_quant_and_cache(None, None, kp, ks, bf16_tensor(q), qp, qs)
    oqp, oqs = oracle.quant8_q(q)
    assert np.array_equal(qs.cpu().numpy(), oqs)
    assert np.array_equal(qp.cpu().numpy(), oqp)


def test_fp8_writer_places_keys_and_skips_slots(ifp4):
    keys = W.normal_bf16(np.random.default_rng(6), (200, 128))
    slots = np.random.default_rng(7).permutation(4 * 64)[:200].astype(np.int64)  # some past the 3-page pool
    slots[::13] = -1
    kp = torch.full((3, 64, 128), 0xA5, dtype=torch.uint8, device=dev())
    ks = torch.full((3, 4, 64), 0x5A, dtype=torch.uint8, device=dev())
    ifp4.indexer_fp8_quant_and_cache(bf16_tensor(keys), to_dev(slots), kp, ks)
    okp = np.full((3, 64, 128), 0xA5, np.uint8)
    oks = np.full((3, 4, 64), 0x5A, np.uint8)
    ok = slots < 3 * 64
    oracle.quant8_and_cache(keys[ok], slots[ok], okp, oks)
    assert np.array_equal(kp.cpu().numpy(), okp)
    assert np.array_equal(ks.cpu().numpy(), oks)


def gpu_decode8(ifp4, case, units=512, fused=False):
    B, H, nn, rows = case.batch, case.heads, case.next_n, case.rows
    ld = case.block_table.shape[1] * 64
    kp = torch.zeros((case.n_pages, 64, 128), dtype=torch.uint8, device=dev())
    ks = torch.zeros((case.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    qp = torch.empty((rows, H, 128), dtype=torch.uint8, device=dev())
    qs = torch.empty((rows, H, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp8_quant_and_cache(bf16_tensor(case.keys), to_dev(case.slots), kp, ks, bf16_tensor(case.q), qp, qs)
    sched = torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, nn, units), dtype=torch.uint8, device=dev())
    row_len = torch.empty(rows, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_decode_schedule(to_dev(case.ctx), nn, units, sched, row_len)
    logits = torch.full((rows, ld), float("nan"), dtype=torch.float32, device=dev())
    hist = ifp4.row_histogram(rows, dev()) if fused else None
    ifp4.indexer_fp8_score_decode(qp, qs, to_dev(case.w), kp, ks, to_dev(case.block_table), nn, sched, units,
                                  row_len, logits, hist)
    top = torch.full((rows, case.topk), -7, dtype=torch.int32, device=dev())
    ws = torch.zeros(max(ifp4.indexer_topk_workspace_bytes(rows, ld, case.topk), 1), dtype=torch.uint8, device=dev())
    ifp4.indexer_topk(logits, row_len, ld, case.topk, top, ws, hist)
    torch.cuda.synchronize()
    return dict(kp=kp.cpu().numpy(), ks=ks.cpu().numpy(), qp=qp.cpu().numpy(), qs=qs.cpu().numpy(),
                logits=logits.cpu().numpy(), top=top.cpu().numpy(), row_len=row_len.cpu().numpy(),
                err=ifp4.sched_error(sched), hist_left=None if hist is None else int(hist.abs().sum().item()))


def oracle_decode8(case):
    ld = case.block_table.shape[1] * 64
    kp = np.zeros((case.n_pages, 64, 128), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant8_and_cache(case.keys, case.slots, kp, ks)
    qp, qs = oracle.quant8_q(case.q)
    rs, rl = oracle.decode_geometry(case.ctx, case.next_n)
    s, _ = oracle.score8(qp, qs, case.w, rs, rl, kp, ks, case.block_table, ld=ld)
    return dict(kp=kp, ks=ks, qp=qp, qs=qs, s=s, row_len=rl, top=oracle.topk(s, rl, case.topk))


FP8_CASES = [
    dict(name="tiny", ctx=[300, 512], heads=16, topk=64),
    dict(name="h64_ragged", ctx=[1000, 64, 1, 129, 4095], heads=64, topk=256),
    dict(name="h128", ctx=[513, 2000], heads=128, topk=300),
    dict(name="next_n2", ctx=[300, 191], heads=64, topk=64, next_n=2),
    dict(name="long", ctx=[20000, 3000], heads=64, topk=2048),
]


@pytest.mark.parametrize("p", FP8_CASES, ids=lambda p: p["name"])
@pytest.mark.parametrize("units", [512, 5])
def test_fp8_decode_scores_and_topk(ifp4, p, units):
    p = dict(p)
    name = p.pop("name")
    case = W.decode_case(name=name, seed=3, **p)
    print(f"fp8 decode {name} units={units}", flush=True)
    g = gpu_decode8(ifp4, case, units=units, fused=units == 5)
    o = oracle_decode8(case)
    assert g["err"] == 0
    for key in ("kp", "ks", "qp", "qs"):
        assert np.array_equal(g[key], o[key]), key
    check_logits(g["logits"], o["s"], o["row_len"])
    check_topk(g["top"], o["top"], o["s"], o["row_len"], case.topk)
    if g["hist_left"] is not None:
        assert g["hist_left"] == 0


def test_fp8_full_size_decode(ifp4):
    case = W.decode_config("decode_b8_128k")
    print("fp8 full-size decode_b8_128k", flush=True)
    g = gpu_decode8(ifp4, case, fused=True)
    o = oracle_decode8(case)
    assert g["err"] == 0
    assert np.array_equal(g["kp"], o["kp"]) and np.array_equal(g["ks"], o["ks"])
    check_logits(g["logits"], o["s"], o["row_len"])
    check_topk(g["top"], o["top"], o["s"], o["row_len"], case.topk)
