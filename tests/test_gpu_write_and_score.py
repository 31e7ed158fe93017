"""indexer_fp4_write_and_score_decode against the two calls it replaces: the fused writer
(indexer_fp4_norm_rope_quant_and_cache) on the step's keys and query rows, then
indexer_fp4_score_decode on its outputs. Both run on the GPU from the same seeded inputs;
the cache planes must match byte for byte, and the logits, the scorer's histogram and the
device flags bit for bit (the two paths quantize with the same code and score the same
bytes). The writer and the scorer are each checked against the oracle in their own tests.

Cases: sequences that share units (a unit's later sequences take the per-wave query path),
new keys on a wave's first pages (written before the first loads) and on later ones, 16 to
128 heads, rotary and LayerNorm variants, a padding row (slot -1) and a rotary position
outside the table (flagged; the row gets the zero query)."""
import numpy as np
import pytest
import torch

import workloads as W
from helpers import bf16_tensor, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ifp4():
    import sparse_attention_indexer_fp4_amd as m

    return m


def _step(ctx, heads, seed, rope_dim, pad=(), bad_pos=()):
    c = W.decode_case(ctx, heads, 64, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    B = c.batch
    last = c.ctx.astype(np.int64) - 1
    k_new = W.bf16_bits(rng.standard_normal((B, W.HEAD_DIM)).astype(np.float32) + np.float32(0.5))
    slots = c.block_table[np.arange(B), last // W.PAGE].astype(np.int64) * W.PAGE + last % W.PAGE
    max_pos = int(c.ctx.max()) + 1
    positions = last.copy()
    for b in pad:
        slots[b] = -1
    for b in bad_pos:
        positions[b] = max_pos + 3
    gamma = rng.uniform(0.5, 1.5, W.HEAD_DIM).astype(np.float32)
    beta = rng.uniform(-0.2, 0.2, W.HEAD_DIM).astype(np.float32)
    return dict(c=c, k=k_new, slots=slots, positions=positions, cos_sin=W.rope_table(max_pos, rope_dim),
                rope_dim=rope_dim, gamma=gamma, beta=beta)


def _run(ifp4, s, units, fused, interleaved, norm):
    c = s["c"]
    B, H = c.batch, c.heads
    kp = torch.zeros((c.n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((c.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(c.keys), to_dev(c.slots), kp, ks)
    sched = torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, 1, units), dtype=torch.uint8, device=dev())
    row_len = torch.empty(B, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_decode_schedule(to_dev(c.ctx), 1, units, sched, row_len)
    ld = c.block_table.shape[1] * W.PAGE
    logits = torch.full((B, ld), float("nan"), dtype=torch.float32, device=dev())
    hist = ifp4.row_histogram(B, dev())
    kw = dict(positions=to_dev(s["positions"]), cos_sin=to_dev(s["cos_sin"]), rope_dim=s["rope_dim"],
              interleaved=interleaved, k_norm_weight=to_dev(s["gamma"]) if norm else None,
              k_norm_bias=to_dev(s["beta"]) if norm else None, eps=1e-6)
    q, w, bt = bf16_tensor(c.q), to_dev(c.w), to_dev(c.block_table)
    werr = torch.zeros(1, dtype=torch.int32, device=dev())
    if fused:
        ifp4.indexer_fp4_write_and_score_decode(bf16_tensor(s["k"]), to_dev(s["slots"]), kp, ks, q, w, bt, sched,
                                                units, row_len, logits, weight_scale=0.125, row_hist=hist, **kw)
    else:
        qp = torch.empty((B, H, 64), dtype=torch.uint8, device=dev())
        qs = torch.empty((B, H, 4), dtype=torch.uint8, device=dev())
        wm = torch.empty((B, H), dtype=torch.float32, device=dev())
        ifp4.indexer_fp4_norm_rope_quant_and_cache(bf16_tensor(s["k"]), to_dev(s["slots"]), kp, ks, q=q,
                                                   q_packed=qp, q_scale=qs, weights=w, weight_scale=0.125,
                                                   weights_mqa=wm, err=werr, **kw)
        ifp4.indexer_fp4_score_decode(qp, qs, wm, kp, ks, bt, 1, sched, units, row_len, logits, hist)
    torch.cuda.synchronize()
    return dict(kp=kp.cpu().numpy(), ks=ks.cpu().numpy(), logits=logits.cpu().numpy(), hist=hist.cpu().numpy(),
                err=ifp4.sched_error(sched) | int(werr.item()))


CASES = [  # ctx, heads, units, rope_dim, interleaved, norm, pad, bad_pos
    ([300, 512], 16, 5, 64, False, True, (), ()),
    ([300, 512], 16, 512, 64, True, True, (), ()),
    ([1, 64, 65, 130, 4000, 777], 64, 7, 64, False, True, (), ()),
    ([1, 64, 65, 130, 4000, 777], 64, 64, 0, False, False, (), ()),
    ([1, 64, 65, 130, 4000, 777], 64, 512, 128, True, False, (), ()),
    ([5000, 3000, 129], 128, 16, 64, False, True, (), ()),
    ([2048, 700, 65], 32, 8, 64, False, True, (1,), (2,)),
    ([20000, 9000], 64, 3, 64, False, True, (), ()),  # waves of more than 64 pages
]


@pytest.mark.parametrize("ctx,heads,units,rope_dim,interleaved,norm,pad,bad_pos", CASES)
def test_write_and_score_equals_writer_then_scorer(ifp4, ctx, heads, units, rope_dim, interleaved, norm, pad,
                                                   bad_pos):
    print(f"write_and_score ctx={ctx} heads={heads} units={units} rope={rope_dim}", flush=True)
    s = _step(ctx, heads, seed=len(ctx) * 7 + heads + units, rope_dim=rope_dim, pad=pad, bad_pos=bad_pos)
    a = _run(ifp4, s, units, False, interleaved, norm)
    b = _run(ifp4, s, units, True, interleaved, norm)
    assert np.array_equal(a["kp"], b["kp"]) and np.array_equal(a["ks"], b["ks"])
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    assert np.array_equal(a["hist"], b["hist"])
    assert a["err"] == b["err"]
    if bad_pos:
        assert b["err"] & ifp4.DEV_BAD_POSITION
