"""GPU parity of the fused writer (key LayerNorm, RoPE on keys and query heads, MXFP4 cache
write, query quantization, weights_mqa) against the CPU oracle.

The kernel normalizes and rotates in fp32, the oracle in fp64; both round once to bf16 and
quantize that. The bf16 value, and with it the stored codes, can differ only where the fp64
value lies within the fp32 error of a bf16 rounding boundary. So: every vector with no element
that close must match the oracle byte for byte; a vector with such elements must equal the
oracle's quantization of one of the bf16 vectors the boundary allows (each close element
rounded down or up); weights_mqa and the error word are exact, and so are the skipped rows."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ifp4():
    import sparse_attention_indexer_fp4_amd as m

    return m


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def run_gpu(ifp4, c, interleaved, norm, all_q, with_q=True, kv_fill=0):
    n_tok, H = c.q.shape[0], c.q.shape[1]
    kp = torch.full((c.n_pages, 64, 64), kv_fill, dtype=torch.uint8, device=dev())
    ks = torch.full((c.n_pages, 4, 64), kv_fill, dtype=torch.uint8, device=dev())
    qp = torch.full((n_tok, H, 64), 0xAB, dtype=torch.uint8, device=dev())
    qs = torch.full((n_tok, H, 4), 0xAB, dtype=torch.uint8, device=dev())
    wm = torch.full((n_tok, H), float("nan"), dtype=torch.float32, device=dev())
    err = torch.zeros(1, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_norm_rope_quant_and_cache(
        _bf16_dev(c.k), to_dev(c.slots), kp, ks, positions=to_dev(c.positions), cos_sin=to_dev(c.cos_sin),
        rope_dim=c.rope_dim, interleaved=interleaved, k_norm_weight=to_dev(c.gamma) if norm else None,
        k_norm_bias=to_dev(c.beta) if norm else None, eps=1e-6, q=_bf16_dev(c.q) if with_q else None,
        q_packed=qp, q_scale=qs, weights=to_dev(c.w), weight_scale=0.125, weights_mqa=wm, all_q=all_q, err=err)
    torch.cuda.synchronize()
    return dict(kp=kp.cpu().numpy(), ks=ks.cpu().numpy(), qp=qp.cpu().numpy(), qs=qs.cpu().numpy(),
                wm=wm.cpu().numpy(), err=int(err.item()))


def run_oracle(c, interleaved, norm, all_q, kv_fill=0):
    kp = np.full((c.n_pages, 64, 64), kv_fill, np.uint8)
    ks = np.full((c.n_pages, 4, 64), kv_fill, np.uint8)
    o = oracle.norm_rope_quant_and_cache(c.k, c.positions, c.cos_sin if c.rope_dim else None, c.rope_dim,
                                         interleaved, c.gamma if norm else None, c.beta if norm else None, 1e-6,
                                         c.slots, kp, ks, c.q, c.w, 0.125, all_q=all_q)
    o.update(kp=kp, ks=ks)
    return o


def _close_to_boundary(pre):
    """Elements whose fp64 value is within the fp32 error (2^-19 relative + 2^-21) of a bf16
    rounding boundary: the two ends of that interval round differently."""
    d = np.abs(pre) * 2.0**-19 + 2.0**-21
    return oracle.bf16_round(pre - d) != oracle.bf16_round(pre + d)


def _alternatives(pre, close):
    idx = np.nonzero(close)[0]
    base = oracle.bf16_round(pre)
    lo, hi = oracle.bf16_round(pre - (np.abs(pre) * 2.0**-19 + 2.0**-21)), oracle.bf16_round(
        pre + (np.abs(pre) * 2.0**-19 + 2.0**-21))
    for choice in itertools.product(*[(lo[i], hi[i]) for i in idx]):
        v = base.copy()
        v[idx] = choice
        yield v


def _check_vector(got_packed, got_scale, want_packed, want_scale, pre):
    if np.array_equal(got_packed, want_packed) and np.array_equal(got_scale, want_scale):
        return "exact"
    close = _close_to_boundary(pre)
    assert close.any(), "bytes differ with no element near a bf16 rounding boundary"
    assert close.sum() <= 6
    for v in _alternatives(pre, close):
        p, s = oracle.quant_q(v.reshape(1, 1, 128))
        if np.array_equal(got_packed, p[0, 0]) and np.array_equal(got_scale, s[0, 0]):
            return "boundary"
    raise AssertionError("bytes match none of the allowed bf16 roundings")


def compare(c, g, o):
    n_tok, H = c.q.shape[0], c.q.shape[1]
    assert g["err"] == o["err"]
    stats = {"exact": 0, "boundary": 0}
    # keys: compare slot by slot (untouched slots must stay as they were)
    written = {}
    for t in range(n_tok):
        s = int(c.slots[t])
        if s >= 0 and s < c.n_pages * 64 and not np.isnan(o["k_pre"][t]).all():
            written[s] = t
    for page in range(c.n_pages):
        for pos in range(64):
            slot = page * 64 + pos
            gsc = g["ks"][page, :, oracle.scale_slot(pos)]
            osc = o["ks"][page, :, oracle.scale_slot(pos)]
            if slot not in written:
                assert np.array_equal(g["kp"][page, pos], o["kp"][page, pos]) and np.array_equal(gsc, osc)
                continue
            stats[_check_vector(g["kp"][page, pos], gsc, o["kp"][page, pos], osc, o["k_pre"][written[slot]])] += 1
    for t in range(n_tok):
        for h in range(H):
            pre = o["q_pre"][t, h]
            if np.isnan(pre).all():  # skipped: the zero query exactly
                assert np.array_equal(g["qp"][t, h], o["qp"][t, h]) and np.array_equal(g["qs"][t, h], o["qs"][t, h])
                continue
            stats[_check_vector(g["qp"][t, h], g["qs"][t, h], o["qp"][t, h], o["qs"][t, h], pre)] += 1
    assert np.array_equal(g["wm"].view(np.uint32), o["w_mqa"].view(np.uint32))
    total = stats["exact"] + stats["boundary"]
    assert stats["exact"] >= 0.95 * total, stats
    return stats


@pytest.mark.parametrize("n_tok,H,rope_dim,interleaved,norm,all_q,pad_every", [
    (300, 64, 64, False, True, False, 7),
    (200, 16, 128, True, True, True, 5),
    (129, 32, 32, False, False, False, 3),
    (64, 128, 64, True, True, False, 0),
    (4096, 64, 64, False, True, False, 0),
])
def test_fused_writer_matches_oracle(ifp4, n_tok, H, rope_dim, interleaved, norm, all_q, pad_every):
    c = W.writer_case(n_tok, H, rope_dim=rope_dim, seed=n_tok + H, pad_every=pad_every)
    print(f"fused writer n_tok={n_tok} H={H} rope_dim={rope_dim} interleaved={interleaved} norm={norm} "
          f"all_q={all_q}", flush=True)
    g = run_gpu(ifp4, c, interleaved, norm, all_q)
    o = run_oracle(c, interleaved, norm, all_q)
    stats = compare(c, g, o)
    print(stats, flush=True)


def test_fused_writer_flags_positions_and_pool(ifp4):
    c = W.writer_case(100, 16, rope_dim=64, max_pos=512, seed=3, pad_every=9)
    c.positions[4] = 512          # one past the table
    c.positions[10] = -1
    c.slots[20] = c.n_pages * 64  # one past the pool
    g = run_gpu(ifp4, c, False, True, False, kv_fill=0x5A)
    o = run_oracle(c, False, True, False, kv_fill=0x5A)
    assert o["err"] == 16 | 32
    compare(c, g, o)


def test_fused_writer_without_norm_or_rope_is_the_plain_writer(ifp4):
    """No arithmetic before the quantizer: byte-identical to indexer_fp4_quant_and_cache."""
    c = W.writer_case(500, 64, rope_dim=0, seed=8, pad_every=11)
    g = run_gpu(ifp4, c, False, False, True)
    kp = torch.zeros((c.n_pages, 64, 64), dtype=torch.uint8, device=dev())
    ks = torch.zeros((c.n_pages, 4, 64), dtype=torch.uint8, device=dev())
    qp = torch.empty((500, 64, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((500, 64, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(_bf16_dev(c.k), to_dev(c.slots), kp, ks, _bf16_dev(c.q), qp, qs)
    torch.cuda.synchronize()
    assert np.array_equal(g["kp"], kp.cpu().numpy()) and np.array_equal(g["ks"], ks.cpu().numpy())
    assert np.array_equal(g["qp"], qp.cpu().numpy()) and np.array_equal(g["qs"], qs.cpu().numpy())
    assert g["err"] == 0
