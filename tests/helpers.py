"""Runners shared by the GPU tests: the same seeded inputs through the HIP path (via the
binding) and through the CPU oracle, plus the comparison rules.

Comparison rules:
  - cache planes, query planes, schedules and row lengths: bit-exact;
  - logits: |gpu - oracle| <= 1e-3 * |oracle| for every valid (row, column), and columns at
    or past the row's length keep the sentinel they were filled with;
  - top-k: both sets have min(k, row_len) distinct in-range columns, and every column in
    their symmetric difference has an oracle score within 1e-3 relative of the oracle's k-th
    score (near-ties may resolve differently between fp32 and fp64 scores).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

RTOL = 1e-3


def dev():
    return torch.device("cuda:0")


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


# ---------------------------------------------------------------------------- decode

def gpu_decode(case: W.DecodeCase, units=None, ld=None, fill=float("nan"), cache_fill=0, run_topk=True, fused=False):
    """fused: the scorer fills the top-k's first histogram (out["hist"]: a copy taken between
    the two calls; out["row_hist"]: the buffer after the top-k)."""
    import sparse_attention_indexer_fp4_amd as ifp4

    units = units or ifp4.DECODE_UNITS
    B, H, nn, rows = case.batch, case.heads, case.next_n, case.rows
    ld = ld or case.block_table.shape[1] * W.PAGE
    kp = torch.full((case.n_pages, 64, 64), cache_fill, dtype=torch.uint8, device=dev())
    ks = torch.full((case.n_pages, 4, 64), cache_fill, dtype=torch.uint8, device=dev())
    qp = torch.empty((rows, H, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((rows, H, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(case.keys), to_dev(case.slots), kp, ks, bf16_tensor(case.q), qp, qs)
    sched = torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, nn, units), dtype=torch.uint8, device=dev())
    row_len = torch.empty(rows, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_decode_schedule(to_dev(case.ctx), nn, units, sched, row_len)
    logits = torch.full((rows, ld), fill, dtype=torch.float32, device=dev())
    row_hist = ifp4.row_histogram(rows, dev()) if fused else None
    ifp4.indexer_fp4_score_decode(qp, qs, to_dev(case.w), kp, ks, to_dev(case.block_table), nn, sched, units,
                                  row_len, logits, row_hist)
    out = dict(kp=kp, ks=ks, qp=qp, qs=qs, sched=sched, row_len=row_len, logits=logits, units=units, ld=ld)
    if fused:
        out["hist"] = row_hist.clone()
        out["row_hist"] = row_hist
    if run_topk:
        top = torch.full((rows, case.topk), -7, dtype=torch.int32, device=dev())
        ws_bytes = ifp4.indexer_topk_workspace_bytes(rows, ld, case.topk)
        ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev())
        ifp4.indexer_topk(logits, row_len, ld, case.topk, top, ws, row_hist)
        out["top"] = top
    torch.cuda.synchronize()
    out["err"] = ifp4.sched_error(sched)
    return out


def oracle_decode(case: W.DecodeCase, ld=None, scores=True):
    ld = ld or case.block_table.shape[1] * W.PAGE
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    qp, qs = oracle.quant_q(case.q)
    rs, rl = oracle.decode_geometry(case.ctx, case.next_n)
    out = dict(kp=kp, ks=ks, qp=qp, qs=qs, row_seq=rs, row_len=rl)
    if scores:
        s, reads = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table, ld=ld)
        out.update(s=s, reads=reads, top=oracle.topk(s, rl, case.topk))
    return out


# ---------------------------------------------------------------------------- prefill

def gpu_prefill_step(case: W.PrefillCase, step: W.PrefillStep, kp, ks, units=None, ld=None, fill=float("nan"),
                     run_topk=True):
    """Writes the step's keys into (kp, ks), then schedules, scores and selects."""
    import sparse_attention_indexer_fp4_amd as ifp4

    units = units or ifp4.PREFILL_UNITS
    H, NP, R = case.heads, step.n_rows_padded, len(step.req_ids)
    bt = W.step_block_table(case, step)
    ld = ld or bt.shape[1] * W.PAGE
    keys, slots = W.step_keys(case, step)
    qp = torch.empty((NP, H, 64), dtype=torch.uint8, device=dev())
    qs = torch.empty((NP, H, 4), dtype=torch.uint8, device=dev())
    ifp4.indexer_fp4_quant_and_cache(bf16_tensor(keys), to_dev(slots), kp, ks, bf16_tensor(step.q), qp, qs)
    sched = torch.empty(ifp4.indexer_fp4_prefill_sched_bytes(R, NP, units, bt.shape[1]), dtype=torch.uint8,
                        device=dev())
    row_len = torch.empty(NP, dtype=torch.int32, device=dev())
    ifp4.indexer_fp4_prefill_schedule(to_dev(step.cu_rows), to_dev(step.start_pos), NP, units, to_dev(bt),
                                      kp.shape[0], sched, row_len)
    logits = torch.full((NP, ld), fill, dtype=torch.float32, device=dev())
    ifp4.indexer_fp4_score_prefill(qp, qs, to_dev(step.w), kp, ks, R, bt.shape[1], sched, units, NP, logits)
    out = dict(qp=qp, qs=qs, sched=sched, row_len=row_len, logits=logits, units=units, ld=ld)
    if run_topk:
        top = torch.full((NP, case.topk), -7, dtype=torch.int32, device=dev())
        ws = torch.zeros(max(ifp4.indexer_topk_workspace_bytes(NP, ld, case.topk), 1), dtype=torch.uint8,
                         device=dev())
        ifp4.indexer_topk(logits, row_len, ld, case.topk, top, ws)
        out["top"] = top
    torch.cuda.synchronize()
    out["err"] = ifp4.sched_error(sched)
    return out


def oracle_prefill_step(case: W.PrefillCase, step: W.PrefillStep, kp, ks, ld=None, scores=True):
    bt = W.step_block_table(case, step)
    ld = ld or bt.shape[1] * W.PAGE
    keys, slots = W.step_keys(case, step)
    oracle.quant_and_cache(keys, slots, kp, ks)
    qp, qs = oracle.quant_q(step.q)
    rs, rl = oracle.prefill_geometry(step.cu_rows, step.start_pos, step.n_rows_padded)
    out = dict(qp=qp, qs=qs, row_seq=rs, row_len=rl)
    if scores:
        s, reads = oracle.score(qp, qs, step.w, rs, rl, kp, ks, bt, ld=ld)
        out.update(s=s, reads=reads, top=oracle.topk(s, rl, case.topk))
    return out


# ---------------------------------------------------------------------------- checks

def check_logits(g: np.ndarray, s: np.ndarray, row_len: np.ndarray, sentinel_nan=True):
    g = g.astype(np.float64)
    worst = 0.0
    for r in range(g.shape[0]):
        L = int(row_len[r])
        if L:
            assert np.isfinite(g[r, :L]).all(), f"row {r}: a column below its length {L} is not finite (never written?)"
            err = np.abs(g[r, :L] - s[r, :L])
            bad = err > RTOL * np.abs(s[r, :L])
            if bad.any():
                j = int(np.nonzero(bad)[0][0])
                raise AssertionError(f"row {r} col {j}: gpu {g[r, j]!r} oracle {s[r, j]!r} (len {L})")
            worst = max(worst, float((err / np.maximum(np.abs(s[r, :L]), 1e-300)).max()))
        if sentinel_nan:
            assert np.isnan(g[r, L:]).all(), f"row {r} wrote at or past its length {L}"
    return worst


def check_topk(gtop: np.ndarray, otop: np.ndarray, s: np.ndarray, row_len: np.ndarray, k: int):
    for r in range(gtop.shape[0]):
        L = int(row_len[r])
        n = min(k, L)
        g = gtop[r]
        assert (g[n:] == -1).all(), f"row {r}: entries past {n} must be -1"
        gs = g[:n]
        assert ((gs >= 0) & (gs < L)).all(), f"row {r}: index out of range"
        assert len(set(gs.tolist())) == n, f"row {r}: duplicate indices"
        if n == 0:
            continue
        os_ = set(otop[r][:n].tolist())
        diff = set(gs.tolist()) ^ os_
        if diff:
            kth = s[r, otop[r][n - 1]]
            for j in diff:
                assert abs(s[r, j] - kth) <= RTOL * abs(kth), \
                    f"row {r}: column {j} (score {s[r, j]!r}) differs but is not near the k-th {kth!r}"
