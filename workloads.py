"""Seeded synthetic inputs for the FP4 sparse-indexer scorer.

This module only draws inputs: bf16 queries and keys, fp32 head weights, context
lengths, paged block tables, slot mappings and prefill chunk schedules. It holds none
of the method's arithmetic (no quantization, no scoring, no top-k), so both the HIP
path and the CPU oracle may take their inputs from it.

Distributions follow the workloads the pages describe ("Score a DSA sparse indexer in
FP4", PR description Performance / Accuracy): q ~ N(0,1) and keys ~ N(0,1) in bf16,
head weights ~ U(0,1) in fp32, 64-token pages placed by a shuffled block table. Every
tensor gets its own child stream of a numpy PCG64 generator seeded by ``seed``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 64
HEAD_DIM = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) bf16 bit patterns, drawn in chunks to bound host memory."""
    total = int(np.prod(shape))
    out = np.empty(total, np.uint16)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        out[s:e] = bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def scale_tokens_pow2(rng: np.random.Generator, keys_bf16: np.ndarray, lo: int = -6, hi: int = 6) -> np.ndarray:
    """Multiply each token (row) by 2^u, u ~ U{lo..hi}: exact in bf16 for these ranges.

    Makes neighbouring keys' block scales differ widely, so a key read with another
    key's exponent changes its score (the failure the pages' second review finding
    describes)."""
    u = rng.integers(lo, hi + 1, size=keys_bf16.shape[0])
    f = bf16_to_f32(keys_bf16) * np.exp2(u.astype(np.float32))[:, None]
    return bf16_bits(f)


@dataclass
class DecodeCase:
    name: str
    ctx: np.ndarray          # int32 [B]
    next_n: int
    heads: int
    topk: int
    q: np.ndarray            # uint16 bf16 [B*next_n, H, 128]
    w: np.ndarray            # float32 [B*next_n, H]
    keys: np.ndarray         # uint16 bf16 [sum(ctx), 128], sequence-major
    slots: np.ndarray        # int64 [sum(ctx)] pool slot of each key
    block_table: np.ndarray  # int32 [B, W], -1 past each sequence's pages
    n_pages: int
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.ctx.shape[0])

    @property
    def rows(self):
        return self.batch * self.next_n


def _paged_layout(rng: np.random.Generator, ctx: np.ndarray, slack: float = 0.10):
    """Random permutation of a pool of (needed pages + slack) over the sequences."""
    pages_per = (ctx.astype(np.int64) + PAGE - 1) // PAGE
    need = int(pages_per.sum())
    n_pages = max(need + int(np.ceil(need * slack)), 1)
    perm = rng.permutation(n_pages).astype(np.int32)
    width = max(int(pages_per.max()) if ctx.size else 1, 1)
    bt = np.full((ctx.shape[0], width), -1, np.int32)
    slots = np.empty(int(ctx.astype(np.int64).sum()), np.int64)
    off = 0
    koff = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[off:off + n]
        off += n
        L = int(ctx[b])
        j = np.arange(L, dtype=np.int64)
        slots[koff:koff + L] = bt[b, j // PAGE].astype(np.int64) * PAGE + (j % PAGE)
        koff += L
    return bt, slots, n_pages


def decode_case(ctx, heads, topk, seed=0, next_n=1, swizzle_sensitive=False, name="decode") -> DecodeCase:
    ctx = np.asarray(ctx, np.int32)
    rq, rw, rk, rp, ru = _streams(seed, 5)
    rows = ctx.shape[0] * next_n
    q = normal_bf16(rq, (rows, heads, HEAD_DIM))
    w = rw.random((rows, heads), dtype=np.float32)
    keys = normal_bf16(rk, (int(ctx.astype(np.int64).sum()), HEAD_DIM))
    if swizzle_sensitive:
        keys = scale_tokens_pow2(ru, keys)
    bt, slots, n_pages = _paged_layout(rp, ctx)
    return DecodeCase(name, ctx, next_n, heads, topk, q, w, keys, slots, bt, n_pages)


# The decode workloads: tiny (2 x {300, 512}, 16 heads, top-64), batch 1 x 4096,
# batch 8 x 131072, and the long sweep (16 x 131072, 8 x 262144); 64 heads and
# top-2048 unless stated.
DECODE_CONFIGS = {
    "decode_tiny": dict(ctx=[300, 512], heads=16, topk=64),
    "decode_b1_4k": dict(ctx=[4096], heads=64, topk=2048),
    "decode_b8_128k": dict(ctx=[131072] * 8, heads=64, topk=2048),
    "decode_b16_128k": dict(ctx=[131072] * 16, heads=64, topk=2048),
    "decode_b8_256k": dict(ctx=[262144] * 8, heads=64, topk=2048),
}


def decode_config(name: str, seed: int = 0, **kw) -> DecodeCase:
    p = dict(DECODE_CONFIGS[name])
    p.update(kw)
    return decode_case(seed=seed, name=name, **p)


# ---------------------------------------------------------------------------------------
# Prefill: requests of length U[2634, 4295] (the prompt-length range of the pages'
# accuracy runs), chunked at 512 tokens per step, all live requests co-scheduled; or, as
# the secondary stream, steps of at most 512 tokens in all (a scheduler's token budget),
# filled by the live requests in order, so requests are cut mid-way and a step can hold
# the end of one request and the start of the next.

def prefill_lengths(n_req=4, lo=2634, hi=4295, multiple=8):
    """First seed s = 0, 1, ... whose draw has a total that is not a multiple of 8,
    so the last step carries padding rows."""
    s = 0
    while True:
        L = np.random.default_rng(s).integers(lo, hi + 1, n_req)
        if int(L.sum()) % multiple != 0:
            return L.astype(np.int32), s
        s += 1


@dataclass
class PrefillStep:
    cu_rows: np.ndarray     # int32 [R+1], rows of request i = [cu_rows[i], cu_rows[i+1])
    start_pos: np.ndarray   # int32 [R], position of request i's first row in this step
    req_ids: np.ndarray     # int32 [R], which request of the case each step-request is
    n_rows_padded: int      # rows rounded up to a multiple of 8
    q: np.ndarray           # uint16 bf16 [n_rows_padded, H, 128]
    w: np.ndarray           # float32 [n_rows_padded, H]; padding rows carry zero weight

    @property
    def n_rows(self):
        return int(self.cu_rows[-1])


@dataclass
class PrefillCase:
    name: str
    lengths: np.ndarray     # int32 [n_req]
    heads: int
    topk: int
    chunk: int
    keys: list              # per request: uint16 bf16 [L_i, 128]
    slots: list             # per request: int64 [L_i]
    block_table: np.ndarray  # int32 [n_req, W], -1 past each request's pages
    n_pages: int
    steps: list             # PrefillStep


def prefill_case(lengths, heads=64, topk=2048, chunk=512, seed=0, pad_multiple=8,
                 swizzle_sensitive=False, name="prefill", budget=None) -> PrefillCase:
    L = np.asarray(lengths, np.int32)
    rk, rp, rq, rw, ru = _streams(seed, 5)
    keys = [normal_bf16(rk, (int(n), HEAD_DIM)) for n in L]
    if swizzle_sensitive:
        keys = [scale_tokens_pow2(ru, k) for k in keys]
    bt, slots_flat, n_pages = _paged_layout(rp, L)
    slots = []
    off = 0
    for n in L:
        slots.append(slots_flat[off:off + int(n)])
        off += int(n)
    steps = []
    done = np.zeros_like(L)
    while (done < L).any():
        live = np.nonzero(done < L)[0].astype(np.int32)
        adv = np.minimum(chunk, L[live] - done[live]).astype(np.int32)
        if budget is not None:  # first come, first served up to the step's token budget
            left = np.maximum(budget - (np.cumsum(adv) - adv), 0)
            adv = np.minimum(adv, left).astype(np.int32)
            live, adv = live[adv > 0], adv[adv > 0]
        cu = np.zeros(live.shape[0] + 1, np.int32)
        cu[1:] = np.cumsum(adv)
        n_rows = int(cu[-1])
        n_pad = -(-n_rows // pad_multiple) * pad_multiple
        q = normal_bf16(rq, (n_pad, heads, HEAD_DIM))
        w = rw.random((n_pad, heads), dtype=np.float32)
        w[n_rows:] = 0.0
        steps.append(PrefillStep(cu, done[live].astype(np.int32), live, n_pad, q, w))
        done[live] += adv
    return PrefillCase(name, L, heads, topk, chunk, keys, slots, bt, n_pages, steps)


def prefill_config(name: str = "prefill_4req", seed: int = 0, **kw) -> PrefillCase:
    if name == "prefill_4req":
        L, _ = prefill_lengths()
        p = dict(lengths=L, heads=64, topk=2048, chunk=512)
    elif name == "prefill_4req_mbt512":
        L, _ = prefill_lengths()
        p = dict(lengths=L, heads=64, topk=2048, chunk=512, budget=512)
    elif name == "prefill_tiny":
        # three short requests, 48-row chunks: several chunks, ragged groups, padding rows
        p = dict(lengths=[70, 5, 133], heads=16, topk=64, chunk=48)
    elif name == "prefill_tiny_mbt":
        # the same requests under a 60-token step budget: requests cut mid-way, steps that
        # end one request and start the next
        p = dict(lengths=[70, 5, 133], heads=16, topk=64, chunk=48, budget=60)
    else:
        raise KeyError(name)
    p.update(kw)
    return prefill_case(seed=seed, name=name, **p)


def step_block_table(case: PrefillCase, step: PrefillStep) -> np.ndarray:
    """Block-table rows of the requests live in a step, in step order (row i = request i)."""
    return np.ascontiguousarray(case.block_table[step.req_ids])


def step_keys(case: PrefillCase, step: PrefillStep):
    """Keys and slots the cache write stores before the step is scored (the chunk's own keys)."""
    ks, ss = [], []
    for i, r in enumerate(step.req_ids):
        a = int(step.start_pos[i])
        b = a + int(step.cu_rows[i + 1] - step.cu_rows[i])
        ks.append(case.keys[r][a:b])
        ss.append(case.slots[r][a:b])
    return np.concatenate(ks), np.concatenate(ss)


# ---------------------------------------------------------------------------- fused writer inputs

@dataclass
class WriterCase:
    """Inputs of the fused writer: per token a bf16 key, H bf16 query heads, fp32 head weights,
    a rotary position and a cache slot, plus the LayerNorm parameters and the cos/sin table."""
    k: np.ndarray          # uint16 [n_tok, 128] (bf16 bits)
    q: np.ndarray          # uint16 [n_tok, H, 128]
    w: np.ndarray          # float32 [n_tok, H]
    gamma: np.ndarray      # float32 [128]
    beta: np.ndarray       # float32 [128]
    cos_sin: np.ndarray    # float32 [max_pos, rope_dim]: cos of the angles, then their sin
    positions: np.ndarray  # int64 [n_tok]
    slots: np.ndarray      # int64 [n_tok]
    n_pages: int
    rope_dim: int


def rope_table(max_pos: int, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """The usual rotary angle table: angle (p, i) = p * base^(-2i / rope_dim), stored as fp32
    cos values for i < rope_dim/2 followed by the sin values."""
    if rope_dim == 0:
        return np.zeros((max_pos, 0), np.float32)
    inv = base ** (-np.arange(rope_dim // 2, dtype=np.float64) * 2.0 / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def writer_case(n_tok, heads, rope_dim=64, max_pos=8192, seed=0, pad_every=0, key_scale=1.0) -> WriterCase:
    """Keys ~ N(key_scale, 1)-ish activations (an offset so LayerNorm has a mean to remove), q ~
    N(0, 1), weights ~ N(0, 1), gamma ~ U(0.5, 1.5), beta ~ U(-0.2, 0.2), positions uniform in the
    table, every token on its own slot of a shuffled pool; every pad_every-th token has slot -1."""
    rk, rq, rw, rg, rp, rs = _streams(seed, 6)
    k = bf16_bits(rk.standard_normal((n_tok, HEAD_DIM)).astype(np.float32) + np.float32(key_scale))
    q = normal_bf16(rq, (n_tok, heads, HEAD_DIM))
    w = rw.standard_normal((n_tok, heads)).astype(np.float32)
    gamma = rg.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
    beta = rg.uniform(-0.2, 0.2, HEAD_DIM).astype(np.float32)
    positions = rp.integers(0, max_pos, n_tok).astype(np.int64)
    n_pages = -(-n_tok // PAGE) + 1
    slots = rs.permutation(n_pages * PAGE)[:n_tok].astype(np.int64)
    if pad_every:
        slots[::pad_every] = -1
    return WriterCase(k, q, w, gamma, beta, rope_table(max_pos, rope_dim), positions, slots, n_pages, rope_dim)
