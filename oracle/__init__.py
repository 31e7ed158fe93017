"""fp64 CPU oracle for the FP4 sparse-indexer scorer (ctypes wrapper over liboracle.so).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the cpu_baseline
leg of ``bench.py`` may import this package. The product path (the HIP library and
its binding) never does, and nothing here is shared with it.

Every wrapper takes and returns numpy arrays in host memory. The arithmetic lives in
``oracle.c``; its header comment lists the readings of the pages it commits to.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C11, fp64, OpenMP over independent rows)."""
    if force or not os.path.exists(LIB_PATH):
        cmd = [
            "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-shared", "-fPIC", "-Wall", "-Wextra", "-Werror",
            os.path.join(HERE, "oracle.c"), "-o", LIB_PATH + ".tmp", "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


def _declare(L):
    L.oracle_e2m1_value.argtypes = [ctypes.c_int]
    L.oracle_e2m1_value.restype = ctypes.c_double
    L.oracle_e8m0_value.argtypes = [ctypes.c_int]
    L.oracle_e8m0_value.restype = ctypes.c_double
    L.oracle_scale_slot.argtypes = [ctypes.c_int]
    L.oracle_scale_slot.restype = ctypes.c_int
    sigs = {
        "oracle_mx_encode_blocks": [P, I64, P, P],
        "oracle_quant_and_cache": [P, I64, I64, P, P, P, I64],
        "oracle_quant_q": [P, I64, I32, P, P],
        "oracle_dequant_key": [P, P, I64, I64, ctypes.c_int, P],
        "oracle_dequant_q": [P, P, I64, I32, I32, P],
        "oracle_decode_geometry": [P, I32, I32, P, P],
        "oracle_prefill_geometry": [P, P, I32, I32, P, P],
        "oracle_score": [P, P, P, I32, I64, P, P, P, P, I64, P, I64, P, I64, P],
        "oracle_topk": [P, I64, I64, P, I32, P, I64],
        "oracle_topk_merge": [P, P, I64, I64, I32, I32, P, I64],
        "oracle_decode_schedule": [P, I32, I32, P, P, P],
        "oracle_prefill_schedule": [P, P, I32, I32, I32, I32, I32, P, P, P, P, P],
        "oracle_layer_norm": [P, I32, P, P, ctypes.c_float, P],
        "oracle_mx8_encode_blocks": [P, I64, P, P],
        "oracle_quant8_and_cache": [P, I64, I64, P, P, P, I64],
        "oracle_quant8_q": [P, I64, I32, P, P],
        "oracle_dequant8_key": [P, P, I64, I64, ctypes.c_int, P],
        "oracle_score8": [P, P, P, I32, I64, P, P, P, P, I64, P, I64, P, I64, P],
        "oracle_rope": [P, I32, I32, P],
        "oracle_norm_rope_quant_and_cache": [P, I64, I64, P, P, ctypes.c_float, P, P, I64, I32, I32, P, P, P, I64,
                                             P, I32, P, P, P, ctypes.c_float, P, I32, P, P, P],
    }
    L.oracle_e4m3_value.argtypes = [ctypes.c_int]
    L.oracle_e4m3_value.restype = ctypes.c_double
    L.oracle_bf16_round.argtypes = [ctypes.c_double]
    L.oracle_bf16_round.restype = ctypes.c_uint16
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc}")


# ---- element encodings --------------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return lib().oracle_e8m0_value(int(byte))


def scale_slot(pos: int) -> int:
    return lib().oracle_scale_slot(int(pos))


def mx_encode_blocks(vals_bf16: np.ndarray):
    """vals_bf16: uint16 [n_blocks, 32] -> (scale uint8 [n_blocks], codes uint8 [n_blocks, 32])."""
    v = _c(vals_bf16, np.uint16).reshape(-1, 32)
    n = v.shape[0]
    scale = np.zeros(n, np.uint8)
    codes = np.zeros((n, 32), np.uint8)
    _check(lib().oracle_mx_encode_blocks(_p(v), n, _p(scale), _p(codes)), "mx_encode_blocks")
    return scale, codes


# ---- cache write / query quantization ------------------------------------------------

def quant_and_cache(k_bf16, slot_mapping, kv_packed, kv_scale):
    """Writes keys into the caller's planes in place (numpy uint8 arrays)."""
    k = _c(k_bf16, np.uint16)
    n_tok, k_ld = k.shape
    slots = _c(slot_mapping, np.int64)
    assert kv_packed.dtype == np.uint8 and kv_scale.dtype == np.uint8
    n_pages = kv_packed.shape[0]
    assert kv_packed.shape == (n_pages, 64, 64) and kv_scale.shape == (n_pages, 4, 64)
    _check(lib().oracle_quant_and_cache(_p(k), n_tok, k_ld, _p(slots), _p(kv_packed), _p(kv_scale), n_pages),
           "quant_and_cache")


def quant_q(q_bf16):
    """q: uint16 [rows, H, 128] -> (q_packed uint8 [rows, H, 64], q_scale uint8 [rows, H, 4])."""
    q = _c(q_bf16, np.uint16)
    rows, h, d = q.shape
    assert d == 128
    qp = np.zeros((rows, h, 64), np.uint8)
    qs = np.zeros((rows, h, 4), np.uint8)
    _check(lib().oracle_quant_q(_p(q), rows, h, _p(qp), _p(qs)), "quant_q")
    return qp, qs


def dequant_key(kv_packed, kv_scale, page, pos):
    out = np.zeros(128, np.float64)
    _check(lib().oracle_dequant_key(_p(kv_packed), _p(kv_scale), kv_packed.shape[0], int(page), int(pos), _p(out)),
           "dequant_key")
    return out


def dequant_q(q_packed, q_scale, row, h):
    out = np.zeros(128, np.float64)
    n_heads = q_packed.shape[1]
    _check(lib().oracle_dequant_q(_p(q_packed), _p(q_scale), int(row), n_heads, int(h), _p(out)), "dequant_q")
    return out


# ---- MXFP8 comparator (reading R16 in oracle.c) ---------------------------------------

def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def mx8_encode_blocks(vals_bf16: np.ndarray):
    """uint16 [n_blocks, 32] -> (scale uint8 [n_blocks], codes uint8 [n_blocks, 32])."""
    v = _c(vals_bf16, np.uint16).reshape(-1, 32)
    n = v.shape[0]
    scale = np.zeros(n, np.uint8)
    codes = np.zeros((n, 32), np.uint8)
    _check(lib().oracle_mx8_encode_blocks(_p(v), n, _p(scale), _p(codes)), "mx8_encode_blocks")
    return scale, codes


def quant8_and_cache(k_bf16, slot_mapping, kv_packed, kv_scale):
    """kv_packed uint8 [n_pages, 64, 128], kv_scale uint8 [n_pages, 4, 64], written in place."""
    k = _c(k_bf16, np.uint16)
    slots = _c(slot_mapping, np.int64)
    n_pages = kv_packed.shape[0]
    assert kv_packed.shape == (n_pages, 64, 128) and kv_scale.shape == (n_pages, 4, 64)
    _check(lib().oracle_quant8_and_cache(_p(k), k.shape[0], k.shape[1], _p(slots), _p(kv_packed), _p(kv_scale),
                                         n_pages), "quant8_and_cache")


def quant8_q(q_bf16):
    q = _c(q_bf16, np.uint16)
    rows, h, d = q.shape
    qp = np.zeros((rows, h, 128), np.uint8)
    qs = np.zeros((rows, h, 4), np.uint8)
    _check(lib().oracle_quant8_q(_p(q), rows, h, _p(qp), _p(qs)), "quant8_q")
    return qp, qs


def dequant8_key(kv_packed, kv_scale, page, pos):
    out = np.zeros(128, np.float64)
    _check(lib().oracle_dequant8_key(_p(kv_packed), _p(kv_scale), kv_packed.shape[0], int(page), int(pos), _p(out)),
           "dequant8_key")
    return out


def score8(q_packed, q_scale, w, row_seq, row_len, kv_packed, kv_scale, block_table, ld=None, fill=np.nan):
    """score() over MXFP8 planes."""
    return _score_impl(lib().oracle_score8, q_packed, q_scale, w, row_seq, row_len, kv_packed, kv_scale,
                       block_table, ld, fill)


# ---- fused writer: k_norm, RoPE, bf16 rounding (readings R12-R15 in oracle.c) ----------

def bf16_round(x) -> np.ndarray:
    """fp64 values -> nearest bf16 bit patterns (ties to even), elementwise."""
    x = np.asarray(x, np.float64)
    f = np.vectorize(lambda v: lib().oracle_bf16_round(float(v)), otypes=[np.uint16])
    return f(x) if x.size else np.zeros(x.shape, np.uint16)


def layer_norm(x, gamma, beta, eps):
    x = _c(x, np.float64)
    y = np.zeros_like(x)
    g = _c(gamma, np.float32)
    b = None if beta is None else _c(beta, np.float32)
    _check(lib().oracle_layer_norm(_p(x), x.size, _p(g), None if b is None else _p(b), float(eps), _p(y)),
           "layer_norm")
    return y


def rope(x, cs_row, rope_dim, interleaved=False):
    """x: fp64 [128] (copied), cs_row: fp32 [rope_dim] = cos[half] then sin[half]."""
    y = np.array(x, np.float64, copy=True)
    c = _c(cs_row, np.float32)
    _check(lib().oracle_rope(_p(y), int(rope_dim), int(interleaved), _p(c)), "rope")
    return y


def norm_rope_quant_and_cache(k_bf16, positions, cos_sin, rope_dim, interleaved, gamma, beta, eps, slot_mapping,
                              kv_packed, kv_scale, q_bf16=None, weights=None, weight_scale=1.0, all_q=False):
    """The fused writer. Writes keys into (kv_packed, kv_scale) in place and returns dict(qp, qs,
    w_mqa, err, k_pre, q_pre): the fp64 vectors just before bf16 rounding (NaN where not computed)."""
    k = _c(k_bf16, np.uint16)
    n_tok, k_ld = k.shape
    pos = _c(positions, np.int64)
    cs = _c(cos_sin if cos_sin is not None else np.zeros((1, 2), np.float32), np.float32)
    max_pos = cs.shape[0] if cos_sin is not None else 0
    slots = _c(slot_mapping, np.int64)
    g = None if gamma is None else _c(gamma, np.float32)
    b = None if beta is None else _c(beta, np.float32)
    k_pre = np.zeros((n_tok, 128), np.float64)
    out = dict(k_pre=k_pre)
    if q_bf16 is not None:
        q = _c(q_bf16, np.uint16)
        H = q.shape[1]
        w = _c(weights, np.float32)
        qp = np.zeros((n_tok, H, 64), np.uint8)
        qs = np.zeros((n_tok, H, 4), np.uint8)
        wm = np.zeros((n_tok, H), np.float32)
        q_pre = np.zeros((n_tok, H, 128), np.float64)
        out.update(qp=qp, qs=qs, w_mqa=wm, q_pre=q_pre)
    else:
        q = w = qp = qs = wm = q_pre = None
        H = 0
    err = np.zeros(1, np.int32)
    _check(lib().oracle_norm_rope_quant_and_cache(
        _p(k), n_tok, k_ld, None if g is None else _p(g), None if b is None else _p(b), float(eps), _p(pos), _p(cs),
        max_pos, int(rope_dim), int(interleaved), _p(slots), _p(kv_packed), _p(kv_scale), kv_packed.shape[0],
        None if q is None else _p(q), H, None if qp is None else _p(qp), None if qs is None else _p(qs),
        None if w is None else _p(w), float(weight_scale), None if wm is None else _p(wm), int(bool(all_q)),
        _p(k_pre), None if q_pre is None else _p(q_pre), _p(err)), "norm_rope_quant_and_cache")
    out["err"] = int(err[0])
    return out


# ---- geometry -------------------------------------------------------------------------

def decode_geometry(ctx, next_n=1):
    ctx = _c(ctx, np.int32)
    b = ctx.shape[0]
    row_seq = np.zeros(b * next_n, np.int32)
    row_len = np.zeros(b * next_n, np.int32)
    _check(lib().oracle_decode_geometry(_p(ctx), b, next_n, _p(row_seq), _p(row_len)), "decode_geometry")
    return row_seq, row_len


def prefill_geometry(cu_rows, start_pos, n_rows_padded):
    cu = _c(cu_rows, np.int32)
    sp = _c(start_pos, np.int32)
    n_req = sp.shape[0]
    row_seq = np.zeros(n_rows_padded, np.int32)
    row_len = np.zeros(n_rows_padded, np.int32)
    _check(lib().oracle_prefill_geometry(_p(cu), _p(sp), n_req, n_rows_padded, _p(row_seq), _p(row_len)),
           "prefill_geometry")
    return row_seq, row_len


# ---- score / top-k --------------------------------------------------------------------

def score(q_packed, q_scale, w, row_seq, row_len, kv_packed, kv_scale, block_table, ld=None, fill=np.nan):
    """fp64 logits [rows, ld]; entries at j >= row_len keep `fill`. Returns (logits, reads)."""
    return _score_impl(lib().oracle_score, q_packed, q_scale, w, row_seq, row_len, kv_packed, kv_scale,
                       block_table, ld, fill)


def _score_impl(fn, q_packed, q_scale, w, row_seq, row_len, kv_packed, kv_scale, block_table, ld, fill):
    qp = _c(q_packed, np.uint8)
    qs = _c(q_scale, np.uint8)
    w = _c(w, np.float32)
    rows, h, _ = qp.shape
    rs = _c(row_seq, np.int32)
    rl = _c(row_len, np.int32)
    bt = _c(block_table, np.int32)
    if ld is None:
        ld = max(int(rl.max()) if rl.size else 1, 1)
    out = np.full((rows, ld), fill, np.float64)
    reads = np.zeros(rows, np.int64)
    _check(fn(_p(qp), _p(qs), _p(w), h, rows, _p(rs), _p(rl), _p(kv_packed), _p(kv_scale), kv_packed.shape[0],
              _p(bt), bt.shape[1], _p(out), ld, _p(reads)), "score")
    return out, reads


def topk(s, row_len, k):
    s = _c(s, np.float64)
    rows, ld = s.shape
    rl = _c(row_len, np.int32)
    idx = np.full((rows, k), -7, np.int32)
    _check(lib().oracle_topk(_p(s), ld, rows, _p(rl), k, _p(idx), k), "topk")
    return idx


def topk_merge(score, index, k):
    """score float [rows, n_cand], index int32 [rows, n_cand] (< 0: empty) -> int32 [rows, k]."""
    sc = _c(score, np.float64)
    ix = _c(index, np.int32)
    rows, n = sc.shape
    out = np.full((rows, k), -7, np.int32)
    _check(lib().oracle_topk_merge(_p(sc), _p(ix), n, rows, n, k, _p(out), k), "topk_merge")
    return out


# ---- schedules ------------------------------------------------------------------------

def decode_schedule(ctx, n_units):
    ctx = _c(ctx, np.int32)
    b = ctx.shape[0]
    cum = np.zeros(b + 1, np.int32)
    ub = np.zeros(n_units + 1, np.int32)
    us = np.zeros(n_units, np.int32)
    _check(lib().oracle_decode_schedule(_p(ctx), b, n_units, _p(cum), _p(ub), _p(us)), "decode_schedule")
    return {"cum_pages": cum, "unit_begin": ub, "unit_seq": us}


def prefill_schedule(cu_rows, start_pos, n_rows_padded, tile_rows, n_units):
    cu = _c(cu_rows, np.int32)
    sp = _c(start_pos, np.int32)
    n_req = sp.shape[0]
    max_tiles = n_rows_padded // tile_rows + n_req + 1
    nt = np.zeros(1, np.int32)
    tiles = np.zeros((max_tiles, 4), np.int32)
    cum = np.zeros(max_tiles + 1, np.int32)
    ub = np.zeros(n_units + 1, np.int32)
    ut = np.zeros(n_units, np.int32)
    _check(lib().oracle_prefill_schedule(_p(cu), _p(sp), n_req, n_rows_padded, tile_rows, n_units, max_tiles,
                                         _p(nt), _p(tiles), _p(cum), _p(ub), _p(ut)), "prefill_schedule")
    n = int(nt[0])
    return {"tiles": tiles[:n].copy(), "cum_items": cum[: n + 1].copy(), "unit_begin": ub, "unit_tile": ut}
