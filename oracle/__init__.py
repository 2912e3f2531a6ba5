"""CPU oracle for the absorbed MLA decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never loads it and
shares no code with it.

Two independent CPU implementations live here:

* ``mla_oracle.c`` (built with gcc into ``liboracle.so``): the plain fp64
  Normal path -- up-project every cached latent through W_UK and W_UV, run
  ordinary attention over 192-wide keys and 128-wide values -- plus an fp64
  absorbed mirror stage by stage (absorb, latent attention with optional
  split partials, merge, un-absorb).  Its header cites the passages followed.
* ``expanded_attention_f64`` / ``absorbed_attention_f64`` below: small numpy
  float64 versions for tiny inputs, used to pin the C code.
* ``e4m3fn_decode`` / ``bf16_round`` / ``fp8_rows_to_bf16``: the FP8 cache
  row (M5.8 0x0B) dequantized to the bf16 rows the stages above read; pinned
  to PyTorch's float8_e4m3fn conversion, the encoding's closed forms, a
  hand-built row and single rounding at constructed ties.

Pages ("MLA in full detail", mlinterviewnotes; "M5.8 - Multi-Head Latent
Attention", transformer-system) define the computation; every stage function
docstring names its passage.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

D_NOPE, D_ROPE, D_V, R_LATENT = 128, 64, 128, 512

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with the host compiler (gcc, fp64, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared",
                               "-fPIC", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L.mlao_normal_decode.argtypes = [P, P, P, P, P, I, I, P, I, P, I, I, I, I, I, I, I,
                                         D, P, I, P, P, I]
        L.mlao_absorb.argtypes = [P, P, I, I, I, I, I, P]
        L.mlao_unabsorb.argtypes = [P, P, I, I, I, I, I, P]
        L.mlao_split_plan.argtypes = [P, I, I, I, P, P, P]
        L.mlao_latent_attention.argtypes = [P, P, P, I, I, P, I, P, I, I, I, I, I, D,
                                            P, P, P, P, I, P, P, I]
        L.mlao_merge.argtypes = [P, P, P, I, I, I, I, P, P]
        L.mlao_phys_row.argtypes = [P, I, I, I, I, I]
        L.mlao_phys_row.restype = ctypes.c_longlong
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check(st, what):
    if st != 0:
        raise RuntimeError(f"oracle {what} failed with status {st}")


def normal_scale() -> float:
    """Softmax scale of MLA: that of the original 192-wide key, 1/sqrt(d_nope + d_rope)
    ("MLA in full detail", numpy parity script; zdszero, scale kept at 192)."""
    return 1.0 / math.sqrt(D_NOPE + D_ROPE)


def phys_row(block_table, b, j, page_size, num_blocks) -> int:
    bt = _c(block_table, np.int32)
    return int(lib().mlao_phys_row(_p(bt), bt.shape[1], b, j, page_size, num_blocks))


def append_rows(kv_cache, block_table, seqlens, c_new, kpe_new, page_size):
    """Cache append of a decode step (M5.8 0x05, "Exact phase algorithms and
    commit state": the step's new row is stored once, at its own position;
    "Paged and ragged address translation" for where that row lives).

    ``seqlens`` are the lengths after the step, so new row t of sequence b is
    logical position seqlens[b] - T + t.  Returns a new cache array with those
    rows set to [c_new || kpe_new] (bit patterns copied); rows whose position
    has no mapped page are skipped."""
    out = np.array(kv_cache, dtype=np.uint16, copy=True)
    flat = out.reshape(-1, out.shape[-1])
    B, T, r = c_new.shape
    for b in range(B):
        for t in range(T):
            j = int(seqlens[b]) - T + t
            if j < 0:
                continue
            row = phys_row(block_table, b, j, page_size, out.shape[0])
            if row < 0:
                continue
            flat[row, :r] = c_new[b, t]
            flat[row, r:] = kpe_new[b, t]
    return out


def dims(case):
    """(d_nope, d_rope, d_v, r) read off the array shapes of a case."""
    return (case.q_nope.shape[-1], case.q_pe.shape[-1], case.w_uv.shape[1], case.w_uk.shape[2])


def normal_decode(case, pairs=None, scale=None, nthreads=None):
    """Normal-path (decompressed) decode in fp64.

    Returns ``(out [B,T,H,d_v] f64, lse [B,T,H] f64)``; only the (b, h) pairs
    listed in ``pairs`` (array [n,2]) are filled, the rest are NaN.  ``scale``
    None means 1/sqrt(d_nope + d_rope)."""
    B, T, H = case.B, case.T, case.H
    dn, dr, dv, r = dims(case)
    out = np.full((B, T, H, dv), np.nan)
    lse = np.full((B, T, H), np.nan)
    pr = None if pairs is None else _c(pairs, np.int32).reshape(-1, 2)
    st = lib().mlao_normal_decode(
        _p(_c(case.q_nope, np.uint16)), _p(_c(case.q_pe, np.uint16)),
        _p(_c(case.w_uk, np.uint16)), _p(_c(case.w_uv, np.uint16)),
        _p(_c(case.kv_cache, np.uint16)), case.num_blocks, case.page_size,
        _p(_c(case.block_table, np.int32)), case.max_blocks,
        _p(_c(case.seqlens, np.int32)), B, T, H, dn, dr, dv, r,
        float(scale) if scale else 0.0, _p(pr), 0 if pr is None else pr.shape[0],
        _p(out), _p(lse), nthreads or default_threads())
    _check(st, "normal_decode")
    return out, lse


def absorb(q_nope, w_uk):
    """q~[b,t,h,c] = sum_n q_nope[b,t,h,n] W_UK[h,n,c] in fp64 ("fold W_UK into the query")."""
    q = _c(q_nope, np.uint16)
    w = _c(w_uk, np.uint16)
    B, T, H, dn = q.shape
    r = w.shape[2]
    out = np.empty((B, T, H, r))
    _check(lib().mlao_absorb(_p(q), _p(w), B, T, H, dn, r, _p(out)), "absorb")
    return out


def unabsorb(latent, w_uv):
    """out[b,t,h,v] = sum_c latent[b,t,h,c] W_UV[h,v,c] in fp64 ("fold W_UV into the output")."""
    x = _c(latent, np.float64)
    w = _c(w_uv, np.uint16)
    B, T, H, r = x.shape
    dv = w.shape[1]
    out = np.empty((B, T, H, dv))
    _check(lib().mlao_unabsorb(_p(x), _p(w), B, T, H, r, dv, _p(out)), "unabsorb")
    return out


def split_plan(seqlens, num_splits, page_size):
    """Uniform split plan: (split_indptr [B+1], begin [B*S], end [B*S])."""
    sl = _c(seqlens, np.int32)
    B = sl.shape[0]
    ind = np.empty(B + 1, np.int32)
    beg = np.empty(B * num_splits, np.int32)
    end = np.empty(B * num_splits, np.int32)
    _check(lib().mlao_split_plan(_p(sl), B, num_splits, page_size, _p(ind), _p(beg), _p(end)),
           "split_plan")
    return ind, beg, end


def latent_attention(case, q_lat, scale=None, plan=None, pairs=None, nthreads=None):
    """Absorbed latent attention in fp64 over ``q_lat`` (float64 [B,T,H,r]).

    Without ``plan``: returns (latent [B,T,H,r], lse [B,T,H]).  With
    ``plan = split_plan(...)``: per-split partials (o [n,T,H,r], lse [n,T,H]).
    Rows of pairs not listed stay NaN.  ``scale`` None means
    1/sqrt(d_nope + d_rope) of the case."""
    B, T, H = case.B, case.T, case.H
    dn, dr, dv, r = dims(case)
    ql = _c(q_lat, np.float64)
    n_rows = B if plan is None else int(plan[0][-1])
    lat = np.full((n_rows, T, H, r), np.nan)
    lse = np.full((n_rows, T, H), np.nan)
    pr = None if pairs is None else _c(pairs, np.int32).reshape(-1, 2)
    ind, beg, end = (None, None, None) if plan is None else plan
    st = lib().mlao_latent_attention(
        _p(ql), _p(_c(case.q_pe, np.uint16)), _p(_c(case.kv_cache, np.uint16)),
        case.num_blocks, case.page_size, _p(_c(case.block_table, np.int32)), case.max_blocks,
        _p(_c(case.seqlens, np.int32)), B, T, H, dr, r,
        float(scale) if scale else 1.0 / math.sqrt(dn + dr),
        _p(ind), _p(beg), _p(end), _p(pr), 0 if pr is None else pr.shape[0],
        _p(lat), _p(lse), nthreads or default_threads())
    _check(st, "latent_attention")
    return lat, lse


def sparse_latent_attention(q_lat, q_pe, kv_cache, indices, topk_length, scale):
    """Sparse absorbed decode in fp64 (M5.8 0x0B, "Sparse indices are physical
    execution metadata"; 0x08, sparse mode of the runtime ABI).

    Query row (b, t, h) attends, without a causal mask, to the cache rows
    ``indices[b, t, k]`` -- flat physical row ids page * P + offset, read with
    no block table -- for k < min(topk_length[b], topk) (every k when
    ``topk_length`` is None), with the score of the dense path,
    (q~ . c + q_pe . k_pe) * scale.  A repeated id counts once per occurrence.
    Returns (latent [B,T,H,r], lse [B,T,H]); a row with no valid entry gives
    latent 0 and lse -inf."""
    ql = _c(q_lat, np.float64)
    qp = bf16_to_f64(q_pe)
    B, T, H, r = ql.shape
    rows = kv_cache.reshape(-1, kv_cache.shape[-1])
    topk = indices.shape[2]
    lat = np.zeros((B, T, H, r))
    lse = np.full((B, T, H), -np.inf)
    for b in range(B):
        n = topk if topk_length is None else max(0, min(int(topk_length[b]), topk))
        if n == 0:
            continue
        for t in range(T):
            sel = bf16_to_f64(rows[np.asarray(indices[b, t, :n], dtype=np.int64)])
            c, kpe = sel[:, :r], sel[:, r:]
            s = (ql[b, t] @ c.T + qp[b, t] @ kpe.T) * scale      # [H, n]
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            lat[b, t] = (e @ c) / z
            lse[b, t] = (m + np.log(z))[:, 0]
    return lat, lse


def merge(part_out, part_lse, split_indptr):
    """Exact LSE merge of normalised partials (M5.8 0x0C); returns (latent, lse)."""
    po = _c(part_out, np.float64)
    pl = _c(part_lse, np.float64)
    ind = _c(split_indptr, np.int32)
    B = ind.shape[0] - 1
    _, T, H, r = po.shape
    out = np.empty((B, T, H, r))
    lse = np.empty((B, T, H))
    _check(lib().mlao_merge(_p(po), _p(pl), _p(ind), B, T, H, r, _p(out), _p(lse)), "merge")
    return out, lse


# ---------------------------------------------------------------------------
# numpy float64 versions for tiny inputs (pins for the C code)

def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gather_rows(case):
    """Logical rows [B][L_b, 576] (float64) through the block table, written
    out token by token from the paged-address formula of M5.8 0x05."""
    P = case.page_size
    cache = bf16_to_f64(case.kv_cache).reshape(-1, case.kv_cache.shape[-1])
    rows = []
    for b in range(case.B):
        L = int(case.seqlens[b])
        idx = []
        for j in range(L):
            page, off = divmod(j, P)
            phys = int(case.block_table[b, page])
            assert phys >= 0
            idx.append(phys * P + off)
        rows.append(cache[np.array(idx, dtype=np.int64)])
    return rows


def expanded_attention_f64(case, scale=None):
    """Tiny-input Normal path in numpy: build K [L,H,d_nope+d_rope] and
    V [L,H,d_v] per sequence explicitly and run masked softmax attention."""
    dn, dr, dv, r = dims(case)
    scale = 1.0 / math.sqrt(dn + dr) if scale is None else scale
    qn = bf16_to_f64(case.q_nope)
    qp = bf16_to_f64(case.q_pe)
    wk = bf16_to_f64(case.w_uk)
    wv = bf16_to_f64(case.w_uv)
    B, T, H = case.B, case.T, case.H
    out = np.zeros((B, T, H, dv))
    lse = np.zeros((B, T, H))
    for b, rows in enumerate(gather_rows(case)):
        L = rows.shape[0]
        c = rows[:, :r]
        kpe = rows[:, r:]
        k_nope = np.einsum("hnc,jc->jhn", wk, c)
        K = np.concatenate([k_nope, np.broadcast_to(kpe[:, None, :], (L, H, dr))], axis=-1)
        V = np.einsum("hvc,jc->jhv", wv, c)
        Q = np.concatenate([qn[b], qp[b]], axis=-1)          # [T,H,192]
        s = np.einsum("thd,jhd->thj", Q, K) * scale
        for t in range(T):
            vis = L - T + t + 1
            s[t, :, vis:] = -np.inf
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=-1, keepdims=True)
        p = e / l
        out[b] = np.einsum("thj,jhv->thv", p, V)
        lse[b] = (m + np.log(l))[..., 0]
    return out, lse


# ---------------------------------------------------------------------------
# FP8 cache rows (M5.8 0x0B, "Exact 656-byte FP8 row"): 512 E4M3 latent
# values, four fp32 scales, 64 bf16 rope values; the decode dequantizes the
# latent to bf16 and attends in bf16.  Row bytes: [0, 512) the code of latent
# column c at byte c, [512, 528) scale g (little-endian fp32) of columns
# [128 g, 128 g + 128) -- one scale per 128 latent values --, [528, 656) rope.

def e4m3fn_decode(codes):
    """Values (float64) of E4M3 codes in the OCP FP8 encoding (the one called
    E4M3FN): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
    field 0 holds the subnormals (m / 8) * 2^-6; no infinities; exponent and
    mantissa all ones is NaN (largest finite magnitude 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_round(x):
    """float64 -> bf16 bits, round to nearest even in one step (no detour
    through float32, whose own rounding could land on a bf16 tie).  Finite
    nonzero magnitudes must lie in bf16's normal range; NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any((a != 0) & np.isfinite(a) & ((a < 2.0 ** -126) | (a >= 2.0 ** 128))):
        raise ValueError("bf16_round: value outside bf16's normal range")
    u = x.view(np.uint64)
    # keep 7 of the 52 fraction bits: add half an ulp minus one, plus the kept lsb
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    r = (u + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) >> drop << drop
    y = r.view(np.float64).astype(np.float32)      # exact: 8 significant bits
    bits = (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits)


def fp8_rows_to_bf16(kv_fp8):
    """Dequantize FP8 rows [..., 656] to bf16 rows [..., 576] (bits): latent
    column c becomes bf16(e4m3(code_c) * scale[c // 128]) -- the exact
    product, rounded once --, and the rope values are copied."""
    rows = np.asarray(kv_fp8, dtype=np.uint8)
    if rows.shape[-1] != 656:
        raise ValueError("an FP8 row is 656 bytes")
    lead = rows.shape[:-1]
    codes = rows[..., :512]
    scales = np.ascontiguousarray(rows[..., 512:528]).view("<f4").astype(np.float64)   # [..., 4]
    vals = e4m3fn_decode(codes).reshape(lead + (4, 128)) * scales[..., :, None]
    out = np.empty(lead + (576,), dtype=np.uint16)
    out[..., :512] = bf16_round(vals.reshape(lead + (512,)))
    out[..., 512:] = np.ascontiguousarray(rows[..., 528:]).view("<u2")
    return out


def fp8_case_as_bf16(fcase):
    """The decode case whose bf16 cache holds the dequantized FP8 rows: every
    oracle stage above then applies unchanged."""
    import dataclasses
    return dataclasses.replace(fcase.case, kv_cache=fp8_rows_to_bf16(fcase.kv_fp8))
