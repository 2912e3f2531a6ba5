"""Seeded synthetic workloads for the absorbed MLA decode path.

This module holds random draws and memory layout only -- none of the method's
arithmetic.  Both sides of every parity check (the CPU oracle and the HIP
library) are fed the arrays built here, so that neither side generates inputs
for the other.

Workload geometry follows the pages' statement of the problem:

* "MLA in full detail" (mlinterviewnotes), shapes table: kv_lora_rank 512,
  nope 128, rope 64, v_head 128, 128 heads (DeepSeek-V3).
* mlxcel "MLA absorbed decode", bytes table: DeepSeek-V2-Lite has 16 heads.
* "M5.8 - Multi-Head Latent Attention", 0x05 "Paged and ragged address
  translation": a logical token j lives at physical row
  block_table[b, j // P] * P + j % P of a paged cache of 576-wide rows.

Recipe (fixed draw order, numpy ``Generator(PCG64(seed))``):

1. seqlens (ragged workloads only): L_b = clip(round(exp(U(ln lo, ln hi))), lo, hi)
2. q_nope [B,T,H,128]  ~ N(0, 1)
3. q_pe   [B,T,H,64]   ~ N(0, 1)   (already rotated; RoPE itself is upstream)
4. W_UK   [H,128,512]  ~ N(0, 1/512)   (variance 1/512, std 1/sqrt(512))
5. W_UV   [H,128,512]  ~ N(0, 1/512)
6. physical block permutation (identity when ``permute`` is False)
7. cache rows [num_blocks, P, 576] ~ N(0, 1)

Every float32 draw is encoded to bfloat16 with round-to-nearest-even; arrays
of bf16 values are returned as their uint16 bit patterns.  With ``poison``
set, every cache row that no sequence may read (unused physical blocks, and
the rows of a sequence's last page at or past its length) is overwritten with
a bf16 quiet NaN so that any stray read surfaces as NaN in the output.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

R_LATENT = 512   # kv_lora_rank
D_ROPE = 64      # qk_rope_head_dim
D_NOPE = 128     # qk_nope_head_dim
D_V = 128        # v_head_dim
ROW = R_LATENT + D_ROPE  # 576 values per cached row
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Input values must be finite (they are normal draws here)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """Shape recipe of one decode workload."""
    name: str
    B: int
    T: int
    H: int
    L: int                      # per-sequence length (max length when ragged)
    page_size: int
    seed: int
    num_splits: int = 1
    permute: bool = True        # physical pages a seeded permutation
    ragged: Optional[tuple] = None   # (lo, hi) log-uniform lengths
    unused_frac: float = 0.0    # fraction of physical blocks left unused
    contiguous: bool = False    # one block holding the whole sequence
    lengths: Optional[tuple] = None  # explicit per-sequence lengths (overrides L)
    r: int = R_LATENT
    d_rope: int = D_ROPE
    d_nope: int = D_NOPE
    d_v: int = D_V
    w_std: Optional[float] = None    # weight std; default 1/sqrt(r)

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d["workload"] = d.pop("name")
        return d


# The five decode workloads (sizes as stated by the workload table of the
# pages' geometry; see module docstring for the distributions).
WORKLOADS = {
    "v2lite_tiny": Workload("v2lite_tiny", B=1, T=1, H=16, L=256, page_size=256,
                            seed=1001, permute=False, contiguous=True),
    "v3_b64_l4096": Workload("v3_b64_l4096", B=64, T=1, H=128, L=4096, page_size=64,
                             seed=1002),
    "v3_ragged_b128": Workload("v3_ragged_b128", B=128, T=1, H=128, L=16384, page_size=64,
                               seed=1003, ragged=(64, 16384), unused_frac=0.10),
    "v3_long_b4_l131072": Workload("v3_long_b4_l131072", B=4, T=1, H=128, L=131072,
                                   page_size=64, seed=1004, num_splits=64),
    "v3_mtp_b32_t4_h32": Workload("v3_mtp_b32_t4_h32", B=32, T=4, H=32, L=8192,
                                  page_size=64, seed=1005),
}


@dataclasses.dataclass
class Case:
    """Materialised inputs of one workload (host numpy arrays)."""
    wl: Workload
    q_nope: np.ndarray      # [B,T,H,128] uint16 (bf16 bits)
    q_pe: np.ndarray        # [B,T,H,64]  uint16
    w_uk: np.ndarray        # [H,128,512] uint16
    w_uv: np.ndarray        # [H,128,512] uint16
    kv_cache: np.ndarray    # [num_blocks,P,576] uint16
    block_table: np.ndarray  # [B,max_blocks] int32, -1 past each sequence's pages
    seqlens: np.ndarray     # [B] int32 (includes the T current rows)
    used_blocks: np.ndarray  # sorted physical ids that some sequence maps

    @property
    def B(self): return self.wl.B

    @property
    def T(self): return self.wl.T

    @property
    def H(self): return self.wl.H

    @property
    def page_size(self): return self.wl.page_size

    @property
    def num_blocks(self): return self.kv_cache.shape[0]

    @property
    def max_blocks(self): return self.block_table.shape[1]

    @property
    def max_seqlen(self): return int(self.seqlens.max())


def _normal_bf16(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def make_case(wl: Workload, poison: bool = True) -> Case:
    """Draw every input of ``wl`` from its seed (see module docstring)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B, T, H, P = wl.B, wl.T, wl.H, wl.page_size
    if wl.lengths is not None:
        seqlens = np.asarray(wl.lengths, dtype=np.int32)
        if seqlens.shape != (B,):
            raise ValueError("lengths must give one length per sequence")
    elif wl.ragged is not None:
        lo, hi = wl.ragged
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        seqlens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    else:
        seqlens = np.full(B, wl.L, dtype=np.int32)
    if (seqlens < T).any():
        raise ValueError("every sequence must hold at least its T current rows")
    r, dr, dn, dv = wl.r, wl.d_rope, wl.d_nope, wl.d_v
    q_nope = _normal_bf16(rng, (B, T, H, dn))
    q_pe = _normal_bf16(rng, (B, T, H, dr))
    std_w = wl.w_std if wl.w_std is not None else 1.0 / math.sqrt(r)
    w_uk = _normal_bf16(rng, (H, dn, r), std_w)
    w_uv = _normal_bf16(rng, (H, dv, r), std_w)

    pages = [(int(L) + P - 1) // P for L in seqlens]
    max_blocks = max((int(seqlens.max()) + P - 1) // P, 1)
    n_used = sum(pages)
    if wl.contiguous:
        if B != 1 or pages[0] != 1:
            raise ValueError("a contiguous workload is one sequence in one block")
        n_phys = 1
    elif wl.unused_frac > 0:
        n_phys = int(math.ceil(n_used / (1.0 - wl.unused_frac)))
    else:
        n_phys = n_used
    perm = rng.permutation(n_phys).astype(np.int32) if wl.permute else np.arange(n_phys, dtype=np.int32)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        for p in range(pages[b]):
            block_table[b, p] = perm[k]
            k += 1
    used = np.sort(perm[:n_used])

    kv_cache = _normal_bf16(rng, (n_phys, P, r + dr))
    if poison:
        mask = np.ones(n_phys, dtype=bool)
        mask[used] = False
        kv_cache[mask] = BF16_NAN
        for b in range(B):
            tail = int(seqlens[b]) % P
            if tail:
                kv_cache[block_table[b, pages[b] - 1], tail:, :] = BF16_NAN
    return Case(wl, q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seqlens, used)


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with some fields changed (reduced parity variants)."""
    return dataclasses.replace(wl, **changes)


def identity_paged_copy(case: Case) -> Case:
    """Same logical contents, physical pages laid out in (b, page) order.

    Used to check that the result depends only on the logical tokens, never on
    where the pages sit."""
    P = case.page_size
    B = case.B
    pages = [(int(L) + P - 1) // P for L in case.seqlens]
    n = sum(pages)
    cache = np.empty((n,) + case.kv_cache.shape[1:], dtype=np.uint16)
    table = np.full_like(case.block_table, -1)
    k = 0
    for b in range(B):
        for p in range(pages[b]):
            cache[k] = case.kv_cache[case.block_table[b, p]]
            table[b, p] = k
            k += 1
    return dataclasses.replace(case, kv_cache=cache, block_table=table,
                               used_blocks=np.arange(n, dtype=np.int32))


def normal_bf16(shape, seed, std=1.0) -> np.ndarray:
    """A standalone seeded N(0, std^2) bf16 array (stage inputs such as an
    absorbed query or a latent output given directly to one stage)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal_bf16(rng, shape, std)


def normal_f32(shape, seed, std=1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x * np.float32(std) if std != 1.0 else x


@dataclasses.dataclass
class Growth:
    """Inputs of a multi-step decode: ``base`` holds the cache before the first
    step (lengths ``base.seqlens``), with pages already mapped up to the
    lengths after the last step and every row at or past the current length
    poisoned; ``steps[s]`` holds that step's new cache rows and queries."""
    base: Case
    final_seqlens: np.ndarray
    steps: list   # dicts: c_new [B,T,r], kpe_new [B,T,d_R], q_lat [B,T,H,r], q_pe [B,T,H,d_R]


def make_growth(wl: Workload, n_steps: int, poison: bool = True) -> Growth:
    """``wl``'s lengths are those after ``n_steps`` decode steps of T tokens
    each; the sequences start ``n_steps * T`` rows shorter.  The new rows and
    per-step positional queries are N(0, 1) bf16 draws, the absorbed queries
    N(0, 1/4) (the spread of W_UK^T q_nope under the recipe: 128 terms of
    variance 1/512), from a second generator seeded from ``wl.seed`` (the
    base case uses the first, as in ``make_case``)."""
    case = make_case(wl, poison=poison)
    B, T, H, P = wl.B, wl.T, wl.H, wl.page_size
    grow = n_steps * T
    final = case.seqlens.copy()
    start = final - grow
    if (start < 0).any():
        raise ValueError("every sequence must hold the rows the steps append")
    if poison:
        for b in range(B):
            for j in range(int(start[b]), int(final[b])):
                page, off = divmod(j, P)
                case.kv_cache[case.block_table[b, page], off, :] = BF16_NAN
    case.seqlens = start.astype(np.int32)
    rng = np.random.Generator(np.random.PCG64(wl.seed + 0x5EED))
    steps = []
    for _ in range(n_steps):
        steps.append(dict(c_new=_normal_bf16(rng, (B, T, wl.r)),
                          kpe_new=_normal_bf16(rng, (B, T, wl.d_rope)),
                          q_lat=_normal_bf16(rng, (B, T, H, wl.r), 0.5),
                          q_pe=_normal_bf16(rng, (B, T, H, wl.d_rope))))
    return Growth(case, final.astype(np.int32), steps)


# Sparse decode workload: the headline geometry (B = 64, H = 128, page 64) over
# 32768-token contexts with 2048 rows selected per query token (top-k over
# physical rows, M5.8 0x0B).  The pages give no top-k value; 2048 of 32768 is
# one sixteenth of the context.
SPARSE_WORKLOADS = {
    "v3_sparse_b64_topk2048": Workload("v3_sparse_b64_topk2048", B=64, T=1, H=128, L=32768, page_size=64,
                                       seed=1006),
}
SPARSE_TOPK = {"v3_sparse_b64_topk2048": 2048}


@dataclasses.dataclass
class SparseCase:
    """Inputs of a sparse (top-k) decode: each query token (b, t) attends to the
    cache rows listed in ``indices[b, t, :]`` -- physical row ids
    page * P + offset -- of which the first ``topk_length[b]`` are valid."""
    wl: Workload
    q_lat: np.ndarray         # [B,T,H,r] uint16 (absorbed query, bf16 bits)
    q_pe: np.ndarray          # [B,T,H,d_R] uint16
    kv_cache: np.ndarray      # [num_blocks,P,r+d_R] uint16
    indices: np.ndarray       # [B,T,topk] int32
    topk_length: Optional[np.ndarray]  # [B] int32, or None (all topk valid)
    seqlens: np.ndarray       # [B] context lengths the positions were drawn from
    block_table: np.ndarray   # [B,max_blocks] (layout record; the sparse path reads no table)

    @property
    def B(self): return self.wl.B

    @property
    def T(self): return self.wl.T

    @property
    def H(self): return self.wl.H

    @property
    def topk(self): return self.indices.shape[2]

    @property
    def page_size(self): return self.wl.page_size

    @property
    def num_blocks(self): return self.kv_cache.shape[0]


def make_sparse(wl: Workload, topk: int, valid: Optional[tuple] = None, poison: bool = True,
                junk: bool = True, duplicates: bool = False, use_length: bool = True) -> SparseCase:
    """Draw a sparse decode workload (fixed draw order, ``Generator(PCG64(wl.seed))``):

    1. context lengths L_b as in ``make_case`` (explicit, ragged or ``wl.L``);
    2. q_lat [B,T,H,r] ~ N(0, 1/4) (the spread of W_UK^T q_nope under the recipe),
       q_pe [B,T,H,d_R] ~ N(0, 1);
    3. the paged layout: pages of each sequence at a seeded permutation of the
       physical blocks (as in ``make_case``);
    4. per query token (b, t): n_b = min(topk, L_b) distinct positions drawn
       uniformly without replacement from [0, L_b), in draw order, stored as
       physical rows block_table[b, j // P] * P + j % P (``duplicates`` then
       overwrites every fourth entry with the entry before it);
    5. the valid prefix: ``valid[b]`` when given, else n_b; entries past it are
       junk (-1 and 2^31 - 1 alternately) when ``junk`` is set, else repeat the
       last valid entry;
    6. the values of every selected row ~ N(0, 1); all other rows bf16 NaN
       (``poison``) or zero.

    ``use_length`` False passes no topk_length (every entry valid; then
    ``valid`` must be None and every L_b >= topk)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B, T, H, P = wl.B, wl.T, wl.H, wl.page_size
    if wl.lengths is not None:
        seqlens = np.asarray(wl.lengths, dtype=np.int32)
    elif wl.ragged is not None:
        lo, hi = wl.ragged
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        seqlens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int32)
    else:
        seqlens = np.full(B, wl.L, dtype=np.int32)
    r, dr = wl.r, wl.d_rope
    q_lat = _normal_bf16(rng, (B, T, H, r), 0.5)
    q_pe = _normal_bf16(rng, (B, T, H, dr))
    pages = [max((int(L) + P - 1) // P, 1) for L in seqlens]
    n_phys = sum(pages)
    perm = rng.permutation(n_phys).astype(np.int32) if wl.permute else np.arange(n_phys, dtype=np.int32)
    block_table = np.full((B, max(pages)), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        for p in range(pages[b]):
            block_table[b, p] = perm[k]
            k += 1
    nb = np.minimum(topk, seqlens).astype(np.int32)
    if valid is not None:
        nv = np.asarray(valid, dtype=np.int32)
        if nv.shape != (B,) or (nv > nb).any() or (nv < 0).any():
            raise ValueError("valid prefix lengths must lie in [0, min(topk, L_b)]")
    else:
        nv = nb
    if not use_length and (valid is not None or (nb < topk).any()):
        raise ValueError("without topk_length every entry must be valid")
    indices = np.empty((B, T, topk), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            pos = rng.choice(int(seqlens[b]), size=int(nb[b]), replace=False)
            phys = block_table[b, pos // P].astype(np.int64) * P + pos % P
            row = np.empty(topk, dtype=np.int64)
            row[:nb[b]] = phys
            if duplicates:
                for i in range(3, int(nv[b]), 4):
                    row[i] = row[i - 1]
            n = int(nv[b])
            if junk:
                row[n:] = np.where(np.arange(topk - n) % 2 == 0, -1, 2 ** 31 - 1)
            elif n > 0:
                row[n:] = row[n - 1]
            else:
                row[:] = 0
            indices[b, t] = row.astype(np.int32)
    fill = BF16_NAN if poison else np.uint16(0)
    kv_cache = np.full((n_phys, P, r + dr), fill, dtype=np.uint16)
    sel = np.unique(np.concatenate([indices[b, t, :nv[b]] for b in range(B) for t in range(T)]
                                   + [np.empty(0, np.int32)]).astype(np.int64))
    flat = kv_cache.reshape(-1, r + dr)
    flat[sel] = _normal_bf16(rng, (sel.shape[0], r + dr))
    return SparseCase(wl, q_lat, q_pe, kv_cache, indices, nv.astype(np.int32) if use_length else None,
                      seqlens, block_table)


# ---------------------------------------------------------------------------
# FP8 cache rows (M5.8 0x0B, "Exact 656-byte FP8 row": 512 one-byte E4M3
# latent values, four fp32 scales, 64 bf16 rope values per row).  The pages
# give the three segments and their sizes but not their order inside the row;
# they are stored in the order listed:
#     bytes [0, 512)    E4M3 code of latent column c at byte c
#     bytes [512, 528)  scale g (little-endian fp32) of columns [128 g, 128 g + 128)
#     bytes [528, 656)  the 64 rope values (bf16)
FP8_ROW_BYTES = 656
# The headline decode geometry (B = 64, 4096-token contexts, 128 heads, page 64)
# over FP8 rows.
FP8_WORKLOADS = {
    "v3_fp8_b64_l4096": Workload("v3_fp8_b64_l4096", B=64, T=1, H=128, L=4096, page_size=64, seed=1007),
}
FP8_NAN_CODE = np.uint8(0x7F)   # E4M3FN: exponent and mantissa all ones
F32_NAN_BITS = np.uint32(0x7FC00000)


@dataclasses.dataclass
class Fp8Case:
    """A decode workload over an FP8 cache: ``case`` supplies queries,
    weights, block table and lengths (its bf16 ``kv_cache`` is not read by
    the FP8 path); ``kv_fp8`` holds the rows."""
    case: Case
    kv_fp8: np.ndarray   # [num_blocks, P, 656] uint8


def make_fp8_case(wl: Workload, poison: bool = True) -> Fp8Case:
    """``make_case(wl)`` for everything but the latent part of the rows, then,
    from a second generator seeded ``wl.seed + 0xF8``:

    1. latent codes [num_blocks, P, 512]: magnitude code
       clip(round(N(108, 10^2)), 0, 126) (the 127 finite E4M3 magnitudes in
       increasing order; 108 encodes 96), sign bit uniform;
    2. scales [num_blocks, P, 4] = 2^U(-10, -6) rounded to float32;
    3. rope values: columns 512..575 of ``make_case``'s bf16 rows.

    With ``poison``, every row no sequence may read holds NaN codes, NaN
    scales and the bf16 NaN rope values of ``make_case``."""
    case = make_case(wl, poison=poison)
    if wl.r != 512 or wl.d_rope != 64:
        raise ValueError("the FP8 row holds 512 latent and 64 rope values")
    return Fp8Case(case, _fp8_rows(wl.seed, case.kv_cache, poison))


def _fp8_rows(seed: int, bf16_rows: np.ndarray, poison: bool) -> np.ndarray:
    """FP8 rows [num_blocks, P, 656] for a pool whose bf16 rows are ``bf16_rows``:
    codes and scales drawn from ``Generator(PCG64(seed + 0xF8))`` (see
    ``make_fp8_case``), rope values copied from the bf16 rows; with ``poison``,
    rows whose bf16 latent is NaN get NaN codes and NaN scales."""
    rng = np.random.Generator(np.random.PCG64(seed + 0xF8))
    nb, P, _ = bf16_rows.shape
    r = 512
    mag = np.clip(np.rint(rng.normal(108.0, 10.0, size=(nb, P, r))), 0, 126).astype(np.uint8)
    sign = rng.integers(0, 2, size=(nb, P, r), dtype=np.uint8) << np.uint8(7)
    codes = mag | sign
    scales = np.exp2(rng.uniform(-10.0, -6.0, size=(nb, P, 4))).astype(np.float32)
    rows = np.empty((nb, P, FP8_ROW_BYTES), dtype=np.uint8)
    rows[:, :, :512] = codes
    rows[:, :, 512:528] = scales.astype("<f4").view(np.uint8).reshape(nb, P, 16)
    rows[:, :, 528:] = np.ascontiguousarray(bf16_rows[:, :, r:]).astype("<u2").view(np.uint8).reshape(nb, P, 128)
    if poison:
        dead = np.isnan(bf16_bits_to_f32(bf16_rows[:, :, r]))   # rows the bf16 generator poisoned
        rows[dead, :512] = FP8_NAN_CODE
        rows[dead, 512:528] = np.full(4, F32_NAN_BITS, dtype="<u4").view(np.uint8)
    return rows


@dataclasses.dataclass
class SparseFp8Case:
    """A sparse decode workload over FP8 rows: ``sparse`` supplies queries,
    index rows and valid prefixes (its bf16 ``kv_cache`` is not read by the
    FP8 path); ``kv_fp8`` holds the pool's rows."""
    sparse: SparseCase
    kv_fp8: np.ndarray   # [num_blocks, P, 656] uint8


def make_sparse_fp8(wl: Workload, topk: int, **kw) -> SparseFp8Case:
    """``make_sparse(wl, topk, **kw)``, then the pool's rows as FP8 rows drawn as
    in ``make_fp8_case`` (codes, scales; rope values from the bf16 rows; rows no
    index selects are NaN when ``poison``)."""
    sc = make_sparse(wl, topk, **kw)
    return SparseFp8Case(sc, _fp8_rows(wl.seed, sc.kv_cache, kw.get("poison", True)))
