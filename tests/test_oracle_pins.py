"""Pins of the CPU oracle to facts fixed outside itself (no GPU).

What pins what:
* the identity "MLA in full detail" states for the absorbed form (expanded and
  absorbed scores and outputs agree; scale (key + rope)^-0.5), checked on this
  project's own draws against a direct matrix evaluation;
* an independent numpy Normal path and PyTorch's float64
  scaled_dot_product_attention on explicitly expanded K/V (library special case);
* associativity: absorbed mirror == Normal path (M5.8 0x04);
* closed forms: one visible key, zero queries (uniform weights, lse = ln n),
  identical rows;
* invariants: split merge == unsplit (M5.8 0x0C), page permutation invariance
  (M5.8 0x05), determinism across thread counts;
* negative controls: the mistakes M5.8 0x04 and mlxcel Stage 2 name must fail
  the product tolerance.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import costs


def tol(ref):
    """Product tolerance: max|err| <= 1e-2 * max|ref| + 1e-3."""
    return 1e-2 * float(np.nanmax(np.abs(ref))) + 1e-3


def tiny(seed, B=2, T=1, H=3, lengths=None, L=37, P=8, r=16, dr=4, dn=8, dv=6,
         permute=True, unused=0.0, w_std=None):
    wl = synth.Workload("tiny", B=B, T=T, H=H, L=L, page_size=P, seed=seed,
                        permute=permute, unused_frac=unused,
                        lengths=lengths, r=r, d_rope=dr, d_nope=dn, d_v=dv, w_std=w_std)
    return synth.make_case(wl)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# 1. the associativity identity the absorbed form rests on

def test_absorbed_equals_expanded_attention_on_a_tiny_head():
    """"MLA in full detail" (the absorbed form and its numpy parity check)
    states that folding the key up-projection into the query leaves every
    score unchanged and folding the value up-projection behind the softmax
    leaves the output unchanged.  Checked with this project's own draws: four
    query tokens against seven cached rows of latent rank 6 (key part 3,
    value 5, rope 2).  A direct matrix evaluation of the expanded attention
    (explicit per-key K = [W_UK c || k_pe] and V = W_UV c), the oracle's
    Normal path and its absorbed mirror agree to 1e-12."""
    rng = np.random.default_rng(2024)
    n_q, n_k, rank, d_key, d_val, d_rope = 4, 7, 6, 3, 5, 2

    def draw(*shape):
        return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))

    lat_b, qn_b, qp_b, kp_b = draw(n_k, rank), draw(n_q, d_key), draw(n_q, d_rope), draw(n_k, d_rope)
    wk_b, wv_b = draw(d_key, rank), draw(d_val, rank)          # W_UK[h], W_UV[h] of the one head
    lat, qn, qp, kp, wk, wv = (oracle.bf16_to_f64(x) for x in (lat_b, qn_b, qp_b, kp_b, wk_b, wv_b))

    keys = np.concatenate([lat @ wk.T, kp], axis=1)           # [n_k, d_key + d_rope]
    vals = lat @ wv.T                                          # [n_k, d_val]
    qry = np.concatenate([qn, qp], axis=1)
    scores = qry @ keys.T / np.sqrt(d_key + d_rope)
    wts = np.exp(scores - scores.max(1, keepdims=True))
    wts /= wts.sum(1, keepdims=True)
    ref_out = wts @ vals
    ref_lse = scores.max(1) + np.log(np.exp(scores - scores.max(1, keepdims=True)).sum(1))
    # the identity itself, both sides
    np.testing.assert_allclose((qn @ wk) @ lat.T, qn @ keys[:, :d_key].T, atol=1e-12)
    np.testing.assert_allclose((wts @ lat) @ wv.T, ref_out, atol=1e-12)

    # the same numbers through the oracle: every query token its own sequence
    # (T = 1) of length n_k, one page of 8 rows
    from types import SimpleNamespace
    rows = np.concatenate([lat_b, kp_b], axis=1)
    case = SimpleNamespace(
        B=n_q, T=1, H=1, page_size=8, num_blocks=1, max_blocks=1,
        q_nope=qn_b.reshape(n_q, 1, 1, d_key), q_pe=qp_b.reshape(n_q, 1, 1, d_rope),
        w_uk=wk_b.reshape(1, d_key, rank), w_uv=wv_b.reshape(1, d_val, rank),
        kv_cache=np.concatenate([rows, np.zeros((8 - n_k, rank + d_rope), np.uint16)]).reshape(1, 8, -1),
        block_table=np.zeros((n_q, 1), np.int32), seqlens=np.full(n_q, n_k, np.int32))
    out, lse = oracle.normal_decode(case)
    np.testing.assert_allclose(out[:, 0, 0, :], ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, 0, 0], ref_lse, rtol=0, atol=1e-12)
    ql = oracle.absorb(case.q_nope, case.w_uk)
    np.testing.assert_allclose(ql[:, 0, 0, :], qn @ wk, atol=1e-12)
    lat_out, lse2 = oracle.latent_attention(case, ql)
    np.testing.assert_allclose(lat_out[:, 0, 0, :], wts @ lat, atol=1e-12)
    np.testing.assert_allclose(oracle.unabsorb(lat_out, case.w_uv)[:, 0, 0, :], ref_out, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


def test_page_causal_pair_count_from_uniform_weights():
    """With zero queries every visible key gets the same weight, so exp(lse)
    counts the visible keys of each query row.  3 new tokens after a prefix of
    5 give 3*5 + 3*4/2 = 21 pairs (the causal visibility of "MLA in full detail",
    Step 3)."""
    case = tiny(3, B=1, T=3, H=2, lengths=(8,))
    case.q_nope[:] = 0
    case.q_pe[:] = 0
    _, lse = oracle.normal_decode(case)
    counts = np.exp(lse)
    assert np.allclose(counts[0, :, 0], [6, 7, 8], atol=1e-12)
    assert round(float(counts[..., 0].sum())) == 21 == costs.causal_pairs(3, 5)


def test_causal_pairs_mtp_geometry_formula():
    """Pairs of T new tokens over lengths L_b: sum_b H * (T*(L_b-T) + T*(T+1)/2);
    checked on a reduced multi-token case against the oracle's uniform weights."""
    case = tiny(4, B=3, T=4, H=2, lengths=(9, 23, 4), P=4)
    case.q_nope[:] = 0
    case.q_pe[:] = 0
    _, lse = oracle.normal_decode(case)
    total = float(np.exp(lse).sum())
    want = sum(2 * costs.causal_pairs(4, int(L) - 4) for L in case.seqlens)
    assert abs(total - want) < 1e-9
    # the 32 x 4 x 32 x 8192 multi-token workload: 33,548,288 visible pairs
    assert 32 * 32 * costs.causal_pairs(4, 8192 - 4) == 33_548_288


# --------------------------------------------------------------------------
# 2. independent implementations of the same definition

@pytest.mark.parametrize("seed", [11, 12, 13])
def test_normal_matches_numpy_expanded(seed):
    case = tiny(seed, B=3, T=2, H=4, lengths=(37, 9, 20), P=8, unused=0.2)
    out, lse = oracle.normal_decode(case)
    ref, ref_lse = oracle.expanded_attention_f64(case)
    assert rel(out, ref) < 1e-12
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def test_normal_matches_torch_sdpa_float64():
    """Library special case: the Normal path is exactly MHA over expanded K/V
    (M5.8 0x05 naive path), so torch's float64 SDPA must reproduce it."""
    case = tiny(21, B=2, T=3, H=4, lengths=(30, 13), P=8)
    out, _ = oracle.normal_decode(case)
    qn = oracle.bf16_to_f64(case.q_nope)
    qp = oracle.bf16_to_f64(case.q_pe)
    wk = oracle.bf16_to_f64(case.w_uk)
    wv = oracle.bf16_to_f64(case.w_uv)
    dn, dr, dv, r = oracle.dims(case)
    for b, rows in enumerate(oracle.gather_rows(case)):
        L = rows.shape[0]
        c, kpe = rows[:, :r], rows[:, r:]
        K = np.concatenate([np.einsum("hnc,jc->hjn", wk, c),
                            np.broadcast_to(kpe[None], (case.H, L, dr))], axis=-1)
        V = np.einsum("hvc,jc->hjv", wv, c)
        Q = np.concatenate([qn[b], qp[b]], axis=-1).transpose(1, 0, 2)   # [H,T,192']
        mask = np.zeros((case.T, L), dtype=bool)
        for t in range(case.T):
            mask[t, : L - case.T + t + 1] = True
        got = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q), torch.from_numpy(np.ascontiguousarray(K)),
            torch.from_numpy(V), attn_mask=torch.from_numpy(mask),
            scale=1.0 / math.sqrt(dn + dr)).numpy()
        assert rel(out[b].transpose(1, 0, 2), got) < 1e-12


@pytest.mark.parametrize("T", [1, 3])
def test_absorbed_mirror_equals_normal(T):
    """Associativity (M5.8 0x04; mlxcel: "without changing the arithmetic")."""
    case = tiny(31 + T, B=3, T=T, H=5, lengths=(40, 17, 5), P=8)
    out, lse = oracle.normal_decode(case)
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, lse2 = oracle.latent_attention(case, ql)
    out2 = oracle.unabsorb(lat, case.w_uv)
    assert rel(out2, out) < 1e-12
    assert np.max(np.abs(lse2 - lse)) < 1e-12


def test_absorbed_mirror_equals_normal_real_dims():
    case = synth.make_case(synth.scaled(synth.WORKLOADS["v3_b64_l4096"], B=2, L=100, H=4, seed=5))
    out, lse = oracle.normal_decode(case)
    lat, lse2 = oracle.latent_attention(case, oracle.absorb(case.q_nope, case.w_uk))
    assert rel(oracle.unabsorb(lat, case.w_uv), out) < 1e-12
    assert np.max(np.abs(lse2 - lse)) < 1e-12


# --------------------------------------------------------------------------
# 3. closed-form special cases

def test_single_visible_key_returns_its_value():
    case = tiny(41, B=2, T=1, H=3, lengths=(1, 1), P=8)
    out, lse = oracle.normal_decode(case)
    dn, dr, dv, r = oracle.dims(case)
    wk = oracle.bf16_to_f64(case.w_uk)
    wv = oracle.bf16_to_f64(case.w_uv)
    for b, rows in enumerate(oracle.gather_rows(case)):
        c, kpe = rows[0, :r], rows[0, r:]
        for h in range(case.H):
            np.testing.assert_allclose(out[b, 0, h], wv[h] @ c, rtol=0, atol=1e-13)
            s = (oracle.bf16_to_f64(case.q_nope[b, 0, h]) @ (wk[h] @ c)
                 + oracle.bf16_to_f64(case.q_pe[b, 0, h]) @ kpe) / math.sqrt(dn + dr)
            assert abs(lse[b, 0, h] - s) < 1e-12


def test_zero_query_gives_mean_of_visible_latents():
    case = tiny(42, B=2, T=2, H=2, lengths=(19, 6), P=4)
    case.q_nope[:] = 0
    case.q_pe[:] = 0
    lat, lse = oracle.latent_attention(case, np.zeros(case.q_nope.shape[:3] + (case.w_uk.shape[2],)))
    dn, dr, dv, r = oracle.dims(case)
    for b, rows in enumerate(oracle.gather_rows(case)):
        L = rows.shape[0]
        for t in range(case.T):
            vis = L - case.T + t + 1
            np.testing.assert_allclose(lat[b, t, 0], rows[:vis, :r].mean(0), atol=1e-13)
            assert abs(lse[b, t, 1] - math.log(vis)) < 1e-13


def test_identical_rows_return_that_row_for_any_query():
    """Weights sum to one: with every visible latent equal to c, out_latent == c."""
    case = tiny(43, B=1, T=2, H=3, lengths=(21,), P=8)
    row = case.kv_cache[case.block_table[0, 0], 0].copy()
    for p in range(3):
        case.kv_cache[case.block_table[0, p], :] = row
    dn, dr, dv, r = oracle.dims(case)
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, _ = oracle.latent_attention(case, ql)
    c = oracle.bf16_to_f64(row[:r])
    np.testing.assert_allclose(lat[0], np.broadcast_to(c, lat[0].shape), atol=1e-13, rtol=0)


# --------------------------------------------------------------------------
# 4. invariants

@pytest.mark.parametrize("S", [1, 2, 3, 7, 64])
def test_split_merge_equals_unsplit(S):
    """M5.8 0x0C exact merge; chunks cut at page multiples, empty ones allowed."""
    case = tiny(51, B=3, T=2, H=3, lengths=(57, 9, 33), P=8)
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, lse = oracle.latent_attention(case, ql)
    plan = oracle.split_plan(case.seqlens, S, case.page_size)
    ind, beg, end = plan
    assert ind[-1] == 3 * S
    if S == 64:
        assert (beg == end).any()            # empty trailing splits exist
    po, pl = oracle.latent_attention(case, ql, plan=plan)
    m, ml = oracle.merge(po, pl, ind)
    assert not np.isnan(m).any()
    assert rel(m, lat) < 1e-12
    assert np.max(np.abs(ml - lse)) < 1e-12


def test_split_plan_rule():
    ind, beg, end = oracle.split_plan(np.array([131072, 100, 64], np.int32), 64, 64)
    assert list(ind) == [0, 64, 128, 192]
    assert beg[1] == 2048 and end[63] == 131072           # 64 chunks of 2048 tokens
    assert beg[64] == 0 and end[64] == 64 and beg[65] == 64 and end[65] == 100
    assert (beg[66:128] == 100).all() and (end[66:128] == 100).all()


def test_page_permutation_is_invisible_bitwise():
    case = tiny(61, B=3, T=2, H=2, lengths=(40, 17, 25), P=8, unused=0.3)
    ident = synth.identity_paged_copy(case)
    assert not np.array_equal(case.block_table, ident.block_table)
    a, la = oracle.normal_decode(case)
    b, lb = oracle.normal_decode(ident)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_thread_count_does_not_change_bits():
    case = tiny(62, B=2, T=2, H=4, lengths=(30, 19), P=8)
    a, la = oracle.normal_decode(case, nthreads=1)
    b, lb = oracle.normal_decode(case, nthreads=5)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_pairs_subset_matches_full_run():
    case = tiny(63, B=3, T=1, H=4, lengths=(22, 9, 30), P=8)
    full, lf = oracle.normal_decode(case)
    pairs = np.array([[2, 3], [0, 1]], np.int32)
    part, lp = oracle.normal_decode(case, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(part[b, :, h], full[b, :, h])
    assert np.isnan(part[1]).all()


def test_paged_address_formula():
    """M5.8 0x05: physical(j) = block_table[b, j // P] * P + j % P; a negative
    page entry (or one past the pool) is rejected."""
    bt = np.array([[3, 1, -1], [0, 2, 4]], np.int32)
    assert oracle.phys_row(bt, 0, 0, 4, 5) == 12
    assert oracle.phys_row(bt, 0, 5, 4, 5) == 5
    assert oracle.phys_row(bt, 0, 8, 4, 5) == -1
    assert oracle.phys_row(bt, 1, 11, 4, 5) == 4 * 4 + 3
    assert oracle.phys_row(bt, 1, 11, 4, 4) == -1   # pool of 4 blocks: id 4 is out of range


def test_bad_block_table_is_an_error():
    case = tiny(64, B=2, T=1, H=2, lengths=(20, 12), P=8)
    case.block_table[1, 1] = -1
    with pytest.raises(RuntimeError):
        oracle.normal_decode(case)


# --------------------------------------------------------------------------
# 5. the input recipe

def test_score_variance_is_one_under_the_recipe():
    """Reading N(0, 1/512) as variance 1/512 makes the scaled scores unit
    variance: 128 * (1/512) * 512 + 64 = 192, divided by 192."""
    case = synth.make_case(synth.scaled(synth.WORKLOADS["v3_b64_l4096"], B=2, L=512, seed=77))
    ql = oracle.absorb(case.q_nope, case.w_uk)          # [2,1,128,512]
    rows = oracle.gather_rows(case)
    s = []
    for b in range(2):
        c, kpe = rows[b][:, :512], rows[b][:, 512:]
        qp = oracle.bf16_to_f64(case.q_pe[b, 0])
        s.append((ql[b, 0] @ c.T + qp @ kpe.T) / math.sqrt(192))
    var = float(np.var(np.concatenate([x.ravel() for x in s])))
    assert abs(var - 1.0) < 0.05


# --------------------------------------------------------------------------
# 6. negative controls: each planted mistake must fail the product tolerance

def _real_small():
    return synth.make_case(synth.scaled(synth.WORKLOADS["v3_b64_l4096"], B=2, T=2, L=24, H=8,
                                        page_size=16, seed=91))


def _mirror(case, scale=None, softmax_axis="keys", share_heads=False, flip_wuv=False,
            extra_key=False):
    """numpy absorbed decode with one selectable mistake (CPU only)."""
    dn, dr, dv, r = oracle.dims(case)
    scale = 1.0 / math.sqrt(dn + dr) if scale is None else scale
    ql = oracle.absorb(case.q_nope, case.w_uk)
    qp = oracle.bf16_to_f64(case.q_pe)
    wv = oracle.bf16_to_f64(case.w_uv)
    if flip_wuv:
        wv = wv[:, :, ::-1]
    out = np.zeros((case.B, case.T, case.H, dv))
    cache = oracle.bf16_to_f64(case.kv_cache).reshape(-1, r + dr)
    for b in range(case.B):
        L = int(case.seqlens[b])
        n = L + 1 if extra_key else L
        idx = [int(case.block_table[b, j // case.page_size]) * case.page_size + j % case.page_size
               for j in range(n)]
        rows = cache[idx]
        c, kpe = rows[:, :r], rows[:, r:]
        s = (np.einsum("thc,jc->thj", ql[b], c) + np.einsum("thr,jr->thj", qp[b], kpe)) * scale
        for t in range(case.T):
            s[t, :, n - case.T + t + 1:] = -np.inf
        if softmax_axis == "keys":
            p = np.exp(s - s.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
        else:   # over heads
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            p = np.nan_to_num(p)
        lat = np.einsum("thj,jc->thc", p, c)
        if share_heads:
            lat[:] = lat.mean(1, keepdims=True)
        out[b] = np.einsum("thc,hvc->thv", lat, wv)
    return out


@pytest.fixture(scope="module")
def small_ref():
    case = _real_small()
    out, _ = oracle.normal_decode(case)
    return case, out


def _fails(got, ref):
    err = np.max(np.abs(got - ref)) if not np.isnan(got).any() else np.inf
    return err > tol(ref)


def test_mirror_without_mistake_passes(small_ref):
    case, ref = small_ref
    assert not _fails(_mirror(case), ref)


@pytest.mark.parametrize("mistake", [
    dict(softmax_axis="heads"),          # M5.8 0x04 bug 1
    dict(share_heads=True),              # M5.8 0x04 bug 2
    dict(flip_wuv=True),                 # M5.8 0x04 bug 3 (d_c axis differs between factors)
    dict(scale=1.0 / math.sqrt(576)),    # "MLA in full detail": latent-width scale changes the function
    dict(extra_key=True),                # reading past the visible length (poisoned row)
])
def test_negative_control_fails(small_ref, mistake):
    case, ref = small_ref
    assert _fails(_mirror(case, **mistake), ref)


def test_averaging_partials_fails():
    """M5.8 0x0C: averaging split outputs is wrong."""
    case = _real_small()
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, _ = oracle.latent_attention(case, ql)
    plan = oracle.split_plan(case.seqlens, 2, case.page_size)
    po, pl = oracle.latent_attention(case, ql, plan=plan)
    avg = po.reshape(case.B, 2, *po.shape[1:]).mean(1)
    assert _fails(avg, lat)


def test_log2_lse_units_fail():
    """mlxcel Stage 2: mixing log2 and natural-log LSE units merges into a
    plausible but wrong average; the merge must see natural logs."""
    case = _real_small()
    ql = oracle.absorb(case.q_nope, case.w_uk)
    lat, _ = oracle.latent_attention(case, ql)
    plan = oracle.split_plan(case.seqlens, 2, case.page_size)
    po, pl = oracle.latent_attention(case, ql, plan=plan)
    good, _ = oracle.merge(po, pl, plan[0])
    assert not _fails(good, lat)
    wrong, _ = oracle.merge(po, pl * math.log2(math.e), plan[0])
    assert _fails(wrong, lat)


# --------------------------------------------------------------------------
# 7. cache append of a decode step (M5.8 0x05)

def _chunked_rebuild(case, T, shift=0):
    """Start from an all-NaN pool with the case's block table and append the
    case's logical rows T at a time (``shift`` offsets the lengths passed)."""
    rows = oracle.gather_rows(case)     # logical rows through divmod, not phys_row
    pool = np.full_like(case.kv_cache, synth.BF16_NAN)
    L = case.seqlens.astype(np.int64)
    r = case.kv_cache.shape[-1] - case.q_pe.shape[-1]
    for s in range(int(math.ceil(L.max() / T))):
        cur = np.minimum(T * (s + 1), L)   # a finished sequence re-appends its last rows
        c_new = np.empty((case.B, T, r), np.uint16)
        k_new = np.empty((case.B, T, case.kv_cache.shape[-1] - r), np.uint16)
        for b in range(case.B):
            lb = rows[b]
            for t in range(T):
                j = int(cur[b]) - T + t
                v = synth.f32_to_bf16_bits(lb[max(j, 0)].astype(np.float32))
                c_new[b, t], k_new[b, t] = v[:r], v[r:]
        pool = oracle.append_rows(pool, case.block_table, (cur + shift).astype(np.int32),
                                  c_new, k_new, case.page_size)
    return pool


@pytest.mark.parametrize("T", [1, 3])
def test_append_rebuilds_the_paged_cache(T):
    """Appending every sequence's rows in steps of T tokens, each at
    seqlens - T + t, reproduces the paged pool bit for bit (poisoned tails and
    unused blocks stay NaN): the append position agrees with the read-side
    address formula."""
    case = tiny(301, B=3, H=2, lengths=(36, 21, 9), P=8, unused=0.2)
    assert np.array_equal(_chunked_rebuild(case, T), case.kv_cache)


@pytest.mark.parametrize("shift", [-1, 1])
def test_append_off_by_one_position_fails(shift):
    """Negative control: lengths that exclude (or double count) the new rows
    put them one position off, which the rebuild detects."""
    case = tiny(302, B=3, H=2, lengths=(36, 21, 9), P=8)
    assert not np.array_equal(_chunked_rebuild(case, 3, shift), case.kv_cache)


def test_append_skips_unmapped_positions():
    bt = np.array([[1, -1]], np.int32)
    pool = np.zeros((2, 4, 6), np.uint16)
    c = np.full((1, 2, 4), 7, np.uint16)
    k = np.full((1, 2, 2), 9, np.uint16)
    out = oracle.append_rows(pool, bt, np.array([5], np.int32), c, k, 4)
    # positions 3 (block 1, offset 3) and 4 (page 1 unmapped: skipped)
    assert (out[1, 3] == [7, 7, 7, 7, 9, 9]).all()
    out[1, 3] = 0
    assert not out.any()


def _explicit_latent(ql, qp, rows, T, scale):
    """numpy latent attention over explicit logical rows (causal over T)."""
    r = ql.shape[-1]
    c, kpe = rows[:, :r], rows[:, r:]
    n = rows.shape[0]
    s = (np.einsum("thc,jc->thj", ql, c) + np.einsum("thd,jd->thj", qp, kpe)) * scale
    for t in range(T):
        s[t, :, n - T + t + 1:] = -np.inf
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    return np.einsum("thj,jc->thc", p, c)


@pytest.mark.parametrize("T", [1, 2])
def test_multistep_decode_sees_the_appended_rows(T):
    """Three decode steps: after each append the oracle's paged latent
    attention equals attention over the explicit concatenation of the
    starting rows and every row appended so far."""
    wl = synth.Workload("grow", B=3, T=T, H=2, L=0, page_size=8, seed=303,
                        lengths=(19, 8 + 3 * T, 3 * T), r=16, d_rope=4, d_nope=8, d_v=6)
    g = synth.make_growth(wl, 3)
    case = g.base
    start = oracle.gather_rows(case)
    cache = case.kv_cache
    scale = 1.0 / math.sqrt(8 + 4)
    for s, st in enumerate(g.steps):
        lens = (g.base.seqlens + (s + 1) * T).astype(np.int32)
        cache = oracle.append_rows(cache, case.block_table, lens, st["c_new"], st["kpe_new"],
                                   case.page_size)
        cs = dataclasses.replace(case, kv_cache=cache, seqlens=lens, q_pe=st["q_pe"])
        ql = oracle.bf16_to_f64(st["q_lat"])
        lat, _ = oracle.latent_attention(cs, ql, scale=scale)
        for b in range(wl.B):
            new = [np.concatenate([oracle.bf16_to_f64(g.steps[k]["c_new"][b]),
                                   oracle.bf16_to_f64(g.steps[k]["kpe_new"][b])], -1)
                   for k in range(s + 1)]
            rows = np.concatenate([start[b]] + new, 0)
            ref = _explicit_latent(ql[b], oracle.bf16_to_f64(st["q_pe"][b]), rows, T, scale)
            assert np.allclose(lat[b], ref, rtol=1e-12, atol=1e-12)
    assert np.array_equal(g.final_seqlens, g.base.seqlens + 3 * T)


# --------------------------------------------------------------------------
# 8. sparse (top-k) decode (M5.8 0x0B)

def _sparse_tiny(seed, T=1, lengths=(40, 9), topk=12, **kw):
    wl = synth.Workload("sp", B=len(lengths), T=T, H=3, L=0, page_size=8, seed=seed,
                        lengths=lengths, r=16, d_rope=4, d_nope=8, d_v=6)
    return synth.make_sparse(wl, topk, **kw)


def _sparse(sc, scale=0.3, indices=None, lengths="case"):
    return oracle.sparse_latent_attention(oracle.bf16_to_f64(sc.q_lat), sc.q_pe, sc.kv_cache,
                                          sc.indices if indices is None else indices,
                                          sc.topk_length if lengths == "case" else lengths, scale)


def test_sparse_full_selection_equals_dense():
    """Selecting every position of the sequence, as physical rows through the
    block table, is dense decode: the sparse oracle (numpy) agrees with the
    dense one (the C oracle) for T = 1."""
    case = tiny(401, B=3, T=1, H=3, lengths=(37, 8, 20), P=8)
    ql = synth.normal_bf16((3, 1, 3, 16), 402, std=0.5)
    topk = 40
    idx = np.full((3, 1, topk), -1, np.int32)
    for b in range(3):
        for j in range(int(case.seqlens[b])):
            idx[b, 0, j] = oracle.phys_row(case.block_table, b, j, case.page_size, case.num_blocks)
    scale = 1.0 / math.sqrt(8 + 4)
    got, got_lse = oracle.sparse_latent_attention(oracle.bf16_to_f64(ql), case.q_pe, case.kv_cache, idx,
                                                  case.seqlens, scale)
    ref, ref_lse = oracle.latent_attention(case, oracle.bf16_to_f64(ql), scale=scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(got_lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_sparse_order_of_selection_is_irrelevant():
    sc = _sparse_tiny(403, T=2)
    lat, lse = _sparse(sc)
    idx = sc.indices.copy()
    rng = np.random.default_rng(5)
    for b in range(sc.B):
        for t in range(sc.T):
            n = int(sc.topk_length[b])
            idx[b, t, :n] = rng.permutation(idx[b, t, :n])
    lat2, lse2 = _sparse(sc, indices=idx)
    assert np.allclose(lat, lat2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lse2, rtol=1e-12, atol=1e-13)


def test_sparse_entries_past_the_valid_prefix_are_ignored():
    sc = _sparse_tiny(404, T=2, valid=(5, 9))
    lat, lse = _sparse(sc)
    idx = sc.indices.copy()
    idx[0, :, 5:] = 3
    idx[1, :, 9:] = 0
    lat2, lse2 = _sparse(sc, indices=idx)
    assert np.array_equal(lat, lat2) and np.array_equal(lse, lse2)


def test_sparse_single_key_and_empty_selection():
    """One valid entry: the latent is that row's c and lse its score; no valid
    entry: latent 0 and lse -inf."""
    sc = _sparse_tiny(405, valid=(1, 0))
    lat, lse = _sparse(sc)
    row = oracle.bf16_to_f64(sc.kv_cache.reshape(-1, 20)[sc.indices[0, 0, 0]])
    ql = oracle.bf16_to_f64(sc.q_lat[0, 0])
    qp = oracle.bf16_to_f64(sc.q_pe[0, 0])
    for h in range(sc.H):
        assert np.allclose(lat[0, 0, h], row[:16], rtol=0, atol=0)
        assert math.isclose(lse[0, 0, h], 0.3 * (ql[h] @ row[:16] + qp[h] @ row[16:]), rel_tol=1e-12)
    assert (lat[1] == 0).all() and np.isneginf(lse[1]).all()


def test_sparse_repeated_entry_counts_twice():
    """Selecting rows (a, a, b): softmax weights 2 e^{s_a} and e^{s_b}."""
    sc = _sparse_tiny(406, lengths=(40,), topk=3, use_length=False)
    idx = sc.indices.copy()
    idx[0, 0, 1] = idx[0, 0, 0]
    lat, lse = _sparse(sc, indices=idx, lengths=None)
    rows = oracle.bf16_to_f64(sc.kv_cache.reshape(-1, 20)[idx[0, 0, [0, 2]].astype(np.int64)])
    ql = oracle.bf16_to_f64(sc.q_lat[0, 0])
    qp = oracle.bf16_to_f64(sc.q_pe[0, 0])
    for h in range(sc.H):
        sa, sb = (0.3 * (ql[h] @ rows[i, :16] + qp[h] @ rows[i, 16:]) for i in range(2))
        wa, wb = 2 * math.exp(sa), math.exp(sb)
        want = (wa * rows[0, :16] + wb * rows[1, :16]) / (wa + wb)
        assert np.allclose(lat[0, 0, h], want, rtol=1e-12, atol=1e-13)
        assert math.isclose(lse[0, 0, h], math.log(wa + wb), rel_tol=1e-12)


def test_sparse_logical_ids_negative_control():
    """M5.8 0x0B: the entries are physical rows.  Reading them as logical token
    positions (through the block table) attends to other rows and fails the
    product tolerance."""
    sc = _sparse_tiny(407, T=2, lengths=(40, 33), topk=12)
    lat, _ = _sparse(sc)
    P = sc.page_size
    wrong = sc.indices.copy()
    for b in range(sc.B):
        for t in range(sc.T):
            for k in range(int(sc.topk_length[b])):
                j = int(sc.indices[b, t, k])
                if j < int(sc.seqlens[b]):
                    wrong[b, t, k] = sc.block_table[b, j // P] * P + j % P
    bad, _ = _sparse(sc, indices=wrong)
    assert _fails(bad, lat)


# --------------------------------------------------------------------------
# 9. FP8 cache rows (M5.8 0x0B, "Exact 656-byte FP8 row")

def test_e4m3_decode_matches_torch_float8_e4m3fn():
    """Every one of the 256 codes against PyTorch's float8_e4m3fn conversion
    (an independent implementation of the OCP E4M3 encoding)."""
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(codes)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e4m3_closed_forms():
    """Values fixed by the encoding: bias 7, subnormal step 2^-9, largest
    finite 448, NaN at exponent and mantissa all ones, sign in bit 7."""
    d = oracle.e4m3fn_decode
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x39) == 1.125 and d(0x3F) == 1.875
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x77) == 240.0 and not np.isnan(d(0x78))      # exponent 15 is finite but for m = 7


def test_bf16_round_nearest_even_and_single_rounding():
    """Ties go to the even neighbour; a value just above a tie goes up even
    when the excess is below float32's precision (a detour through float32
    would land on the tie and go down)."""
    got = oracle.bf16_round(np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8,
                                      -(1 + 3 * 2.0 ** -8), 1 + 2.0 ** -9, -2.5, 0.0, np.nan]))
    assert list(got[:7]) == [0x3F80, 0x3F81, 0x3F82, 0xBF82, 0x3F80, 0xC020, 0x0000]
    assert np.isnan(synth.bf16_bits_to_f32(got[7:]))
    # on float32 inputs it agrees with the float32 -> bf16 encoder of the input recipe
    x = np.random.default_rng(5).standard_normal(20000).astype(np.float32) * np.float32(37.0)
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), synth.f32_to_bf16_bits(x))


def test_fp8_product_rounded_once():
    """e4m3(code) * scale is rounded to bf16 from its exact value: for codes
    and fp32 scales whose exact product lies within float32's half ulp above
    a bf16 tie, the result is the upper neighbour (a detour through float32
    would land on the tie and round to even)."""
    hits = []
    for code in range(0x39, 0x40):                     # 1.125 .. 1.875
        v = float(oracle.e4m3fn_decode(code))
        for i in range(128):
            mid = 1.0 + (2 * i + 1) * 2.0 ** -8         # tie between two bf16 values in [1, 2)
            s0 = np.float32(mid / v)
            for s in (np.nextafter(s0, np.float32(0)), s0, np.nextafter(s0, np.float32(2))):
                p = v * float(s)                         # exact (4 x 24 significant bits)
                if p > mid and float(np.float32(p)) == mid:
                    hits.append((code, s, mid + 2.0 ** -8))
    assert len(hits) >= 4
    for code, s, upper in hits:
        row = np.zeros((1, 656), dtype=np.uint8)
        row[0, :512] = code
        row[0, 512:528] = np.full(4, s, dtype="<f4").view(np.uint8)
        out = oracle.fp8_rows_to_bf16(row)
        assert (synth.bf16_bits_to_f32(out[0, :512]) == upper).all()


def test_fp8_row_layout_hand_built():
    """Codes at bytes [0, 512), four little-endian fp32 scales at [512, 528)
    each covering 128 consecutive latent columns, 64 bf16 rope values at
    [528, 656)."""
    row = np.zeros((2, 656), dtype=np.uint8)
    row[:, :512] = 0x38                                # 1.0
    row[1, 5] = 0xB0                                   # -0.5
    row[:, 512:528] = np.array([1.0, 2.0, 4.0, 8.0], dtype="<f4").view(np.uint8)
    row[:, 528:] = np.full(64, 0x3F00, dtype="<u2").view(np.uint8)       # 0.5
    vals = synth.bf16_bits_to_f32(oracle.fp8_rows_to_bf16(row)).astype(np.float64)
    want = np.concatenate([np.repeat([1.0, 2.0, 4.0, 8.0], 128), np.full(64, 0.5)])
    assert np.array_equal(vals[0], want)
    want[5] = -0.5
    assert np.array_equal(vals[1], want)


def test_fp8_dequant_matches_torch_when_float32_is_exact():
    """With scales of at most 12 significant bits the product is exact in
    float32, so PyTorch's float8 -> float32 -> bf16 route is a second
    implementation of the same rounding."""
    rng = np.random.default_rng(11)
    n = 300
    codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                      # no NaN codes
    sc = np.round(rng.uniform(2048, 4095, size=(n, 4))) * np.exp2(rng.integers(-20, -8, size=(n, 4)))
    sc = sc.astype(np.float32)
    rows = np.zeros((n, 656), dtype=np.uint8)
    rows[:, :512] = codes
    rows[:, 512:528] = sc.astype("<f4").view(np.uint8)
    rows[:, 528:] = rng.integers(0, 256, size=(n, 128), dtype=np.uint8)
    got = oracle.fp8_rows_to_bf16(rows)
    lat = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    prod = lat.view(n, 4, 128) * torch.from_numpy(sc)[:, :, None]
    want = prod.reshape(n, 512).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[:, :512], want)
    assert np.array_equal(got[:, 512:], rows[:, 528:].copy().view("<u2"))


def test_fp8_case_reads_like_its_dequantized_bf16_case():
    """The FP8 decode is the bf16 decode of the dequantized rows; the rows no
    sequence reads stay NaN after dequantization, the live rows finite."""
    wl = synth.Workload("f8", B=2, T=1, H=2, L=0, page_size=16, seed=77, lengths=(40, 17))
    f = synth.make_fp8_case(wl)
    bc = oracle.fp8_case_as_bf16(f)
    live = np.zeros(bc.kv_cache.shape[:2], dtype=bool)
    for b in range(bc.B):
        for j in range(int(bc.seqlens[b])):
            live[bc.block_table[b, j // 16], j % 16] = True
    vals = synth.bf16_bits_to_f32(bc.kv_cache)
    assert np.isfinite(vals[live]).all() and np.isnan(vals[~live]).all()
    out, lse = oracle.normal_decode(bc)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
