"""GPU parity of mla_merge_unabsorb, the split merge (M5.8 0x0C) and the
un-absorb ("MLA in full detail", Step 4) in one kernel.

Fed partials the oracle computed, it matches the oracle's merge followed by its
un-absorb; fed the decode kernel's own partials, it matches the oracle's latent
attention followed by its un-absorb, and the two separate GPU calls (merge to a
bf16 latent, then un-absorb): the merged lse bit for bit, the output up to the
order of the fp32 sums.  Cases cover 1 to 70 splits per row (the kernel loads
up to four before any arithmetic and takes the rest 64 lse values and eight
rows at a time), fp32 and bf16 partials, rows without a split, query-row counts
that are not a multiple of the 32-row block, workgroups that take several
blocks, head counts that are and are not multiples of 8, sparse partials, and
the benchmark's full-size configuration."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (SCALE, assert_close, assert_lse_close, bf16_tensor, bits_to_f64, log, to_f64,
                            upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()  # raises if the HIP library is missing
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


W = synth.WORKLOADS


def _q_lat(case, seed):
    # absorbed queries are W_UK^T q_nope: N(0, 128/512) per element under the recipe
    return synth.normal_bf16(case.q_nope.shape[:3] + (512,), seed, std=0.5)


def _partials(case, S, part, seed, dev="cuda:0"):
    """Oracle partials of a uniform S-split plan, rounded to the partial dtype;
    returns (device partials, device lse, device indptr, the rounded values in
    fp64, lse in fp64, indptr)."""
    import torch
    q64 = bits_to_f64(_q_lat(case, seed))
    plan = oracle.split_plan(case.seqlens, S, case.page_size)
    po, pl = oracle.latent_attention(case, q64, plan=plan)
    if part == "f32":
        po_in = po.astype(np.float32).astype(np.float64)
        t_po = torch.from_numpy(po.astype(np.float32)).to(dev)
    else:
        bits = synth.f32_to_bf16_bits(po.astype(np.float32))
        po_in = bits_to_f64(bits)
        t_po = bf16_tensor(bits, dev)
    pl32 = pl.astype(np.float32)
    return (t_po, torch.from_numpy(pl32).to(dev), torch.from_numpy(plan[0]).to(dev), po_in,
            pl32.astype(np.float64), plan[0])


@pytest.mark.parametrize("part", ["f32", "bf16"])
@pytest.mark.parametrize("S", [1, 3, 4, 5, 9, 70])
def test_fused_on_oracle_partials(mk, S, part):
    """70 splits of sequences of 4 to 100 tokens: most chunks are empty
    (lse -inf, weight 0) and one row's lse values span two 64-lane passes."""
    import torch
    log(f"[merge+unabsorb] oracle partials S={S} ({part})")
    case = synth.make_case(synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2501))
    t_po, t_pl, t_ind, po_in, pl_in, ind = _partials(case, S, part, 2502)
    lat, ref_lse = oracle.merge(po_in, pl_in, ind)
    ref = oracle.unabsorb(lat, case.w_uv)
    d = upload(case)
    out, lse = mk.mla_merge_unabsorb(t_po, t_pl, t_ind, d["w_uv"], case.B)
    torch.cuda.synchronize()
    assert_close(to_f64(out), ref, "out")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def test_rows_without_splits(mk):
    """A sequence whose split range is empty gives out = 0 and lse = -inf; the
    other sequences are unaffected."""
    import torch
    log("[merge+unabsorb] a sequence without splits")
    case = synth.make_case(synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 40, 77), seed=2511))
    S = 3
    t_po, t_pl, t_ind, po_in, pl_in, ind = _partials(case, S, "bf16", 2512)
    # drop sequence 1's three split rows
    keep = np.r_[0:S, 2 * S:3 * S]
    ind2 = np.array([0, S, S, 2 * S], np.int32)
    dev = "cuda:0"
    lat, ref_lse = oracle.merge(po_in[keep], pl_in[keep], ind2)
    ref = oracle.unabsorb(lat, case.w_uv)
    d = upload(case)
    out, lse = mk.mla_merge_unabsorb(t_po[torch.from_numpy(keep).to(dev)].contiguous(),
                                     t_pl[torch.from_numpy(keep).to(dev)].contiguous(),
                                     torch.from_numpy(ind2).to(dev), d["w_uv"], case.B)
    torch.cuda.synchronize()
    o, ls = to_f64(out), to_f64(lse)
    assert (o[1] == 0).all() and np.isneginf(ls[1]).all()
    sel = [0, 2]
    assert_close(o[sel], ref[sel], "out of the other sequences")
    assert_lse_close(ls[sel], ref_lse[sel], "lse of the other sequences")


CHAIN = {
    # 70 query rows (B*T): a partial third 32-row block; 2 heads (not a multiple of 8)
    "m70_h2": (synth.scaled(W["v3_b64_l4096"], B=35, T=2, H=2, L=40, seed=2503), 3, "bf16"),
    "ragged_b5_auto": (synth.scaled(W["v3_ragged_b128"], B=5, ragged=None, lengths=(1, 17, 64, 250, 1000),
                                    seed=2504), 0, "bf16"),
    "mtp_t4_f32": (synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2505), 4, "f32"),
    "h16_s64": (synth.scaled(W["v3_b64_l4096"], B=2, H=16, lengths=(4096, 333), seed=2506), 64, "bf16"),
    # 200 rows of 128 heads: 7 blocks per head over 2 workgroups, each taking several
    "b200_h128": (synth.scaled(W["v3_b64_l4096"], B=200, L=48, seed=2507), 2, "bf16"),
    # one head, 1024 query rows: 32 workgroups of one block
    "t1024_h1": (synth.scaled(W["v3_mtp_b32_t4_h32"], B=1, T=1024, H=1, lengths=(1100,), seed=2508), 2, "bf16"),
    # 12 heads: not a multiple of 8, several workgroups per head
    "h12_b40": (synth.scaled(W["v3_b64_l4096"], B=40, H=12, L=100, seed=2509), 4, "f32"),
}


def _chain(mk, case, d, S, part):
    import torch
    q_lat = mk.mla_absorb_q(d["q_nope"], d["w_uk"])
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, "cuda:0",
                           part_dtype=torch.float32 if part == "f32" else torch.bfloat16)
    mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"], case.max_seqlen,
                         SCALE, num_splits=S, buffers=buf, merge=False)
    fused, fused_lse = mk.mla_merge_unabsorb(buf.part_out, buf.part_lse, buf.split_indptr, d["w_uv"], case.B)
    lat, lse = mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, case.B,
                                   out_dtype=torch.bfloat16)
    sep = mk.mla_unabsorb_out(lat, d["w_uv"])
    torch.cuda.synchronize()
    return q_lat, fused, fused_lse, sep, lse


def _close_to_separate(fused, sep):
    """Same merged bf16 latent, same products: only the order of the fp32 sums
    over the 512 latent columns differs (one chain against four partial sums)."""
    f, s = to_f64(fused), to_f64(sep)
    err = float(np.max(np.abs(f - s)))
    bound = 1e-5 * float(np.max(np.abs(s))) + 1e-7
    log(f"  fused vs separate: max|diff| {err:.3e}  bound {bound:.3e}")
    assert err <= bound


@pytest.mark.parametrize("name", sorted(CHAIN))
def test_fused_after_decode(mk, name):
    import torch
    wl, S, part = CHAIN[name]
    log(f"[merge+unabsorb] after the decode: {name} S={S} ({part})")
    case = synth.make_case(wl)
    d = upload(case)
    q_lat, fused, fused_lse, sep, lse = _chain(mk, case, d, S, part)
    assert torch.equal(fused_lse, lse), "merged lse differs from mla_merge_splits"
    _close_to_separate(fused, sep)
    lat_ref, lse_ref = oracle.latent_attention(case, to_f64(q_lat))
    ref = oracle.unabsorb(lat_ref, case.w_uv)
    assert_close(to_f64(fused), ref, "out vs oracle")
    assert_lse_close(to_f64(fused_lse), lse_ref, "lse vs oracle")


def test_fused_on_sparse_partials(mk):
    """Partials of the sparse (top-k) decode: each query token is its own row
    of the split table (B*T rows, one token each)."""
    import torch
    log("[merge+unabsorb] sparse partials")
    sc = synth.make_sparse(synth.scaled(W["v3_b64_l4096"], B=3, lengths=(1000, 400, 300), seed=2521), 300)
    dev = "cuda:0"
    q_lat, q_pe = bf16_tensor(sc.q_lat, dev), bf16_tensor(sc.q_pe, dev)
    kv = bf16_tensor(sc.kv_cache, dev)
    idx = torch.from_numpy(sc.indices).to(dev)
    tl = torch.from_numpy(sc.topk_length).to(dev)
    buf = mk.SparseBuffers(sc.B, sc.T, sc.H, sc.topk, 3, dev, part_dtype=torch.bfloat16)
    mk.mla_decode_sparse(q_lat, q_pe, kv, idx, tl, SCALE, num_splits=3, buffers=buf, merge=False)
    w_bits = synth.normal_bf16((sc.H, 128, 512), 2522, std=512 ** -0.5)
    w_uv = bf16_tensor(w_bits, dev)
    BT = sc.B * sc.T
    out, lse = mk.mla_merge_unabsorb(buf.part_out.view(BT * 3, 1, sc.H, 512), buf.part_lse.view(BT * 3, 1, sc.H),
                                     buf.split_indptr, w_uv, BT)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.sparse_latent_attention(oracle.bf16_to_f64(sc.q_lat), sc.q_pe, sc.kv_cache,
                                                      sc.indices, sc.topk_length, SCALE)
    ref = oracle.unabsorb(ref_lat.reshape(BT, 1, sc.H, 512), w_bits)
    assert_close(to_f64(out), ref, "out")
    assert_lse_close(to_f64(lse).reshape(sc.B, sc.T, sc.H), ref_lse, "lse")


def test_fused_full_size(mk):
    """The benchmark's configuration: 64 sequences of 4096 tokens, 128 heads, 4
    uniform splits, bf16 partials; every output element against the separate
    merge and un-absorb, the lse bit for bit."""
    import torch
    log("[merge+unabsorb] full size b64 l4096 S=4")
    case = synth.make_case(W["v3_b64_l4096"], poison=False)
    d = upload(case)
    _, fused, fused_lse, sep, lse = _chain(mk, case, d, 4, "bf16")
    assert torch.equal(fused_lse, lse)
    _close_to_separate(fused, sep)
