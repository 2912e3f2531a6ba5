"""GPU parity of the Normal path (mla_decode_normal: per-head up-projected K/V,
chunked over the cache) against the oracle's fp64 Normal path, for one chunk
and for several (the carried max/sum/output state), ragged lengths, causal
multi-token rows up to T = 130 (two query tiles per head) and 2 to 128 heads;
plus the absorbed chain at T = 64 and 130 (the same function in the other
association order) against the same oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import SCALE, assert_close, assert_lse_close, log, sample_pairs, to_f64, upload

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
CASES = {
    "b3_l300_h128": synth.scaled(W["v3_b64_l4096"], B=3, L=300, seed=2401),
    "ragged_h128": synth.scaled(W["v3_b64_l4096"], B=5, lengths=(1, 17, 64, 250, 1000), seed=2402),
    "mtp_t4_h32": synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2403),
    "t64_h16_p16": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, T=64, H=16, page_size=16, lengths=(64, 300),
                                seed=2404),
    # 130 query tokens: two 128-row query tiles per head, the second with 2 rows
    "t130_h2": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, T=130, H=2, lengths=(130, 333), seed=2406),
}


def _ref(case, n_pairs=48):
    pairs = sample_pairs(case.B, case.H, n_pairs, seed=7)
    out, lse = oracle.normal_decode(case, pairs=pairs)
    return pairs, out, lse


@pytest.mark.parametrize("chunk", [None, 128, 48])
@pytest.mark.parametrize("name", sorted(CASES))
def test_normal_parity(mk, name, chunk):
    import torch
    log(f"[normal] {name} chunk={chunk}")
    case = synth.make_case(CASES[name])
    d = upload(case)
    out, lse = mk.mla_decode_normal(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                    d["block_table"], d["seqlens"], case.max_seqlen, SCALE, chunk=chunk)
    torch.cuda.synchronize()
    pairs, ref, ref_lse = _ref(case)
    got, got_lse = to_f64(out), to_f64(lse)
    b, h = pairs[:, 0], pairs[:, 1]
    assert_close(got[b, :, h], ref[b, :, h], f"{name} out")
    assert_lse_close(got_lse[b, :, h], ref_lse[b, :, h], f"{name} lse")
    assert np.isfinite(got).all()


@pytest.mark.parametrize("name", ["t64_h16_p16", "t130_h2"])
def test_absorbed_chain_large_t(mk, name):
    """The absorbed path at prefill-sized blocks of query tokens."""
    import torch
    log(f"[absorbed] {name} splits 1 and 3")
    case = synth.make_case(CASES[name])
    d = upload(case)
    pairs, ref, ref_lse = _ref(case)
    b, h = pairs[:, 0], pairs[:, 1]
    for splits in (1, 3):
        out, lse = mk.absorbed_decode(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                      d["block_table"], d["seqlens"], case.max_seqlen, num_splits=splits,
                                      latent_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(to_f64(out)[b, :, h], ref[b, :, h], f"absorbed {name} S={splits} out")
        assert_lse_close(to_f64(lse)[b, :, h], ref_lse[b, :, h], f"absorbed {name} S={splits} lse")


def test_normal_equals_absorbed_full_workload(mk):
    """At the 64 x 4096 benchmark shape the two association orders agree (every
    element, the product tolerance), and sampled pairs match the oracle."""
    import torch
    log("[normal vs absorbed] v3_b64_l4096, chunk 1024")
    case = synth.make_case(W["v3_b64_l4096"])
    d = upload(case)
    n_out, n_lse = mk.mla_decode_normal(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                        d["block_table"], d["seqlens"], case.max_seqlen, SCALE, chunk=1024)
    a_out, a_lse = mk.absorbed_decode(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                      d["block_table"], d["seqlens"], case.max_seqlen, num_splits=4,
                                      latent_dtype=torch.float32)
    torch.cuda.synchronize()
    pairs, ref, ref_lse = _ref(case, n_pairs=12)
    b, h = pairs[:, 0], pairs[:, 1]
    assert_close(to_f64(n_out)[b, :, h], ref[b, :, h], "normal out vs oracle")
    assert_close(to_f64(n_out), to_f64(a_out), "normal vs absorbed out")
    assert_lse_close(to_f64(n_lse), to_f64(a_lse), "normal vs absorbed lse")


def test_absorbed_automatic_runs_unsplit_when_units_fill_the_chip(mk):
    """num_splits = 0 with 4 x 64 query tokens x 128 heads: 256 work units
    already reach the CU count, so the call runs unsplit (partials untouched)
    and still matches the oracle."""
    import torch
    log("[absorbed] automatic mode at B*ceil(T*H/128) >= CUs")
    case = synth.make_case(synth.scaled(W["v3_b64_l4096"], B=4, T=64, L=300, seed=2405))
    d = upload(case)
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, 0, "cuda:0")
    buf.split_indptr.fill_(-7)
    q_lat = mk.mla_absorb_q(d["q_nope"], d["w_uk"])
    lat, lse = mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                    case.max_seqlen, SCALE, num_splits=0, out_dtype=torch.float32, buffers=buf)
    out = mk.mla_unabsorb_out(lat, d["w_uv"])
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if case.B * case.T * case.H // 128 >= cus:
        assert (buf.split_indptr.cpu().numpy() == -7).all()
    pairs, ref, ref_lse = _ref(case, n_pairs=24)
    b, h = pairs[:, 0], pairs[:, 1]
    assert_close(to_f64(out)[b, :, h], ref[b, :, h], "absorbed auto-unsplit out")
    assert_lse_close(to_f64(lse)[b, :, h], ref_lse[b, :, h], "absorbed auto-unsplit lse")
