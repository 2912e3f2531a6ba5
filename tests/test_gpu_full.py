"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (uniform 4-way split on the headline workload): the end-to-end
chain against the Normal (decompressed) path on a seeded sample of (sequence,
head) pairs that the CPU oracle computes one by one, and the latent stage
(latent output and lse) against the fp64 absorbed mirror on EVERY (sequence,
token, head) row (the mirror costs 2,176 FLOP per row and key, a few seconds
per workload on the host cores).  Unreadable cache rows are NaN-poisoned, so a
stray read anywhere fails."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import SCALE, assert_close, assert_lse_close, bits_to_f64, bf16_tensor, log, to_f64, upload, sample_pairs

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


def _buffers(mk, case, S, part):
    import torch
    if S == 1:
        return None
    return mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, "cuda:0",
                            part_dtype=torch.bfloat16 if part == "bf16" else torch.float32)


def _run_chain(mk, case, d, S, part):
    import torch
    q_lat = mk.mla_absorb_q(d["q_nope"], d["w_uk"])
    lat, lse = mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                    case.max_seqlen, SCALE, num_splits=S, out_dtype=torch.bfloat16,
                                    buffers=_buffers(mk, case, S, part))
    out = mk.mla_unabsorb_out(lat, d["w_uv"])
    torch.cuda.synchronize()
    return q_lat, out, lse


def _check_pairs(got, ref, pairs, what, check=assert_close):
    g = np.stack([got[b, :, h] for b, h in pairs])
    r = np.stack([ref[b, :, h] for b, h in pairs])
    check(g, r, what)


@pytest.mark.parametrize("name,S,part,n_normal", [
    ("v2lite_tiny", 1, "-", 16),
    ("v3_b64_l4096", 4, "bf16", 10),
    ("v3_b64_l4096", 4, "f32", 4),
    ("v3_b64_l4096", 1, "-", 6),
    ("v3_b64_l4096", 0, "bf16", 4),
    ("v3_ragged_b128", 0, "bf16", 6),
    ("v3_long_b4_l131072", 64, "f32", 3),
    ("v3_long_b4_l131072", 64, "bf16", 2),
    ("v3_mtp_b32_t4_h32", 1, "-", 8),
    ("v3_mtp_b32_t4_h32", 0, "bf16", 4),
])
def test_full_size(mk, name, S, part, n_normal):
    log(f"[full] {name} num_splits={S} partials={part}: generating inputs")
    case = synth.make_case(W[name])
    d = upload(case)
    log(f"[full] {name}: running the GPU chain")
    q_lat, out, lse = _run_chain(mk, case, d, S, part)
    out_h = to_f64(out)
    lse_h = to_f64(lse)
    assert np.isfinite(out_h).all() and np.isfinite(lse_h).all(), "non-finite output (stray read?)"

    pairs = sample_pairs(case.B, case.H, n_normal, seed=31)
    log(f"[full] {name}: Normal-path oracle on {len(pairs)} pairs")
    ref, ref_lse = oracle.normal_decode(case, pairs=pairs)
    _check_pairs(out_h, ref, pairs, "out (Normal path)")
    _check_pairs(lse_h, ref_lse, pairs, "lse (Normal path)", assert_lse_close)

    # latent stage on more pairs: seeded absorbed query given to both sides
    import torch
    ql_bits = synth.normal_bf16(case.q_nope.shape[:3] + (512,), 9100, std=0.5)
    lat, lse2 = mk.mla_decode_latent(bf16_tensor(ql_bits, "cuda:0"), d["q_pe"], d["kv_cache"],
                                     d["block_table"], d["seqlens"], case.max_seqlen, SCALE,
                                     num_splits=S, out_dtype=torch.float32,
                                     buffers=_buffers(mk, case, S, part))
    torch.cuda.synchronize()
    log(f"[full] {name}: absorbed mirror on all {case.B * case.T * case.H} rows")
    ref_lat, ref_lse2 = oracle.latent_attention(case, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent (mirror, every row)")
    assert_lse_close(to_f64(lse2), ref_lse2, "lse (mirror, every row)")


def test_headline_split_matches_unsplit_closely(mk):
    """Same inputs, 1 vs 4 vs automatic splits: all within tolerance of each other."""
    import torch
    case = synth.make_case(W["v3_b64_l4096"])
    d = upload(case)
    ql = bf16_tensor(synth.normal_bf16(case.q_nope.shape[:3] + (512,), 9200, std=0.5), "cuda:0")
    res = []
    for S in (1, 4, 0):
        lat, lse = mk.mla_decode_latent(ql, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                        case.max_seqlen, SCALE, num_splits=S, out_dtype=torch.float32)
        res.append((to_f64(lat), to_f64(lse)))
    for k in (1, 2):
        assert_close(res[k][0], res[0][0], f"latent split variant {k}")
        assert_lse_close(res[k][1], res[0][1], f"lse split variant {k}")
