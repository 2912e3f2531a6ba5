"""GPU parity of the cache append (mla_append_cache) and of multi-step
decoding: each step appends its new rows on the GPU and then decodes over the
grown cache.  The cache is compared with the oracle's append bit for bit, the
decode output and lse with the oracle's latent attention over the oracle's
own cache.  Rows a step has not yet appended start as NaN, so a decode that
read one, or an append that missed its position, shows up."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import SCALE, assert_close, assert_lse_close, bf16_bits, bf16_tensor, log, to_f64, upload

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

GROWTH = {
    # T = 1: a sequence that starts empty, one whose appends cross the 64-token
    # page boundary (62, 63, 64), one that starts a fresh page, a long one
    "t1_b4": (synth.scaled(W["v3_b64_l4096"], B=4, H=128, lengths=(3, 65, 67, 700), seed=2201), 3),
    # T = 4 (multi-token decode): 12 rows per sequence over three steps
    "t4_h32": (synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(12, 70, 300), seed=2202), 3),
    # T = 8, page 16: every step fills half a page
    "t8_p16": (synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, T=8, H=16, page_size=16,
                            lengths=(24, 41), seed=2203), 3),
}


def _tensors(st, dev="cuda:0"):
    return {k: bf16_tensor(v, dev) for k, v in st.items()}


@pytest.mark.parametrize("splits", [1, 0])
@pytest.mark.parametrize("name", sorted(GROWTH))
def test_multistep_append_decode(mk, name, splits):
    import torch
    wl, n_steps = GROWTH[name]
    log(f"[append+decode] {name} splits={splits}")
    g = synth.make_growth(wl, n_steps)
    case = g.base
    d = upload(case)
    kv, bt = d["kv_cache"], d["block_table"]
    cache = case.kv_cache
    T = wl.T
    for s, st in enumerate(g.steps):
        lens = (case.seqlens + (s + 1) * T).astype(np.int32)
        sl = torch.from_numpy(lens).to("cuda:0")
        t = _tensors(st)
        mk.mla_append_cache(t["c_new"], t["kpe_new"], kv, bt, sl)
        lat, lse = mk.mla_decode_latent(t["q_lat"], t["q_pe"], kv, bt, sl, int(lens.max()), SCALE,
                                        num_splits=splits, out_dtype=torch.float32)
        torch.cuda.synchronize()
        cache = oracle.append_rows(cache, case.block_table, lens, st["c_new"], st["kpe_new"],
                                   case.page_size)
        got_cache = bf16_bits(kv)
        n_bad = int(np.count_nonzero(got_cache != cache))
        assert n_bad == 0, f"step {s}: {n_bad} cache elements differ from the oracle's append"
        cs = dataclasses.replace(case, kv_cache=cache, seqlens=lens, q_pe=st["q_pe"])
        ref_lat, ref_lse = oracle.latent_attention(cs, oracle.bf16_to_f64(st["q_lat"]), scale=SCALE)
        assert_close(to_f64(lat), ref_lat, f"step {s} latent")
        assert_lse_close(to_f64(lse), ref_lse, f"step {s} lse")


def test_append_full_size_bitwise(mk):
    """One T = 1 append into the 64 x 4096-token, 128-head workload's paged
    pool (each sequence's row 4095 is the new one): the whole pool after the
    append equals the oracle's, bit for bit."""
    import torch
    log("[append] v3_b64_l4096 full pool")
    g = synth.make_growth(W["v3_b64_l4096"], 1)
    case = g.base
    st = g.steps[0]
    kv = bf16_tensor(case.kv_cache, "cuda:0")
    bt = torch.from_numpy(case.block_table).to("cuda:0")
    sl = torch.from_numpy(g.final_seqlens).to("cuda:0")
    t = _tensors({"c_new": st["c_new"], "kpe_new": st["kpe_new"]})
    mk.mla_append_cache(t["c_new"], t["kpe_new"], kv, bt, sl)
    torch.cuda.synchronize()
    ref = oracle.append_rows(case.kv_cache, case.block_table, g.final_seqlens, st["c_new"],
                             st["kpe_new"], case.page_size)
    got = bf16_bits(kv)
    assert np.array_equal(got, ref)


def test_append_skips_unmapped_and_empty(mk):
    """Rows whose page is unmapped (-1) are skipped; an empty batch is a no-op."""
    import torch
    log("[append] unmapped pages")
    P = 16
    pool = np.full((3, P, 576), 0x1234, np.uint16)
    bt = np.array([[2, -1], [0, 1]], np.int32)
    lens = np.array([17, 18], np.int32)   # seq 0: position 16 -> page 1 unmapped; seq 1: 17 -> block 1
    c = synth.normal_bf16((2, 1, 512), 2204)
    k = synth.normal_bf16((2, 1, 64), 2205)
    kv = bf16_tensor(pool, "cuda:0")
    mk.mla_append_cache(bf16_tensor(c, "cuda:0"), bf16_tensor(k, "cuda:0"), kv,
                        torch.from_numpy(bt).to("cuda:0"), torch.from_numpy(lens).to("cuda:0"))
    torch.cuda.synchronize()
    ref = oracle.append_rows(pool, bt, lens, c, k, P)
    assert np.array_equal(bf16_bits(kv), ref)
    assert int(np.count_nonzero(ref != pool)) <= 576
    empty = torch.empty((0, 1, 512), dtype=torch.bfloat16, device="cuda:0")
    mk.mla_append_cache(empty, empty[..., :64], kv, torch.from_numpy(bt).to("cuda:0"),
                        torch.from_numpy(lens).to("cuda:0"))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(kv), ref)
