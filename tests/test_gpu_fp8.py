"""GPU parity of the decode over 656-byte FP8 rows (mla_decode_latent_fp8,
M5.8 0x0B) against the CPU oracle, which dequantizes every row to bf16 (the
exact product code x scale, rounded once) and runs its latent attention.

The kernel forms the product in fp32 before rounding to bf16; the two differ
only where the fp32 product lands exactly on a bf16 tie.  Where the seeded
rows hold no such element, the FP8 kernel must also reproduce, bit for bit,
the bf16 kernel run on the oracle's dequantized rows (same tiles, same
arithmetic order): that pins the conversion and its placement in the tile
exactly."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (SCALE, assert_close, assert_lse_close, bf16_tensor, bits_to_f64, log, sample_pairs, to_f64,
                            upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


W = synth.WORKLOADS
CASES = {
    "v3_b3_l300": synth.scaled(W["v3_b64_l4096"], B=3, L=300, seed=2601),
    "v3_ragged_b5": synth.scaled(W["v3_ragged_b128"], B=5, ragged=None, lengths=(1, 17, 64, 250, 1000),
                                 seed=2602),
    "mtp_t4_h32": synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2603),
    "t2_h128_rows256": synth.scaled(W["v3_b64_l4096"], B=2, T=2, lengths=(70, 33), seed=2604),
    "h1_short": synth.scaled(W["v3_b64_l4096"], B=3, H=1, lengths=(1, 15, 16), seed=2605),
    "page16_h64": synth.scaled(W["v3_b64_l4096"], B=2, H=64, page_size=16, lengths=(100, 47), seed=2606),
    "page256_h16": synth.scaled(W["v3_b64_l4096"], B=2, H=16, page_size=256, lengths=(600, 257), seed=2607),
    "mtp_p16_tail": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, page_size=16, lengths=(35, 51), seed=2608),
    "history_matrix": synth.scaled(W["v3_b64_l4096"], B=5, H=16, lengths=(1, 127, 128, 129, 4096), seed=2609),
    "page1024_h8": synth.scaled(W["v3_b64_l4096"], B=2, H=8, page_size=1024, lengths=(1500, 1024), seed=2610),
    "b300_tiny_h4": synth.scaled(W["v3_b64_l4096"], B=300, H=4, lengths=tuple(1 + (7 * i) % 40 for i in range(300)),
                                 seed=2611),
    "t1024_h1": synth.scaled(W["v3_mtp_b32_t4_h32"], B=1, T=1024, H=1, lengths=(1100,), seed=2612),
    "t8_h16_p16": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, T=8, H=16, page_size=16, lengths=(8, 300), seed=2613),
}


def _prep(name):
    import torch
    f = synth.make_fp8_case(CASES[name])
    bc = oracle.fp8_case_as_bf16(f)
    d = upload(f.case)
    d["kv_fp8"] = torch.from_numpy(f.kv_fp8).to("cuda:0")
    ql_bits = synth.normal_bf16(f.case.q_nope.shape[:3] + (512,), 9100 + len(name), std=0.5)
    return f, bc, d, ql_bits


@pytest.mark.parametrize("out_f32", [True, False])
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_decode_unsplit(mk, name, out_f32):
    import torch
    log(f"[fp8 unsplit] {name} out_f32={out_f32}")
    f, bc, d, ql_bits = _prep(name)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"],
                                        bc.max_seqlen, SCALE, num_splits=1,
                                        out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


@pytest.mark.parametrize("part", ["f32", "bf16"])
@pytest.mark.parametrize("S", [2, 3, 7])
@pytest.mark.parametrize("name", ["v3_ragged_b5", "mtp_p16_tail", "history_matrix", "page1024_h8", "b300_tiny_h4"])
def test_fp8_split_partials_and_merge(mk, name, S, part):
    import torch
    log(f"[fp8 split] {name} S={S} partials={part}")
    f, bc, d, ql_bits = _prep(name)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    buf = mk.DecodeBuffers(bc.B, bc.T, bc.H, bc.max_seqlen, bc.page_size, S, "cuda:0",
                           part_dtype=torch.float32 if part == "f32" else torch.bfloat16)
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"],
                                        bc.max_seqlen, SCALE, num_splits=S, out_dtype=torch.float32,
                                        buffers=buf)
    torch.cuda.synchronize()
    plan = oracle.split_plan(bc.seqlens, S, bc.page_size)
    assert np.array_equal(buf.split_indptr.cpu().numpy(), plan[0])
    q64 = bits_to_f64(ql_bits)
    ref_po, ref_pl = oracle.latent_attention(bc, q64, plan=plan)
    n = int(plan[0][-1])
    got_pl = buf.part_lse[:n].cpu().numpy().astype(np.float64)
    empty = np.isneginf(ref_pl)
    assert np.array_equal(np.isneginf(got_pl), empty), "empty partials must carry lse = -inf"
    assert_lse_close(np.where(empty, 0, got_pl), np.where(empty, 0, ref_pl), "partial lse")
    assert_close(to_f64(buf.part_out[:n]), ref_po, "partial out")
    ref_lat, ref_lse = oracle.latent_attention(bc, q64)
    assert_close(to_f64(lat), ref_lat, "merged latent")
    assert_lse_close(to_f64(lse), ref_lse, "merged lse")


def test_fp8_auto_split(mk):
    import torch
    log("[fp8 split auto] v3_ragged_b5")
    f, bc, d, ql_bits = _prep("v3_ragged_b5")
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"],
                                        bc.max_seqlen, SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def _single_rounding_agrees(f):
    """True when no latent element's fp32 product sits on a bf16 tie, i.e. the
    float32 route (PyTorch on the CPU) gives the oracle's dequantized bits."""
    import torch
    rows = f.kv_fp8.reshape(-1, 656)
    live = ~np.isnan(rows[:, 512:528].copy().view("<f4")).any(axis=1)
    rows = rows[live]
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :512])).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(np.ascontiguousarray(rows[:, 512:528]).view("<f4").copy())
    via32 = (codes.view(-1, 4, 128) * sc[:, :, None]).reshape(-1, 512).to(torch.bfloat16)
    via32 = via32.view(torch.int16).numpy().view(np.uint16)
    return np.array_equal(via32, oracle.fp8_rows_to_bf16(rows)[:, :512])


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("name", ["v3_b3_l300", "mtp_t4_h32", "page16_h64", "t1024_h1"])
def test_fp8_equals_bf16_kernel_on_dequantized_rows(mk, name, S):
    import torch
    log(f"[fp8 vs bf16 rows] {name} S={S}")
    f, bc, d, ql_bits = _prep(name)
    exact = _single_rounding_agrees(f)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    kv_bf16 = bf16_tensor(bc.kv_cache, "cuda:0")
    a = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"], bc.max_seqlen,
                                 SCALE, num_splits=S, out_dtype=torch.float32)
    b = mk.mla_decode_latent(q_lat, d["q_pe"], kv_bf16, d["block_table"], d["seqlens"], bc.max_seqlen,
                             SCALE, num_splits=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    log(f"  rows free of fp32 ties: {exact}")
    if exact:
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert_close(to_f64(a[0]), to_f64(b[0]), "latent vs bf16 kernel")


def test_fp8_end_to_end_vs_normal_path(mk):
    """absorb -> FP8 decode (4 splits, bf16 partials) -> merge -> un-absorb,
    against the oracle's Normal path over the dequantized rows."""
    import torch
    log("[fp8 end-to-end] mtp_t4_h32")
    f, bc, d, _ = _prep("mtp_t4_h32")
    q_lat = mk.mla_absorb_q(d["q_nope"], d["w_uk"])
    buf = mk.DecodeBuffers(bc.B, bc.T, bc.H, bc.max_seqlen, bc.page_size, 4, "cuda:0",
                           part_dtype=torch.bfloat16)
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"],
                                        bc.max_seqlen, SCALE, num_splits=4, buffers=buf)
    out = mk.mla_unabsorb_out(lat, d["w_uv"])
    torch.cuda.synchronize()
    ref, ref_lse = oracle.normal_decode(bc)
    assert_close(to_f64(out), ref, "out")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def test_fp8_full_headline_sampled(mk):
    """The 64 x 4096, 128-head workload in the launch configuration the
    benchmark times (4 uniform splits, bf16 partials, merge), checked on
    sampled (sequence, head) pairs the oracle computes one by one."""
    import torch
    log("[fp8 full] v3_b64_l4096 (sampled pairs)")
    f = synth.make_fp8_case(W["v3_b64_l4096"])
    c = f.case
    pairs = sample_pairs(c.B, c.H, 12, 2620)
    d = upload(c)
    kv = torch.from_numpy(f.kv_fp8).to("cuda:0")
    ql_bits = synth.normal_bf16(c.q_nope.shape[:3] + (512,), 9200, std=0.5)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    buf = mk.DecodeBuffers(c.B, c.T, c.H, c.max_seqlen, c.page_size, 4, "cuda:0", part_dtype=torch.bfloat16)
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], kv, d["block_table"], d["seqlens"], c.max_seqlen,
                                        SCALE, num_splits=4, buffers=buf)
    torch.cuda.synchronize()
    bc = oracle.fp8_case_as_bf16(f)
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits), pairs=pairs)
    got = to_f64(lat)
    got_lse = lse.cpu().numpy().astype(np.float64)
    for b, h in pairs:
        assert_close(got[b, :, h], ref_lat[b, :, h], f"latent b={b} h={h}")
        assert_lse_close(got_lse[b, :, h], ref_lse[b, :, h], f"lse b={b} h={h}")


def test_fp8_full_long_context_sampled(mk):
    """The 4 x 131072 long-context workload over FP8 rows with its 64 uniform
    splits (256 work units) and the merge, on sampled pairs."""
    import torch
    log("[fp8 full] v3_long_b4_l131072 (sampled pairs)")
    f = synth.make_fp8_case(W["v3_long_b4_l131072"])
    c = f.case
    pairs = sample_pairs(c.B, c.H, 6, 2630)
    d = upload(c)
    kv = torch.from_numpy(f.kv_fp8).to("cuda:0")
    ql_bits = synth.normal_bf16(c.q_nope.shape[:3] + (512,), 9210, std=0.5)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    buf = mk.DecodeBuffers(c.B, c.T, c.H, c.max_seqlen, c.page_size, 64, "cuda:0", part_dtype=torch.bfloat16)
    lat, lse = mk.mla_decode_latent_fp8(q_lat, d["q_pe"], kv, d["block_table"], d["seqlens"], c.max_seqlen,
                                        SCALE, num_splits=64, buffers=buf, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bc = oracle.fp8_case_as_bf16(f)
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits), pairs=pairs)
    got = to_f64(lat)
    got_lse = lse.cpu().numpy().astype(np.float64)
    for b, h in pairs:
        assert_close(got[b, :, h], ref_lat[b, :, h], f"latent b={b} h={h}")
        assert_lse_close(got_lse[b, :, h], ref_lse[b, :, h], f"lse b={b} h={h}")


@pytest.mark.parametrize("S", [1, 2, 0])
@pytest.mark.parametrize("hot_token", [3, 137, 290])
def test_fp8_score_growth_past_reference(mk, S, hot_token):
    """One FP8 row whose dequantized latent is 448 x scale x sign(q~[0,0,0,:])
    (scale chosen so its entries are 16 times the query's mean magnitude):
    head 0's score there exceeds every earlier one by far more than the
    kernel's tolerated growth, so the work unit is replayed with a raised
    reference -- the FP8 prologue then runs a second time.  The result must
    match the oracle, and head 0 of sequence 0 must return that row."""
    import torch
    log(f"[fp8 growth] hot key at {hot_token}, num_splits={S}")
    f = synth.make_fp8_case(CASES["v3_b3_l300"])
    ql_bits = synth.normal_bf16(f.case.q_nope.shape[:3] + (512,), 9400 + hot_token, std=0.5)
    q0 = bits_to_f64(ql_bits[0, 0, 0, :])
    P = f.case.page_size
    blk, off = int(f.case.block_table[0, hot_token // P]), hot_token % P
    f.kv_fp8[blk, off, :512] = np.where(q0 < 0, 0xFE, 0x7E).astype(np.uint8)      # -448 / +448
    scale = np.float32(16.0 * np.mean(np.abs(q0)) / 448.0)
    f.kv_fp8[blk, off, 512:528] = np.full(4, scale, dtype="<f4").view(np.uint8)
    bc = oracle.fp8_case_as_bf16(f)
    d = upload(f.case)
    kv = torch.from_numpy(f.kv_fp8).to("cuda:0")
    lat, lse = mk.mla_decode_latent_fp8(bf16_tensor(ql_bits, "cuda:0"), d["q_pe"], kv, d["block_table"],
                                        d["seqlens"], bc.max_seqlen, SCALE, num_splits=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits))
    hot = bits_to_f64(bc.kv_cache[blk, off, :512])
    assert float(np.max(np.abs(ref_lat[0, 0, 0] - hot))) < 1e-6 * float(np.max(np.abs(hot)))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def test_fp8_auto_split_full_chip_runs_unsplit(mk):
    """Automatic splits with an output wanted and one work unit per sequence
    already reaching the CU count (300 sequences): the call runs unsplit and
    leaves the partial buffers untouched."""
    import torch
    log("[fp8 split auto, full chip] b300_tiny_h4")
    f, bc, d, ql_bits = _prep("b300_tiny_h4")
    buf = mk.DecodeBuffers(bc.B, bc.T, bc.H, bc.max_seqlen, bc.page_size, 0, "cuda:0")
    buf.part_lse.fill_(123.0)
    lat, lse = mk.mla_decode_latent_fp8(bf16_tensor(ql_bits, "cuda:0"), d["q_pe"], d["kv_fp8"], d["block_table"],
                                        d["seqlens"], bc.max_seqlen, SCALE, num_splits=0, out_dtype=torch.float32,
                                        buffers=buf)
    torch.cuda.synchronize()
    assert bool((buf.part_lse == 123.0).all())
    ref_lat, ref_lse = oracle.latent_attention(bc, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def test_fp8_page_placement_is_bitwise_invisible(mk):
    """The same logical FP8 rows laid out in (sequence, page) order instead of
    the seeded permutation give bit-identical results."""
    import torch
    log("[fp8 bitwise] permuted vs identity pages")
    f, bc, d, ql_bits = _prep("v3_ragged_b5")
    c = f.case
    P = c.page_size
    pages = [(int(L) + P - 1) // P for L in c.seqlens]
    rows = np.empty((sum(pages), P, 656), dtype=np.uint8)
    table = np.full_like(c.block_table, -1)
    k = 0
    for b in range(c.B):
        for pg in range(pages[b]):
            rows[k] = f.kv_fp8[c.block_table[b, pg]]
            table[b, pg] = k
            k += 1
    ql = bf16_tensor(ql_bits, "cuda:0")
    outs = []
    for kv, bt in ((f.kv_fp8, c.block_table), (rows, table)):
        lat, lse = mk.mla_decode_latent_fp8(ql, d["q_pe"], torch.from_numpy(kv).to("cuda:0"),
                                            torch.from_numpy(bt).to("cuda:0"), d["seqlens"], bc.max_seqlen,
                                            SCALE, out_dtype=torch.float32)
        outs.append((lat.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("S", [1, 4, 0])
def test_fp8_graph_replays_match_eager(mk, S):
    """The FP8 decode (and its merge) captured in a HIP graph: every replay,
    with eager work overwriting the outputs in between, equals the eager
    result bit for bit."""
    import torch
    log(f"[fp8 graph] num_splits={S}")
    f, bc, d, ql_bits = _prep("mtp_t4_h32")
    B, T, H = bc.B, bc.T, bc.H
    dev = "cuda:0"
    q_lat = bf16_tensor(ql_bits, dev)
    buf = mk.DecodeBuffers(B, T, H, bc.max_seqlen, bc.page_size, S, dev, part_dtype=torch.bfloat16) \
        if S != 1 else None
    latent = torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)

    def step():
        if S == 1:
            mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"], bc.max_seqlen,
                                     SCALE, num_splits=1, out_latent=latent, lse=lse)
        else:
            mk.mla_decode_latent_fp8(q_lat, d["q_pe"], d["kv_fp8"], d["block_table"], d["seqlens"], bc.max_seqlen,
                                     SCALE, num_splits=S, buffers=buf, merge=False)
            mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, B, out_latent=latent, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = (latent.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        latent.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(latent, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep} differs from eager"
