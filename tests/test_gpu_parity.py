"""GPU parity of every entry point of the C ABI against the CPU oracle, on
seeded inputs small enough for the oracle to run in full (several KV tiles,
ragged tails, causal multi-token rows, more than 128 query rows, tiny and
single-key sequences, page sizes 16/64/256).

Stage inputs are generated, never taken from the GPU: the decode stage gets a
seeded absorbed query, the un-absorb stage a seeded latent.  The end-to-end
chain runs the GPU's own intermediates and is compared with the oracle's
Normal (decompressed) path."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (SCALE, assert_close, assert_lse_close, bf16_tensor, bits_to_f64, log, to_f64, upload)

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


def small_cases():
    return {
        "v2lite_tiny": W["v2lite_tiny"],
        "v3_b3_l300": synth.scaled(W["v3_b64_l4096"], B=3, L=300, seed=2101),
        "v3_ragged_b5": synth.scaled(W["v3_ragged_b128"], B=5, ragged=None,
                                     lengths=(1, 17, 64, 250, 1000), seed=2102),
        "mtp_t4_h32": synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2103),
        "t2_h128_rows256": synth.scaled(W["v3_b64_l4096"], B=2, T=2, lengths=(70, 33), seed=2104),
        "h1_short": synth.scaled(W["v3_b64_l4096"], B=3, H=1, lengths=(1, 15, 16), seed=2105),
        "page16_h64": synth.scaled(W["v3_b64_l4096"], B=2, H=64, page_size=16, lengths=(100, 47),
                                   seed=2106),
        "page256_h16": synth.scaled(W["v3_b64_l4096"], B=2, H=16, page_size=256,
                                    lengths=(600, 257), seed=2107),
        # page 16, T=4: with 2 or 3 splits the last chunk of the 35-token sequence
        # starts at 32 = L - T + 1, where query t=0 sees none of its keys
        "mtp_p16_tail": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, page_size=16, lengths=(35, 51),
                                     seed=2108),
        # 70 query tokens (B*T): the weight GEMMs take a second, partial 64-row chunk
        "m70_h2": synth.scaled(W["v3_b64_l4096"], B=35, T=2, H=2, L=40, seed=2109),
        # the history lengths M5.8 0x0E's shape matrix names (around a 128-token
        # boundary, a single key, a long history)
        "history_matrix": synth.scaled(W["v3_b64_l4096"], B=5, H=16, lengths=(1, 127, 128, 129, 4096),
                                       seed=2111),
        # the largest multi-token decode the boundary takes (T = 8), 8 x 16 = 128 rows
        "t8_h16": synth.scaled(W["v3_mtp_b32_t4_h32"], B=2, T=8, H=16, lengths=(8, 300), seed=2112),
        # the largest page size the boundary takes (one partial second page)
        "page1024_h8": synth.scaled(W["v3_b64_l4096"], B=2, H=8, page_size=1024, lengths=(1500, 1024),
                                    seed=2113),
        # many tiny sequences (1..40 tokens): more work units than CUs, most of them one step
        "b300_tiny_h4": synth.scaled(W["v3_b64_l4096"], B=300, H=4,
                                     lengths=tuple(1 + (7 * i) % 40 for i in range(300)), seed=2114),
        # the largest query block the boundary takes: T = 1024 rows of one head, 8 row groups
        "t1024_h1": synth.scaled(W["v3_mtp_b32_t4_h32"], B=1, T=1024, H=1, lengths=(1100,), seed=2115),
    }


CASES = small_cases()


def _case(name):
    return synth.make_case(CASES[name])


@pytest.mark.parametrize("name", sorted(CASES))
def test_absorb(mk, name):
    log(f"[absorb] {name}")
    case = _case(name)
    d = upload(case)
    q_lat = mk.mla_absorb_q(d["q_nope"], d["w_uk"])
    ref = oracle.absorb(case.q_nope, case.w_uk)
    assert_close(to_f64(q_lat), ref, "q_lat")


def _stage_q_lat(case, seed):
    # absorbed queries are W_UK^T q_nope: N(0, 128/512) per element under the recipe
    return synth.normal_bf16(case.q_nope.shape[:3] + (512,), seed, std=0.5)


@pytest.mark.parametrize("out_f32", [True, False])
@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_unsplit(mk, name, out_f32):
    import torch
    log(f"[decode unsplit] {name} out_f32={out_f32}")
    case = _case(name)
    d = upload(case)
    ql_bits = _stage_q_lat(case, 7000 + len(name))
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    lat, lse = mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                    case.max_seqlen, SCALE, num_splits=1,
                                    out_dtype=torch.float32 if out_f32 else torch.bfloat16)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(case, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


@pytest.mark.parametrize("latent_f32", [True, False])
@pytest.mark.parametrize("name", ["v3_b3_l300", "mtp_t4_h32", "h1_short", "v2lite_tiny"])
def test_unabsorb(mk, name, latent_f32):
    import torch
    log(f"[unabsorb] {name} latent_f32={latent_f32}")
    case = _case(name)
    d = upload(case)
    shape = case.q_nope.shape[:3] + (512,)
    if latent_f32:
        x = synth.normal_f32(shape, 8100, std=0.1)
        lat = torch.from_numpy(x).to("cuda:0")
        ref = oracle.unabsorb(x.astype(np.float64), case.w_uv)
    else:
        bits = synth.normal_bf16(shape, 8101, std=0.1)
        lat = bf16_tensor(bits, "cuda:0")
        ref = oracle.unabsorb(bits_to_f64(bits), case.w_uv)
    out = mk.mla_unabsorb_out(lat, d["w_uv"])
    assert_close(to_f64(out), ref, "out")


@pytest.mark.parametrize("S", [1, 4])
@pytest.mark.parametrize("name", sorted(CASES))
def test_end_to_end_vs_normal_path(mk, name, S):
    """S = 1: absorb, decode, un-absorb; S = 4: absorb, split decode with bf16
    partials, merge and un-absorb in one kernel."""
    import torch
    log(f"[end-to-end] {name} S={S}")
    case = _case(name)
    d = upload(case)
    out, lse = mk.absorbed_decode(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                  d["block_table"], d["seqlens"], case.max_seqlen, num_splits=S)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.normal_decode(case)
    assert_close(to_f64(out), ref, "out")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


@pytest.mark.parametrize("part", ["f32", "bf16"])
@pytest.mark.parametrize("S", [2, 3, 7])
@pytest.mark.parametrize("name", ["v3_ragged_b5", "mtp_t4_h32", "page16_h64", "mtp_p16_tail", "history_matrix",
                                  "t8_h16", "page1024_h8", "b300_tiny_h4"])
def test_split_partials_and_merge(mk, name, S, part):
    import torch
    log(f"[split] {name} S={S} partials={part}")
    case = _case(name)
    d = upload(case)
    ql_bits = _stage_q_lat(case, 7100 + S)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, S, "cuda:0",
                           part_dtype=torch.float32 if part == "f32" else torch.bfloat16)
    lat, lse = mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                    case.max_seqlen, SCALE, num_splits=S, out_dtype=torch.float32,
                                    buffers=buf)
    torch.cuda.synchronize()
    plan = oracle.split_plan(case.seqlens, S, case.page_size)
    # the split plan is integer work: bit-exact
    assert np.array_equal(buf.split_indptr.cpu().numpy(), plan[0])
    q64 = bits_to_f64(ql_bits)
    ref_po, ref_pl = oracle.latent_attention(case, q64, plan=plan)
    n = int(plan[0][-1])
    got_pl = buf.part_lse[:n].cpu().numpy().astype(np.float64)
    empty = np.isneginf(ref_pl)
    assert np.array_equal(np.isneginf(got_pl), empty), "empty partials must carry lse = -inf"
    assert_lse_close(np.where(empty, 0, got_pl), np.where(empty, 0, ref_pl), "partial lse")
    assert_close(to_f64(buf.part_out[:n]), ref_po, "partial out")
    ref_lat, ref_lse = oracle.latent_attention(case, q64)
    assert_close(to_f64(lat), ref_lat, "merged latent")
    assert_lse_close(to_f64(lse), ref_lse, "merged lse")


def test_auto_split(mk):
    import torch
    log("[split auto] v3_ragged_b5")
    case = _case("v3_ragged_b5")
    d = upload(case)
    ql_bits = _stage_q_lat(case, 7200)
    q_lat = bf16_tensor(ql_bits, "cuda:0")
    lat, lse = mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                    case.max_seqlen, SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(case, bits_to_f64(ql_bits))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


@pytest.mark.parametrize("part", ["f32", "bf16"])
def test_merge_of_oracle_partials(mk, part):
    """The merge kernel alone, fed partials the oracle computed (rounded to the
    partial dtype on the host; the expected value merges the same rounded values)."""
    import torch
    log(f"[merge] oracle partials ({part})")
    case = _case("mtp_t4_h32")
    q64 = bits_to_f64(_stage_q_lat(case, 7300))
    plan = oracle.split_plan(case.seqlens, 5, case.page_size)
    po, pl = oracle.latent_attention(case, q64, plan=plan)
    dev = "cuda:0"
    if part == "f32":
        po_in = po.astype(np.float32)
        t_po = torch.from_numpy(po_in).to(dev)
    else:
        bits = synth.f32_to_bf16_bits(po.astype(np.float32))
        po_in = bits_to_f64(bits)
        t_po = bf16_tensor(bits, dev)
    pl_in = pl.astype(np.float32)
    ref, ref_lse = oracle.merge(po_in.astype(np.float64), pl_in.astype(np.float64), plan[0])
    out, lse = mk.mla_merge_splits(t_po, torch.from_numpy(pl_in).to(dev),
                                   torch.from_numpy(plan[0]).to(dev), case.B,
                                   out_dtype=torch.float32)
    assert_close(to_f64(out), ref, "merged")
    assert_lse_close(to_f64(lse), ref_lse, "merged lse")


def test_merge_of_log2_lse_fails_parity(mk):
    """Negative control on the GPU (mlxcel "MLA absorbed decode", Stage 2: an
    lse in log2 units merges into a plausible but wrong average).  The merge
    kernel is given the oracle's partials with their lse converted to log2
    units: its output must FAIL the product tolerance against the exact merge,
    while the same call with natural-log lse passes it.  Partials are drawn so
    that the splits' lse values differ by several units, where the wrong base
    changes the weights by far more than the tolerance."""
    import torch
    log("[merge] negative control: log2-unit lse")
    case = _case("mtp_t4_h32")
    q64 = bits_to_f64(_stage_q_lat(case, 7310)) * 3.0   # sharper scores: lse spread across splits
    plan = oracle.split_plan(case.seqlens, 4, case.page_size)
    po, pl = oracle.latent_attention(case, q64, plan=plan)
    dev = "cuda:0"
    po32 = po.astype(np.float32)
    ref, _ = oracle.merge(po32.astype(np.float64), pl.astype(np.float32).astype(np.float64), plan[0])
    t_po = torch.from_numpy(po32).to(dev)
    ind = torch.from_numpy(plan[0]).to(dev)
    good, _ = mk.mla_merge_splits(t_po, torch.from_numpy(pl.astype(np.float32)).to(dev), ind, case.B,
                                  out_dtype=torch.float32)
    assert_close(to_f64(good), ref, "merged (natural-log lse)")
    pl2 = np.where(np.isfinite(pl), pl / np.log(2.0), pl).astype(np.float32)
    bad, _ = mk.mla_merge_splits(t_po, torch.from_numpy(pl2).to(dev), ind, case.B, out_dtype=torch.float32)
    err = float(np.max(np.abs(to_f64(bad) - ref)))
    t = 1e-2 * float(np.max(np.abs(ref))) + 1e-3
    log(f"  log2-unit lse: max|err| {err:.3e} against tol {t:.3e} (must exceed it)")
    assert np.isfinite(to_f64(bad)).all()
    assert err > t, "a merge fed log2-unit lse passed parity: the control does not discriminate"


def _hot_key_case(name, seed, hot_token, gain=16):
    """A case whose sequence 0 holds, at logical token `hot_token`, a key row
    c = gain * q~[0,0,0,:]: head 0's score there exceeds every earlier score by
    about gain * |q~|^2 * scale (about 200 in log2 units for gain 16), far past
    the first tile's reference.  Returns (case, absorbed-query bits)."""
    case = _case(name)
    ql_bits = _stage_q_lat(case, seed)
    P = case.page_size
    blk, off = int(case.block_table[0, hot_token // P]), hot_token % P
    q0 = bits_to_f64(ql_bits[0, 0, 0, :])
    case.kv_cache[blk, off, :512] = synth.f32_to_bf16_bits((gain * q0).astype(np.float32))
    return case, ql_bits


@pytest.mark.parametrize("S", [1, 2, 0])
@pytest.mark.parametrize("hot_token", [3, 137, 290])
def test_score_growth_past_reference(mk, S, hot_token):
    """A score far above the first tile's maximum (a replay of the work unit
    with a raised reference) gives the same result as ordinary inputs: exact
    softmax, no overflow leaking from the discarded pass."""
    import torch
    log(f"[growth] hot key at {hot_token}, num_splits={S}")
    case, ql_bits = _hot_key_case("v3_b3_l300", 7500 + hot_token, hot_token)
    d = upload(case)
    lat, lse = mk.mla_decode_latent(bf16_tensor(ql_bits, "cuda:0"), d["q_pe"], d["kv_cache"],
                                    d["block_table"], d["seqlens"], case.max_seqlen, SCALE,
                                    num_splits=S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = oracle.latent_attention(case, bits_to_f64(ql_bits))
    # head 0 of sequence 0 attends almost only to the hot row (whose c is 16 q~)
    hot = bits_to_f64(case.kv_cache[int(case.block_table[0, hot_token // case.page_size]),
                                    hot_token % case.page_size, :512])
    assert float(np.max(np.abs(ref_lat[0, 0, 0] - hot))) < 1e-9 * float(np.max(np.abs(hot)))
    assert_close(to_f64(lat), ref_lat, "latent")
    assert_lse_close(to_f64(lse), ref_lse, "lse")


def test_page_placement_is_bitwise_invisible(mk):
    """Accumulation follows logical tokens, so moving pages changes no bit."""
    import torch
    log("[bitwise] permuted vs identity pages")
    case = _case("v3_ragged_b5")
    ident = synth.identity_paged_copy(case)
    ql = bf16_tensor(_stage_q_lat(case, 7400), "cuda:0")
    outs = []
    for c in (case, ident):
        d = upload(c)
        lat, lse = mk.mla_decode_latent(ql, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                        c.max_seqlen, SCALE, out_dtype=torch.float32)
        outs.append((lat.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_deterministic(mk):
    import torch
    log("[bitwise] repeat run")
    case = _case("mtp_t4_h32")
    d = upload(case)
    res = []
    for _ in range(2):
        out, lse = mk.absorbed_decode(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                      d["block_table"], d["seqlens"], case.max_seqlen, num_splits=3)
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_validate_inputs(mk):
    import torch
    log("[validate]")
    case = _case("v3_ragged_b5")
    d = upload(case)
    args = (1, case.max_seqlen, case.page_size, case.num_blocks)
    assert mk.mla_validate_inputs(d["block_table"], d["seqlens"], *args) == 0
    bad = case.block_table.copy()
    bad[2, 0] = case.num_blocks          # out of the pool
    assert mk.mla_validate_inputs(torch.from_numpy(bad).cuda(), d["seqlens"], *args) == -7
    bad = case.block_table.copy()
    bad[4, 3] = -1                       # a needed page left unmapped
    assert mk.mla_validate_inputs(torch.from_numpy(bad).cuda(), d["seqlens"], *args) == -7
    sl = case.seqlens.copy()
    sl[1] = case.max_seqlen + 1
    assert mk.mla_validate_inputs(d["block_table"], torch.from_numpy(sl).cuda(), *args) == -7


@pytest.mark.parametrize("lengths,page", [
    (None, 64),                                   # the ragged case above (5 sequences)
    (tuple(range(100, 100 + 37 * 211, 211)), 64),  # 37 sequences, growing lengths
    ((1, 16, 4000, 9000, 70000), 16),            # one very long sequence, small pages
    ((1, 16, 4000, 9000, 200000), 16),           # a search range of 39 pages: two rounds of 32 candidates
])
def test_auto_split_counts(mk, lengths, page):
    """The automatic split counts equal the rule the header states, evaluated
    here by brute force over every page multiple: the smallest chunk c >= 256
    with sum_b clamp(ceil(L_b/c), 1, 128) <= CUs."""
    import torch
    base = CASES["v3_ragged_b5"]
    wl = base if lengths is None else synth.scaled(base, B=len(lengths), lengths=lengths, page_size=page,
                                                   seed=2110)
    case = synth.make_case(wl)
    d = upload(case)
    log(f"[split auto counts] B={case.B} page={case.page_size}")
    buf = mk.DecodeBuffers(case.B, case.T, case.H, case.max_seqlen, case.page_size, 0, "cuda:0")
    q_lat = bf16_tensor(_stage_q_lat(case, 7400), "cuda:0")
    mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                         case.max_seqlen, SCALE, num_splits=0, buffers=buf, merge=False)
    torch.cuda.synchronize()
    counts = np.diff(buf.split_indptr.cpu().numpy())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    target = cus // ((case.T * case.H + 127) // 128)
    L = case.seqlens.astype(np.int64)
    P = case.page_size

    def split(c):
        return np.clip(-(-L // c), 1, 128)

    kmax = max(1, -(-int(L.max()) // P))
    if case.B >= target:
        want = split(kmax * P)
    else:
        want = None
        for k in range(-(-256 // P), max(-(-256 // P), kmax) + 1):
            if split(k * P).sum() <= target:
                want = split(k * P)
                break
    assert want is not None
    assert np.array_equal(counts, want), (counts, want)
