"""GPU parity of sparse (top-k) decode (mla_decode_sparse) against the
oracle's sparse latent attention, on seeded selections: single pass, uniform
and automatic splits, multi-token rows, fewer than 128 heads, valid prefixes
down to zero, repeated ids, no topk_length, a pool larger than 4 GiB (64-bit
row addresses) and the full 64 x 2048-of-32768 workload.  Every cache row no
index selects is NaN, so a stray read shows up."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import SCALE, assert_close, assert_lse_close, bf16_tensor, log, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()  # raises if the HIP library is missing
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


W = synth.WORKLOADS["v3_b64_l4096"]

CASES = {
    "b3_h128": (synth.scaled(W, B=3, lengths=(1000, 400, 300), seed=2301), 300, {}),
    "ragged_valid": (synth.scaled(W, B=4, lengths=(2000, 50, 700, 33), seed=2302), 256,
                     dict(valid=(256, 50, 17, 0))),
    "t2_h64": (synth.scaled(W, B=2, T=2, H=64, lengths=(500, 800), seed=2303), 200, {}),
    "dup_h16": (synth.scaled(W, B=2, H=16, lengths=(300, 300), seed=2304), 128, dict(duplicates=True)),
    "no_length": (synth.scaled(W, B=2, lengths=(512, 600), seed=2305), 256, dict(use_length=False)),
    "t4_h32_p16": (synth.scaled(W, B=2, T=4, H=32, page_size=16, lengths=(100, 70), seed=2306), 64, {}),
}


def _upload(sc, dev="cuda:0"):
    import torch
    return dict(q_lat=bf16_tensor(sc.q_lat, dev), q_pe=bf16_tensor(sc.q_pe, dev),
                kv_cache=bf16_tensor(sc.kv_cache, dev),
                indices=torch.from_numpy(sc.indices).to(dev),
                topk_length=None if sc.topk_length is None else torch.from_numpy(sc.topk_length).to(dev))


def _check(lat, lse, ref_lat, ref_lse, what):
    got_lse = to_f64(lse)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), f"{what}: empty rows differ"
    assert (to_f64(lat)[empty] == 0).all(), f"{what}: empty rows not zero"
    full = ~empty
    assert_close(to_f64(lat)[full], ref_lat[full], f"{what} latent")
    assert_lse_close(got_lse[full], ref_lse[full], f"{what} lse")


def _oracle(sc):
    return oracle.sparse_latent_attention(oracle.bf16_to_f64(sc.q_lat), sc.q_pe, sc.kv_cache, sc.indices,
                                          sc.topk_length, SCALE)


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_parity(mk, name, splits):
    import torch
    wl, topk, kw = CASES[name]
    log(f"[sparse] {name} topk={topk} splits={splits}")
    sc = synth.make_sparse(wl, topk, **kw)
    d = _upload(sc)
    lat, lse = mk.mla_decode_sparse(d["q_lat"], d["q_pe"], d["kv_cache"], d["indices"], d["topk_length"],
                                    SCALE, num_splits=splits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(sc)
    _check(lat, lse, ref_lat, ref_lse, name)


def test_sparse_bf16_output_and_partials(mk):
    """bf16 output and bf16 split partials, merged separately."""
    import torch
    log("[sparse] bf16 partials, separate merge")
    wl, topk, kw = CASES["b3_h128"]
    sc = synth.make_sparse(wl, topk, **kw)
    d = _upload(sc)
    buf = mk.SparseBuffers(sc.B, sc.T, sc.H, topk, 2, "cuda:0", part_dtype=torch.bfloat16)
    mk.mla_decode_sparse(d["q_lat"], d["q_pe"], d["kv_cache"], d["indices"], d["topk_length"], SCALE,
                         num_splits=2, buffers=buf, merge=False)
    BT = sc.B * sc.T
    lat, lse = mk.mla_merge_splits(buf.part_out.view(BT * 2, 1, sc.H, 512),
                                   buf.part_lse.view(BT * 2, 1, sc.H), buf.split_indptr, BT)
    torch.cuda.synchronize()
    assert buf.split_indptr.cpu().numpy().tolist() == list(range(0, 2 * BT + 1, 2))
    ref_lat, ref_lse = _oracle(sc)
    _check(lat.view(sc.B, sc.T, sc.H, 512), lse.view(sc.B, sc.T, sc.H), ref_lat, ref_lse, "bf16 partials")


def test_sparse_pool_beyond_4gib(mk):
    """The selected rows sit above byte 4 GiB of a 4.6 GB pool: row addresses
    need 64 bits."""
    import torch
    log("[sparse] pool beyond 4 GiB")
    wl, topk, kw = CASES["b3_h128"]
    sc = synth.make_sparse(wl, topk, **kw)
    P = sc.page_size
    big_blocks = 62_500                     # 4.0M rows of 1152 bytes = 4.6 GB
    off_blocks = big_blocks - sc.num_blocks
    assert off_blocks * P * 1152 > (1 << 32)
    pool = torch.empty((big_blocks, P, 576), dtype=torch.bfloat16, device="cuda:0")
    pool.view(torch.int16).fill_(int(np.int16(np.uint16(synth.BF16_NAN).view(np.int16))))
    pool[off_blocks:] = bf16_tensor(sc.kv_cache, "cuda:0")
    idx = sc.indices.astype(np.int64)
    n = sc.topk_length
    for b in range(sc.B):
        idx[b, :, :n[b]] += off_blocks * P
    d = _upload(sc)
    lat, lse = mk.mla_decode_sparse(d["q_lat"], d["q_pe"], pool,
                                    torch.from_numpy(idx.astype(np.int32)).to("cuda:0"), d["topk_length"],
                                    SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(sc)
    _check(lat, lse, ref_lat, ref_lse, "pool beyond 4 GiB")
    del pool
    torch.cuda.empty_cache()


def test_sparse_full_workload(mk):
    """64 sequences of 32768 tokens, 2048 selected per query token, 128 heads,
    automatic splits (the configuration the benchmark times); every output
    element against the oracle."""
    import torch
    log("[sparse] full workload b64 topk2048 of 32768")
    sc = synth.make_sparse(synth.SPARSE_WORKLOADS["v3_sparse_b64_topk2048"], 2048)
    d = _upload(sc)
    lat, lse = mk.mla_decode_sparse(d["q_lat"], d["q_pe"], d["kv_cache"], d["indices"], d["topk_length"],
                                    SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(sc)
    _check(lat, lse, ref_lat, ref_lse, "full workload")
