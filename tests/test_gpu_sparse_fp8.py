"""GPU parity of sparse (top-k) decode over FP8 rows (mla_decode_sparse_fp8;
M5.8 0x0B: the sparse path reads the 656-byte FP8 row and dequantizes the
selected rows to bf16) against the oracle's sparse latent attention over the
oracle's dequantized rows: single pass, uniform and automatic splits,
multi-token rows, fewer than 128 heads, valid prefixes down to zero, repeated
ids, no topk_length, bf16 partials with a separate merge, a pool larger than
4 GiB (64-bit row addresses) and the full 64 x 2048-of-32768 workload.  Every
row no index selects holds NaN codes, scales and rope values.  Where no
selected element's fp32 product sits on a bf16 tie, the result must also equal,
bit for bit, the bf16 sparse kernel run on the oracle's dequantized rows."""
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
    mk.load_library()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


W = synth.WORKLOADS["v3_b64_l4096"]

CASES = {
    "b3_h128": (synth.scaled(W, B=3, lengths=(1000, 400, 300), seed=2701), 300, {}),
    "ragged_valid": (synth.scaled(W, B=4, lengths=(2000, 50, 700, 33), seed=2702), 256,
                     dict(valid=(256, 50, 17, 0))),
    "t2_h64": (synth.scaled(W, B=2, T=2, H=64, lengths=(500, 800), seed=2703), 200, {}),
    "dup_h16": (synth.scaled(W, B=2, H=16, lengths=(300, 300), seed=2704), 128, dict(duplicates=True)),
    "no_length": (synth.scaled(W, B=2, lengths=(512, 600), seed=2705), 256, dict(use_length=False)),
    "t4_h32_p16": (synth.scaled(W, B=2, T=4, H=32, page_size=16, lengths=(100, 70), seed=2706), 64, {}),
}


def _upload(f, dev="cuda:0"):
    import torch
    sc = f.sparse
    return dict(q_lat=bf16_tensor(sc.q_lat, dev), q_pe=bf16_tensor(sc.q_pe, dev),
                kv_fp8=torch.from_numpy(f.kv_fp8).to(dev),
                indices=torch.from_numpy(sc.indices).to(dev),
                topk_length=None if sc.topk_length is None else torch.from_numpy(sc.topk_length).to(dev))


def _oracle(f):
    sc = f.sparse
    return oracle.sparse_latent_attention(oracle.bf16_to_f64(sc.q_lat), sc.q_pe, oracle.fp8_rows_to_bf16(f.kv_fp8),
                                          sc.indices, sc.topk_length, SCALE)


def _check(lat, lse, ref_lat, ref_lse, what):
    got_lse = to_f64(lse)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty), f"{what}: empty rows differ"
    assert (to_f64(lat)[empty] == 0).all(), f"{what}: empty rows not zero"
    full = ~empty
    assert_close(to_f64(lat)[full], ref_lat[full], f"{what} latent")
    assert_lse_close(got_lse[full], ref_lse[full], f"{what} lse")


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_fp8_parity(mk, name, splits):
    import torch
    wl, topk, kw = CASES[name]
    log(f"[sparse fp8] {name} topk={topk} splits={splits}")
    f = synth.make_sparse_fp8(wl, topk, **kw)
    d = _upload(f)
    lat, lse = mk.mla_decode_sparse_fp8(d["q_lat"], d["q_pe"], d["kv_fp8"], d["indices"], d["topk_length"],
                                        SCALE, num_splits=splits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(f)
    _check(lat, lse, ref_lat, ref_lse, name)


def _selected_rows_tie_free(f):
    """True when no selected row holds an element whose fp32 product code x
    scale lies on a bf16 tie (there the kernel, rounding the fp32 product,
    and the oracle, rounding the exact product, may differ by one ulp)."""
    import torch
    sc = f.sparse
    flat = f.kv_fp8.reshape(-1, 656)
    sel = np.unique(np.concatenate([sc.indices[b, t, :(sc.topk if sc.topk_length is None else sc.topk_length[b])]
                                    for b in range(sc.B) for t in range(sc.T)] + [np.empty(0, np.int32)]))
    rows = flat[sel.astype(np.int64)]
    codes = torch.from_numpy(np.ascontiguousarray(rows[:, :512])).view(torch.float8_e4m3fn).to(torch.float32)
    scales = torch.from_numpy(np.ascontiguousarray(rows[:, 512:528]).view("<f4").copy())
    via32 = (codes.view(-1, 4, 128) * scales[:, :, None]).reshape(-1, 512).to(torch.bfloat16)
    return np.array_equal(via32.view(torch.int16).numpy().view(np.uint16), oracle.fp8_rows_to_bf16(rows)[:, :512])


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("name", ["b3_h128", "t2_h64", "t4_h32_p16"])
def test_sparse_fp8_equals_bf16_sparse_kernel_on_dequantized_rows(mk, name, splits):
    import torch
    wl, topk, kw = CASES[name]
    log(f"[sparse fp8 vs bf16 rows] {name} splits={splits}")
    f = synth.make_sparse_fp8(wl, topk, **kw)
    d = _upload(f)
    kv_bf16 = bf16_tensor(oracle.fp8_rows_to_bf16(f.kv_fp8), "cuda:0")
    a = mk.mla_decode_sparse_fp8(d["q_lat"], d["q_pe"], d["kv_fp8"], d["indices"], d["topk_length"], SCALE,
                                 num_splits=splits, out_dtype=torch.float32)
    b = mk.mla_decode_sparse(d["q_lat"], d["q_pe"], kv_bf16, d["indices"], d["topk_length"], SCALE,
                             num_splits=splits, out_dtype=torch.float32)
    torch.cuda.synchronize()
    exact = _selected_rows_tie_free(f)
    log(f"  selected rows free of fp32 ties: {exact}")
    if exact:
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert_close(to_f64(a[0]), to_f64(b[0]), "latent vs bf16 sparse kernel")


def test_sparse_fp8_bf16_partials_separate_merge(mk):
    import torch
    log("[sparse fp8] bf16 partials, separate merge")
    wl, topk, kw = CASES["b3_h128"]
    f = synth.make_sparse_fp8(wl, topk, **kw)
    sc = f.sparse
    d = _upload(f)
    buf = mk.SparseBuffers(sc.B, sc.T, sc.H, topk, 2, "cuda:0", part_dtype=torch.bfloat16)
    mk.mla_decode_sparse_fp8(d["q_lat"], d["q_pe"], d["kv_fp8"], d["indices"], d["topk_length"], SCALE,
                             num_splits=2, buffers=buf, merge=False)
    BT = sc.B * sc.T
    lat, lse = mk.mla_merge_splits(buf.part_out.view(BT * 2, 1, sc.H, 512), buf.part_lse.view(BT * 2, 1, sc.H),
                                   buf.split_indptr, BT)
    torch.cuda.synchronize()
    assert buf.split_indptr.cpu().numpy().tolist() == list(range(0, 2 * BT + 1, 2))
    ref_lat, ref_lse = _oracle(f)
    _check(lat.view(sc.B, sc.T, sc.H, 512), lse.view(sc.B, sc.T, sc.H), ref_lat, ref_lse, "bf16 partials")


def test_sparse_fp8_pool_beyond_4gib(mk):
    """The selected rows sit above byte 4 GiB of a 4.3 GB FP8 pool: row
    addresses need 64 bits."""
    import torch
    log("[sparse fp8] pool beyond 4 GiB")
    wl, topk, kw = CASES["b3_h128"]
    f = synth.make_sparse_fp8(wl, topk, **kw)
    sc = f.sparse
    P = sc.page_size
    nb = f.kv_fp8.shape[0]
    big_blocks = 102_500                    # 6.56M rows of 656 bytes = 4.3 GB
    off_blocks = big_blocks - nb
    assert off_blocks * P * 656 > (1 << 32)
    pool = torch.full((big_blocks, P, 656), 0x7F, dtype=torch.uint8, device="cuda:0")   # NaN codes
    pool[off_blocks:] = torch.from_numpy(f.kv_fp8).to("cuda:0")
    idx = sc.indices.astype(np.int64)
    n = sc.topk_length
    for b in range(sc.B):
        idx[b, :, :n[b]] += off_blocks * P
    d = _upload(f)
    lat, lse = mk.mla_decode_sparse_fp8(d["q_lat"], d["q_pe"], pool,
                                        torch.from_numpy(idx.astype(np.int32)).to("cuda:0"), d["topk_length"],
                                        SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(f)
    _check(lat, lse, ref_lat, ref_lse, "pool beyond 4 GiB")
    del pool
    torch.cuda.empty_cache()


def test_sparse_fp8_full_workload(mk):
    """64 sequences of 32768 tokens, 2048 selected per query token, 128 heads,
    automatic splits, FP8 rows; every output element against the oracle."""
    import torch
    log("[sparse fp8] full workload b64 topk2048 of 32768")
    f = synth.make_sparse_fp8(synth.SPARSE_WORKLOADS["v3_sparse_b64_topk2048"], 2048)
    d = _upload(f)
    lat, lse = mk.mla_decode_sparse_fp8(d["q_lat"], d["q_pe"], d["kv_fp8"], d["indices"], d["topk_length"],
                                        SCALE, num_splits=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref_lat, ref_lse = _oracle(f)
    _check(lat, lse, ref_lat, ref_lse, "full workload")
