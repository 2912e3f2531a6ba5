"""The seeded input recipe: encodings, paging layout, poison (no GPU)."""
import numpy as np
import torch

import synth


def test_bf16_encoding_matches_torch_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37.0
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 0.0]     # exact ties both ways
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ragged_layout_and_unused_fraction():
    wl = synth.scaled(synth.WORKLOADS["v3_ragged_b128"], B=40)
    case = synth.make_case(wl)
    L = case.seqlens
    assert L.min() >= 64 and L.max() <= 16384
    pages = (L + 63) // 64
    used = case.block_table[case.block_table >= 0]
    assert len(used) == pages.sum() == len(np.unique(used))
    frac_unused = 1.0 - len(used) / case.num_blocks
    assert 0.09 <= frac_unused <= 0.11
    for b in range(case.B):
        assert (case.block_table[b, :pages[b]] >= 0).all()
        assert (case.block_table[b, pages[b]:] == -1).all()


def test_poison_marks_every_unreadable_row():
    wl = synth.Workload("p", B=3, T=1, H=2, L=0, page_size=16, seed=3, lengths=(20, 16, 5),
                        unused_frac=0.25)
    case = synth.make_case(wl)
    nan = synth.BF16_NAN
    readable = np.zeros(case.kv_cache.shape[:2], bool)
    for b in range(case.B):
        for j in range(int(case.seqlens[b])):
            readable[case.block_table[b, j // 16], j % 16] = True
    assert (case.kv_cache[~readable] == nan).all()
    assert not (case.kv_cache[readable] == nan).any()


def test_same_seed_same_bits_and_draw_distribution():
    wl = synth.scaled(synth.WORKLOADS["v3_b64_l4096"], B=2, L=256)
    a, b = synth.make_case(wl), synth.make_case(wl)
    for k in ("q_nope", "q_pe", "w_uk", "w_uv", "kv_cache", "block_table", "seqlens"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    w = synth.bf16_bits_to_f32(a.w_uk).astype(np.float64)
    assert abs(w.var() * 512 - 1.0) < 0.02          # N(0, 1/512): variance 1/512
    q = synth.bf16_bits_to_f32(a.q_nope).astype(np.float64)
    assert abs(q.var() - 1.0) < 0.05


def test_contiguous_tiny_workload():
    case = synth.make_case(synth.WORKLOADS["v2lite_tiny"])
    assert case.kv_cache.shape == (1, 256, 576)
    assert case.block_table.tolist() == [[0]]
    assert case.q_nope.shape == (1, 1, 16, 128)


def test_fp8_rows_layout_and_poison():
    """FP8 rows: 656 bytes; codes never NaN in readable rows, NaN codes and
    scales in every other row; the rope bytes are make_case's bf16 rope
    columns; same seed, same bytes; scales in [2^-10, 2^-6]."""
    wl = synth.scaled(synth.WORKLOADS["v3_ragged_b128"], B=3, ragged=None, lengths=(5, 64, 150), seed=77)
    f = synth.make_fp8_case(wl)
    g = synth.make_fp8_case(wl)
    assert np.array_equal(f.kv_fp8, g.kv_fp8)
    c = f.case
    assert f.kv_fp8.shape == c.kv_cache.shape[:2] + (656,) and f.kv_fp8.dtype == np.uint8
    readable = np.zeros(c.kv_cache.shape[:2], dtype=bool)
    for b in range(c.B):
        for j in range(int(c.seqlens[b])):
            readable[c.block_table[b, j // c.page_size], j % c.page_size] = True
    codes = f.kv_fp8[..., :512]
    nan_code = (codes & 0x7F) == 0x7F
    assert not nan_code[readable].any() and nan_code[~readable].all()
    sc = np.ascontiguousarray(f.kv_fp8[..., 512:528]).view("<f4")
    assert np.isnan(sc[~readable]).all()
    live = sc[readable]
    assert (live >= 2.0 ** -10).all() and (live <= 2.0 ** -6).all()
    rope = np.ascontiguousarray(f.kv_fp8[..., 528:]).view("<u2")
    assert np.array_equal(rope, c.kv_cache[..., 512:])
    # magnitude codes centred near 108 (the value 96), both signs
    mag = (codes[readable] & 0x7F).astype(np.float64)
    assert abs(mag.mean() - 108) < 1.0 and 0.45 < (codes[readable] >> 7).mean() < 0.55
