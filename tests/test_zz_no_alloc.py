"""GPU test of mla_decode_latent_noalloc, the entry point that keeps its split
scratch in the library's own device array: two calls in a row, the second on
a smaller input, each compared element by element with mla_decode_latent run
on the same inputs with caller buffers (bf16 partials, the same split mode),
and with the fp64 absorbed mirror to the product tolerance.  The second call
reuses the array the first one left behind."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import SCALE, assert_close, assert_lse_close, bf16_tensor, bits_to_f64, log, to_f64, upload

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


def _compare(mk, case, S, seed):
    import torch
    d = upload(case)
    ql_bits = synth.normal_bf16(case.q_nope.shape[:3] + (512,), seed, std=0.5)
    ql = bf16_tensor(ql_bits, "cuda:0")
    B, T, H = case.B, case.T, case.H
    out_n = torch.full((B, T, H, 512), float("nan"), dtype=torch.float32, device="cuda:0")
    lse_n = torch.full((B, T, H), float("nan"), dtype=torch.float32, device="cuda:0")
    mk.mla_decode_latent_noalloc(ql, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"], case.max_seqlen,
                                 SCALE, num_splits=S, out_latent=out_n, lse=lse_n)
    buf = mk.DecodeBuffers(B, T, H, case.max_seqlen, case.page_size, S, "cuda:0", part_dtype=torch.bfloat16)
    out_c, lse_c = mk.mla_decode_latent(ql, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                        case.max_seqlen, SCALE, num_splits=S, out_dtype=torch.float32, buffers=buf)
    torch.cuda.synchronize()
    got, got_lse = to_f64(out_n), to_f64(lse_n)
    # same kernels, same plan, same inputs: the same bits
    assert np.array_equal(got, to_f64(out_c)), "no-alloc output differs from mla_decode_latent's"
    assert np.array_equal(got_lse, to_f64(lse_c)), "no-alloc lse differs from mla_decode_latent's"
    ref, ref_lse = oracle.latent_attention(case, bits_to_f64(ql_bits))
    assert_close(got, ref, "latent vs fp64 mirror")
    assert_lse_close(got_lse, ref_lse, "lse vs fp64 mirror")


@pytest.mark.parametrize("S", [0, 4])
def test_noalloc_two_calls_second_smaller(mk, S):
    first = synth.make_case(W["v3_b64_l4096"])                       # 64 x 4096, 128 heads
    second = synth.make_case(synth.scaled(W["v3_mtp_b32_t4_h32"], B=3, lengths=(100, 4, 77), seed=2203))
    log(f"[noalloc] S={S}: call 1 on {first.B} x {first.max_seqlen} (H={first.H})")
    _compare(mk, first, S, 9400 + S)
    log(f"[noalloc] S={S}: call 2 on {second.B} sequences of up to {second.max_seqlen} (T={second.T}, H={second.H})")
    _compare(mk, second, S, 9500 + S)
