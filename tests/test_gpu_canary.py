"""Every output and scratch buffer of every entry point placed inside
sentinel-filled padding: after the call (and after the merge that reads the
partials), the padding must be unchanged -- no kernel writes outside the
region its sizes give it.  Sizes are ragged (partial last tiles, empty
trailing chunks) so that the edge paths run."""
import numpy as np
import pytest

import synth
from tests.gpu_util import SCALE, bf16_tensor, log, upload

pytestmark = pytest.mark.gpu

PAD = 4096          # bytes of sentinel on each side (a multiple of 16: alignment kept)
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


class Canaried:
    """Tensors carved out of sentinel-filled byte buffers."""

    def __init__(self):
        self.raw = []

    def new(self, shape, dtype, fill=None):
        import torch
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        raw = torch.full((n + 2 * PAD,), SENTINEL, dtype=torch.uint8, device="cuda:0")
        t = raw[PAD:PAD + n].view(dtype).view(shape)
        if fill is not None:
            t.copy_(fill)
        self.raw.append((raw, n))
        return t

    def check(self, what):
        import torch
        torch.cuda.synchronize()
        for i, (raw, n) in enumerate(self.raw):
            head, tail = raw[:PAD], raw[PAD + n:]
            assert bool((head == SENTINEL).all()) and bool((tail == SENTINEL).all()), \
                f"{what}: buffer {i} written outside its region"


def _case():
    wl = synth.scaled(synth.WORKLOADS["v3_ragged_b128"], B=5, ragged=None, lengths=(1, 17, 64, 250, 1000),
                      seed=2701)
    return synth.make_case(wl)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("S", [1, 3, 0])
def test_decode_chain_writes_stay_in_bounds(mk, S, fp8):
    import torch
    log(f"[canary] decode chain S={S} fp8={fp8}")
    if fp8:
        f = synth.make_fp8_case(synth.scaled(synth.WORKLOADS["v3_ragged_b128"], B=5, ragged=None,
                                             lengths=(1, 17, 64, 250, 1000), seed=2701))
        case = f.case
    else:
        case = _case()
    d = upload(case)
    cn = Canaried()
    B, T, H = case.B, case.T, case.H
    kv = cn.new(f.kv_fp8.shape, torch.uint8, torch.from_numpy(f.kv_fp8)) if fp8 else \
        cn.new(tuple(d["kv_cache"].shape), torch.bfloat16, d["kv_cache"])
    q_lat = cn.new((B, T, H, 512), torch.bfloat16)
    mk.mla_absorb_q(d["q_nope"], d["w_uk"], q_lat=q_lat)
    lat = cn.new((B, T, H, 512), torch.bfloat16)
    lse = cn.new((B, T, H), torch.float32)
    dec = mk.mla_decode_latent_fp8 if fp8 else mk.mla_decode_latent
    if S == 1:
        dec(q_lat, d["q_pe"], kv, d["block_table"], d["seqlens"], case.max_seqlen, SCALE, num_splits=1,
            out_latent=lat, lse=lse)
    else:
        buf = mk.DecodeBuffers(B, T, H, case.max_seqlen, case.page_size, S, "cuda:0", part_dtype=torch.bfloat16)
        buf.workspace = cn.new(tuple(buf.workspace.shape), torch.uint8)
        buf.part_out = cn.new(tuple(buf.part_out.shape), torch.bfloat16)
        buf.part_lse = cn.new(tuple(buf.part_lse.shape), torch.float32)
        buf.split_indptr = cn.new(tuple(buf.split_indptr.shape), torch.int32)
        dec(q_lat, d["q_pe"], kv, d["block_table"], d["seqlens"], case.max_seqlen, SCALE, num_splits=S,
            buffers=buf, merge=False)
        mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, B, out_latent=lat, lse=lse)
    out = cn.new((B, T, H, 128), torch.float32)
    mk.mla_unabsorb_out(lat, d["w_uv"], out=out)
    cn.check(f"decode chain S={S} fp8={fp8}")
    assert bool(torch.isfinite(out).all())


def test_append_writes_stay_in_bounds(mk):
    import torch
    log("[canary] append")
    case = _case()
    d = upload(case)
    cn = Canaried()
    kv = cn.new(tuple(d["kv_cache"].shape), torch.bfloat16, d["kv_cache"])
    c_new = bf16_tensor(synth.normal_bf16((case.B, case.T, 512), 2702), "cuda:0")
    kpe_new = bf16_tensor(synth.normal_bf16((case.B, case.T, 64), 2703), "cuda:0")
    mk.mla_append_cache(c_new, kpe_new, kv, d["block_table"], d["seqlens"])
    cn.check("append")


@pytest.mark.parametrize("S", [1, 3])
def test_sparse_writes_stay_in_bounds(mk, S):
    import torch
    log(f"[canary] sparse S={S}")
    wl = synth.Workload("sp", B=3, T=2, H=16, L=0, page_size=16, seed=2704, lengths=(300, 40, 97))
    sc = synth.make_sparse(wl, 64)
    cn = Canaried()
    lat = cn.new((sc.B, sc.T, sc.H, 512), torch.float32)
    lse = cn.new((sc.B, sc.T, sc.H), torch.float32)
    buf = mk.SparseBuffers(sc.B, sc.T, sc.H, sc.topk, S, "cuda:0", part_dtype=torch.bfloat16)
    if buf.part_out is not None:
        buf.part_out = cn.new(tuple(buf.part_out.shape), torch.bfloat16)
        buf.part_lse = cn.new(tuple(buf.part_lse.shape), torch.float32)
        buf.split_indptr = cn.new(tuple(buf.split_indptr.shape), torch.int32)
    mk.mla_decode_sparse(bf16_tensor(sc.q_lat, "cuda:0"), bf16_tensor(sc.q_pe, "cuda:0"),
                         bf16_tensor(sc.kv_cache, "cuda:0"), torch.from_numpy(sc.indices).to("cuda:0"),
                         torch.from_numpy(sc.topk_length).to("cuda:0"), SCALE, num_splits=S, buffers=buf,
                         out_latent=lat, lse=lse)
    cn.check(f"sparse S={S}")


def test_normal_path_writes_stay_in_bounds(mk):
    import torch
    log("[canary] Normal path")
    case = _case()
    d = upload(case)
    cn = Canaried()
    chunk = 128
    ws = cn.new((max(mk.mla_normal_workspace_size(case.B, case.T, case.H, case.max_seqlen, chunk), 16),),
                torch.uint8)
    out = cn.new((case.B, case.T, case.H, 128), torch.float32)
    lse = cn.new((case.B, case.T, case.H), torch.float32)
    mk.mla_decode_normal(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
                         d["seqlens"], case.max_seqlen, SCALE, chunk=chunk, workspace=ws, out=out, lse=lse)
    cn.check("normal path")
