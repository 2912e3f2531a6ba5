"""The decode step captured as a HIP graph: every replay, with eager work and
synchronisations between replays, gives exactly the eager result (the kernels
are deterministic, so the comparison is bitwise).  The step takes the merge and
un-absorb as two kernels and, as the benchmark's step does for bf16 partials
and up to four splits, as one (mla_merge_unabsorb)."""
import numpy as np
import pytest

import synth
from tests.gpu_util import SCALE, log, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mk():
    import torch
    import mla_latent_kv_amd as mk
    mk.load_library()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return mk


@pytest.mark.parametrize("S, fused", [(1, False), (4, False), (0, False), (4, True), (2, True)])
def test_graph_replays_match_eager(mk, S, fused):
    import torch
    log(f"[graph] num_splits={S} fused={fused}")
    wl = synth.scaled(synth.WORKLOADS["v3_b64_l4096"], B=3, T=2, L=300, lengths=(300, 131, 77), seed=2201)
    case = synth.make_case(wl)
    d = upload(case)
    B, T, H = case.B, case.T, case.H
    dev = "cuda:0"
    buf = mk.DecodeBuffers(B, T, H, case.max_seqlen, case.page_size, S, dev,
                           part_dtype=torch.bfloat16) if S != 1 else None
    q_lat = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device=dev)
    latent = torch.empty((B, T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    out = torch.empty((B, T, H, 128), dtype=torch.float32, device=dev)

    def step():
        mk.mla_absorb_q(d["q_nope"], d["w_uk"], q_lat=q_lat)
        if S == 1:
            mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                 case.max_seqlen, SCALE, num_splits=1, out_latent=latent, lse=lse)
        else:
            mk.mla_decode_latent(q_lat, d["q_pe"], d["kv_cache"], d["block_table"], d["seqlens"],
                                 case.max_seqlen, SCALE, num_splits=S, buffers=buf, merge=False)
            if fused:
                mk.mla_merge_unabsorb(buf.part_out, buf.part_lse, buf.split_indptr, d["w_uv"], B, out=out,
                                      lse=lse)
                return
            mk.mla_merge_splits(buf.part_out, buf.part_lse, buf.split_indptr, B, out_latent=latent,
                                lse=lse)
        mk.mla_unabsorb_out(latent, d["w_uv"], out=out)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), latent.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    checked = (("out", 0), ("lse", 1)) if fused else (("out", 0), ("lse", 1), ("latent", 2))
    for rep in range(4):
        # eager work between replays that overwrites every output
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        latent.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        now = (out, lse, latent)
        for what, i in checked:
            assert torch.equal(now[i], ref[i]), f"replay {rep}: {what} differs from the eager result"
