"""The oracle's closed-form byte/FLOP counts against the values the pages print
(tests/golden/closed_forms.txt lists each value with its passage)."""
import os

import pytest

from oracle import costs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


def _golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value, tol, src = [x.strip() for x in line.split("|", 3)]
            rows[name] = (float(value), float(tol), src)
    return rows


G = _golden()

COMPUTED = {
    "latent_bytes_per_token_layer": lambda: costs.latent_bytes_per_token_layer(),
    "decompressed_bytes_h128": lambda: costs.decompressed_bytes_per_token_layer(128),
    "decompressed_bytes_h16": lambda: costs.decompressed_bytes_per_token_layer(16),
    "decompressed_ratio_h128": lambda: costs.decompressed_bytes_per_token_layer(128)
    / costs.latent_bytes_per_token_layer(),
    "decompressed_ratio_h16": lambda: costs.decompressed_bytes_per_token_layer(16)
    / costs.latent_bytes_per_token_layer(),
    "naive_upprojection_flops_per_token": lambda: costs.naive_upprojection_flops_per_token(),
    "absorbed_core_flops_per_pair": lambda: costs.absorbed_core_flops_per_pair(),
    "normal_core_flops_per_pair": lambda: costs.normal_core_flops_per_pair(),
    "core_ratio": lambda: costs.absorbed_core_flops_per_pair() / costs.normal_core_flops_per_pair(),
    "core_flops_4096_ctx": lambda: costs.absorbed_core_flops_per_pair() * 4096,
    "fold_flops_per_query": lambda: costs.fold_flops_per_query(),
    "core_flops_61_layers_4096": lambda: costs.absorbed_core_flops_per_pair() * 4096 * 61,
    "cache_bytes_61_layers_4096": lambda: costs.model_cache_bytes_per_token(61) * 4096,
    "decode_intensity_tp1": lambda: costs.decode_intensity(tp=1),
    "decode_intensity_tp8": lambda: costs.decode_intensity(tp=8),
    "cache_bytes_per_token_61_layers": lambda: costs.model_cache_bytes_per_token(61),
    "expanded_mib_per_token_61_layers": lambda: 61 * costs.decompressed_bytes_per_token_layer(128)
    / 2**20,
    "expanded_to_latent_ratio_61_layers": lambda: costs.decompressed_bytes_per_token_layer(128)
    / costs.latent_bytes_per_token_layer(),
    "cache_kib_per_token_60_layers": lambda: costs.model_cache_bytes_per_token(60) / 1024,
    "cache_mib_60_layers_4096": lambda: costs.model_cache_bytes_per_token(60) * 4096 / 2**20,
    "causal_pairs_q3_p5": lambda: costs.causal_pairs(3, 5),
    "fp8_row_bytes": lambda: costs.fp8_row_bytes(),
    "fp8_row_ratio": lambda: costs.fp8_row_bytes() / costs.latent_bytes_per_token_layer(),
    "rectangular_query_bound": lambda: costs.rectangular_query_bound(),
    "vllm_workspace_latent_bytes": lambda: costs.latent_bytes_per_token_layer() * 65536,
    "vllm_workspace_expanded_bytes": lambda: 2 * 192 * 128 * 65536,
}


@pytest.mark.parametrize("name", sorted(G))
def test_closed_form(name):
    value, tol, src = G[name]
    got = COMPUTED[name]()
    if tol == 0:
        assert got == value, (name, got, value, src)
    else:
        assert abs(got - value) <= tol * abs(value), (name, got, value, src)


def test_every_golden_row_is_checked():
    assert set(G) == set(COMPUTED)


def test_teaching_crossover_is_about_one_token():
    # M5.8 0x04: with d_N=128, d_c=512 the historical expansion dominates
    # almost immediately; the crossover sits just above one cached token.
    x = costs.teaching_crossover()
    assert 1.0 < x < 1.01
