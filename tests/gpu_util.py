"""Helpers shared by the GPU parity tests: device upload of seeded cases,
the product tolerance, and sampling of (b, h) pairs for full-size checks."""
from __future__ import annotations

import math
import sys

import numpy as np

D_NOPE, D_ROPE = 128, 64
SCALE = 1.0 / math.sqrt(D_NOPE + D_ROPE)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol(ref) -> float:
    """max|err| <= 1e-2 * max|ref| + 1e-3 over the compared elements."""
    ref = np.asarray(ref, dtype=np.float64)
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(ref).all(), what
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(got - ref)))
    t = tol(ref)
    log(f"  {what}: max|err| {err:.3e}  tol {t:.3e}  max|ref| {np.max(np.abs(ref)):.3e}")
    assert err <= t, f"{what}: max|err| {err} > tol {t}"


# Absolute bound on lse.  A split's merge weight is exp(lse_k - M), so an lse
# error d scales that weight by exp(d): |d| <= 1e-2 keeps every weight within
# about 1% (the log-sum-exp merge contract of mlxcel "MLA absorbed decode",
# Stage 2, and of M5.8 0x0C).  The output tolerance above, 1e-2 * max|lse| + 1e-3,
# would allow 0.06-0.1 on lse values of 6-12 (ln of the context length).
LSE_ABS_TOL = 1e-2


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(ref).all(), what
    assert np.isfinite(got).all(), f"{what}: non-finite GPU lse"
    err = float(np.max(np.abs(got - ref)))
    log(f"  {what}: max|err| {err:.3e}  abs tol {LSE_ABS_TOL:.1e}  max|ref| {np.max(np.abs(ref)):.3e}")
    assert err <= LSE_ABS_TOL, f"{what}: max|err| {err} > {LSE_ABS_TOL}"


def bf16_tensor(bits, dev):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev)


def upload(case, dev="cuda:0"):
    import torch
    return dict(
        q_nope=bf16_tensor(case.q_nope, dev),
        q_pe=bf16_tensor(case.q_pe, dev),
        w_uk=bf16_tensor(case.w_uk, dev),
        w_uv=bf16_tensor(case.w_uv, dev),
        kv_cache=bf16_tensor(case.kv_cache, dev),
        block_table=torch.from_numpy(case.block_table).to(dev),
        seqlens=torch.from_numpy(case.seqlens).to(dev),
    )


def bf16_bits(t):
    """torch bf16 tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def sample_pairs(B, H, n, seed):
    """Deterministic (b, h) sample: the four corners plus n random pairs."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (B - 1, H - 1), (0, H - 1), (B - 1, 0)}
    while len(pairs) < min(n + 4, B * H):
        pairs.add((int(rng.integers(B)), int(rng.integers(H))))
    return np.array(sorted(pairs), dtype=np.int32)
