"""Python binding of libmla_latent.so, the MI355X (gfx950) absorbed MLA decode path.

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in ``include/mla_latent.h``.  PyTorch provides device
memory (output tensors allocated here with ``torch.empty``) and the current HIP
stream.  There is no fallback: if the shared library is missing or fails to
load, importing the functions below raises.

Entry points (same names as the C ABI):

* ``mla_absorb_q``      q~ = W_UK^T q_nope                   ("MLA in full detail", Step 2)
* ``mla_decode_latent`` latent attention over the paged cache ("MLA in full detail", Step 3)
* ``mla_decode_latent_fp8``  the same over 656-byte FP8 rows    (M5.8 0x0B)
* ``mla_merge_splits``  log-sum-exp merge of split partials   (M5.8 0x0C)
* ``mla_unabsorb_out``  out = W_UV latent                    ("MLA in full detail", Step 4)
* ``mla_merge_unabsorb``  the merge and the un-absorb in one kernel (no latent round trip)
* ``mla_append_cache``  new tokens' rows into the paged cache (M5.8 0x05)
* ``mla_decode_sparse``  top-k latent attention over physical row ids (M5.8 0x0B)
* ``mla_decode_workspace_size``, ``mla_validate_inputs``, ``mla_status_string``

and, from the separate comparison library ``libmla_normal.so`` (``include/mla_normal.h``,
which links rocBLAS and keeps its handle per device):

* ``mla_decode_normal``  the Normal path on the GPU (per-head K/V), for comparison

``absorbed_decode`` chains the four calls for one decode step.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_latent.so")
NORMAL_LIB_PATH = os.path.join(_HERE, "libmla_normal.so")

MLA_BF16 = 0
MLA_F32 = 1
R_LATENT, D_ROPE, D_NOPE, D_V = 512, 64, 128, 128

_lib = None
_normal_lib = None


class MLAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} (status {status})")


def load_library():
    """Load the in-tree shared library (built by ``mla_latent_kv_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run mla_latent_kv_amd._build.build()")
    # torch first: the library then binds to the HIP runtime torch has loaded
    # (loaded before torch, its HIP calls found no device)
    _torch()
    L = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    SZ = ctypes.c_size_t
    L.mla_status_string.argtypes = [I]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_absorb_q.argtypes = [P, P, P, I, I, I, I, I, P]
    L.mla_decode_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(SZ), ctypes.POINTER(I)]
    L.mla_decode_latent.argtypes = [P, P, P, I, I, P, I, P, I, I, I, I, I, I, F, I,
                                    P, SZ, P, I, P, P, P, I, P, P]
    L.mla_decode_latent_fp8.argtypes = L.mla_decode_latent.argtypes
    L.mla_decode_latent_noalloc.argtypes = [P, P, P, I, I, P, I, P, I, I, I, I, I, I, F, I, P, I, P, P]
    L.mla_merge_splits.argtypes = [P, I, P, P, I, I, I, I, P, I, P, P]
    L.mla_unabsorb_out.argtypes = [P, I, P, P, I, I, I, I, I, P]
    L.mla_merge_unabsorb.argtypes = [P, I, P, P, P, I, I, I, I, I, P, P, P]
    L.mla_append_cache.argtypes = [P, P, P, I, I, P, I, P, I, I, I, I, P]
    L.mla_sparse_split_count.argtypes = [I, I, I, I, I, P]
    L.mla_decode_sparse.argtypes = [P, P, P, I, I, P, I, P, I, I, I, I, I, F, I, P, I, P, P, P, I, P, P]
    L.mla_decode_sparse_fp8.argtypes = L.mla_decode_sparse.argtypes
    L.mla_validate_inputs.argtypes = [P, I, P, I, I, I, I, I, P]
    for name in ("mla_absorb_q", "mla_decode_workspace_size", "mla_decode_latent",
                 "mla_merge_splits", "mla_unabsorb_out", "mla_append_cache", "mla_sparse_split_count",
                 "mla_decode_sparse", "mla_validate_inputs", "mla_decode_latent_fp8",
                 "mla_decode_latent_noalloc", "mla_decode_sparse_fp8", "mla_merge_unabsorb"):
        getattr(L, name).restype = I
    _lib = L
    return L


def load_normal_library():
    """Load the in-tree Normal-path comparison library (rocBLAS GEMMs)."""
    global _normal_lib
    if _normal_lib is not None:
        return _normal_lib
    if not os.path.exists(NORMAL_LIB_PATH):
        raise ImportError(f"{NORMAL_LIB_PATH} is not built; run mla_latent_kv_amd._build.build()")
    _torch()   # (as in load_library)
    L = ctypes.CDLL(NORMAL_LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.mla_normal_workspace_size.argtypes = [I, I, I, I, I, P]
    L.mla_decode_normal.argtypes = [P, P, P, P, P, I, I, P, I, P, I, I, I, I, I, I, I, I, F, I, P,
                                    ctypes.c_size_t, P, P, P]
    L.mla_normal_workspace_size.restype = I
    L.mla_decode_normal.restype = I
    _normal_lib = L
    return L


def status_string(status: int) -> str:
    return load_library().mla_status_string(int(status)).decode()


mla_status_string = status_string


def _torch():
    import torch
    return torch


def _ptr(t):
    """Device address of a tensor the C ABI reads as dense row-major memory."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the MLA library must be device (HIP) tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MLA library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, shape, what):
    """Reject a tensor whose shape disagrees with the sizes passed to the C ABI
    (the kernels index by those sizes)."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _need(t, dtypes, what):
    """Reject a tensor whose element type the C ABI would misread."""
    if t is not None and t.dtype not in dtypes:
        raise ValueError(f"{what}: expected {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(st, what):
    if st != 0:
        raise MLAError(st, what)


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return MLA_BF16
    if dtype == torch.float32:
        return MLA_F32
    raise ValueError(f"unsupported dtype {dtype}")


def mla_absorb_q(q_nope, w_uk, q_lat=None, stream=None):
    """q_nope [B,T,H,128] bf16, w_uk [H,128,512] bf16 -> q_lat [B,T,H,512] bf16."""
    torch = _torch()
    for t, n in ((q_nope, "q_nope"), (w_uk, "w_uk"), (q_lat, "q_lat")):
        _need(t, (torch.bfloat16,), "mla_absorb_q " + n)
    B, T, H, dn = q_nope.shape
    _shape(w_uk, (H, dn, w_uk.shape[2]), "mla_absorb_q w_uk")
    _shape(q_lat, (B, T, H, w_uk.shape[2]), "mla_absorb_q q_lat")
    r = w_uk.shape[2]
    if q_lat is None:
        q_lat = torch.empty((B, T, H, r), dtype=torch.bfloat16, device=q_nope.device)
    _check(load_library().mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(q_lat), B, T, H, dn, r,
                                       _stream(stream)), "mla_absorb_q")
    return q_lat


def mla_decode_workspace_size(B, T, H, max_seqlen, page_size, num_splits, r=R_LATENT):
    """(workspace bytes, max_total_splits) for mla_decode_latent."""
    nb = ctypes.c_size_t(0)
    ms = ctypes.c_int(0)
    _check(load_library().mla_decode_workspace_size(B, T, H, r, max_seqlen, page_size, num_splits,
                                                    ctypes.byref(nb), ctypes.byref(ms)),
           "mla_decode_workspace_size")
    return int(nb.value), int(ms.value)


class DecodeBuffers:
    """Caller-owned scratch of mla_decode_latent in split mode (allocated once, reused)."""

    def __init__(self, B, T, H, max_seqlen, page_size, num_splits, device, part_dtype=None):
        torch = _torch()
        nbytes, max_splits = mla_decode_workspace_size(B, T, H, max_seqlen, page_size, num_splits)
        self.num_splits = num_splits
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.workspace_bytes = nbytes
        self.part_out = torch.empty((max(max_splits, 1), T, H, R_LATENT),
                                    dtype=part_dtype or torch.float32, device=device)
        self.part_lse = torch.empty((max(max_splits, 1), T, H), dtype=torch.float32, device=device)
        self.split_indptr = torch.empty(B + 1, dtype=torch.int32, device=device)


def _check_buffer(t, shape_ok, dtypes, device, what):
    if t is None or not shape_ok(tuple(t.shape)) or t.dtype not in dtypes or t.device != device \
            or not t.is_contiguous():
        raise ValueError(what)


def _check_decode_buffers(buf, B, T, H, max_seqlen, page_size, num_splits, device, what):
    """A caller's DecodeBuffers must be large enough for THIS call: the kernels
    write part_out / part_lse rows and split_indptr entries by the call's own
    geometry (the C ABI sees no buffer sizes), so a buffer built for fewer
    splits, sequences, tokens or heads would be written past its end."""
    torch = _torch()
    nbytes, rows = mla_decode_workspace_size(B, T, H, max_seqlen, page_size, num_splits)
    rows = max(rows, 1)
    _check_buffer(buf.part_out, lambda s: len(s) == 4 and s[0] >= rows and s[1:] == (T, H, R_LATENT),
                  (torch.bfloat16, torch.float32), device,
                  f"{what}: buffers.part_out must be [>= {rows}, {T}, {H}, {R_LATENT}] bf16/f32 on {device}")
    _check_buffer(buf.part_lse, lambda s: len(s) == 3 and s[0] >= rows and s[1:] == (T, H),
                  (torch.float32,), device, f"{what}: buffers.part_lse must be [>= {rows}, {T}, {H}] f32")
    _check_buffer(buf.split_indptr, lambda s: len(s) == 1 and s[0] >= B + 1, (torch.int32,), device,
                  f"{what}: buffers.split_indptr must hold >= {B + 1} int32")
    if nbytes > 0:
        _check_buffer(buf.workspace, lambda s: len(s) == 1 and s[0] >= nbytes, (torch.uint8,), device,
                      f"{what}: buffers.workspace must hold >= {nbytes} bytes")
        if buf.workspace_bytes < nbytes:
            raise ValueError(f"{what}: buffers.workspace_bytes {buf.workspace_bytes} < {nbytes}")


def mla_decode_latent(q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                      num_splits=1, out_dtype=None, buffers: Optional[DecodeBuffers] = None,
                      out_latent=None, lse=None, merge=True, stream=None):
    """Absorbed latent attention (see include/mla_latent.h for the contract).

    Returns (out_latent, lse).  With num_splits != 1 and merge=False the merge
    is skipped, out_latent is None and the partials stay in ``buffers``."""
    return _decode(False, q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                   num_splits, out_dtype, buffers, out_latent, lse, merge, stream)


def mla_decode_latent_fp8(q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                          num_splits=1, out_dtype=None, buffers: Optional[DecodeBuffers] = None,
                          out_latent=None, lse=None, merge=True, stream=None):
    """mla_decode_latent over FP8 rows: ``kv_cache`` is uint8 [num_blocks, P, 656]."""
    torch = _torch()
    if kv_cache.dtype != torch.uint8 or kv_cache.shape[-1] != 656:
        raise ValueError("mla_decode_latent_fp8: kv_cache must be uint8 [num_blocks, page_size, 656]")
    return _decode(True, q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                   num_splits, out_dtype, buffers, out_latent, lse, merge, stream)


def _decode(fp8, q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
            num_splits, out_dtype, buffers, out_latent, lse, merge, stream):
    torch = _torch()
    what = "mla_decode_latent_fp8" if fp8 else "mla_decode_latent"
    _need(q_lat, (torch.bfloat16,), what + " q_lat")
    _need(q_pe, (torch.bfloat16,), what + " q_pe")
    _need(kv_cache, (torch.uint8,) if fp8 else (torch.bfloat16,), what + " kv_cache")
    _need(block_table, (torch.int32,), what + " block_table")
    _need(seqlens, (torch.int32,), what + " seqlens")
    _need(lse, (torch.float32,), what + " lse")
    B, T, H, r = q_lat.shape
    dr = q_pe.shape[3]
    num_blocks, page_size, _ = kv_cache.shape
    max_blocks = block_table.shape[1]
    _shape(q_pe, (B, T, H, dr), what + " q_pe")
    _shape(kv_cache, (num_blocks, page_size, 656 if fp8 else r + dr), what + " kv_cache")
    if block_table.dim() != 2 or block_table.shape[0] < B or seqlens.dim() != 1 or seqlens.shape[0] < B:
        raise ValueError(what + ": block_table [>=B, max_blocks] and seqlens [>=B] expected")
    _shape(out_latent, (B, T, H, r), what + " out_latent")
    _shape(lse, (B, T, H), what + " lse")
    if out_dtype is None:
        out_dtype = out_latent.dtype if out_latent is not None else torch.bfloat16
    elif out_latent is not None and out_latent.dtype != out_dtype:
        raise ValueError("out_latent's dtype differs from out_dtype")
    want_out = num_splits == 1 or merge
    if want_out and out_latent is None:
        out_latent = torch.empty((B, T, H, r), dtype=out_dtype, device=q_lat.device)
    if want_out and lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q_lat.device)
    if num_splits != 1:
        if buffers is None:
            buffers = DecodeBuffers(B, T, H, max_seqlen, page_size, num_splits, q_lat.device)
        else:
            _check_decode_buffers(buffers, B, T, H, int(max_seqlen), page_size, int(num_splits), q_lat.device, what)
    ws = buffers.workspace if num_splits != 1 else None
    lib = load_library()
    st = (lib.mla_decode_latent_fp8 if fp8 else lib.mla_decode_latent)(
        _ptr(q_lat), _ptr(q_pe), _ptr(kv_cache), num_blocks, page_size, _ptr(block_table),
        max_blocks, _ptr(seqlens), B, T, H, r, dr, int(max_seqlen), float(softmax_scale),
        int(num_splits), _ptr(ws), buffers.workspace_bytes if num_splits != 1 else 0,
        _ptr(buffers.part_out if num_splits != 1 else None),
        _dtype_code(buffers.part_out.dtype) if num_splits != 1 else MLA_F32,
        _ptr(buffers.part_lse if num_splits != 1 else None),
        _ptr(buffers.split_indptr if num_splits != 1 else None),
        _ptr(out_latent if want_out else None), _dtype_code(out_dtype),
        _ptr(lse if want_out else None), _stream(stream))
    _check(st, "mla_decode_latent_fp8" if fp8 else "mla_decode_latent")
    return (out_latent, lse) if want_out else (None, None)


def mla_decode_latent_noalloc(q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                              num_splits=0, out_latent=None, lse=None, out_dtype=None, stream=None):
    """mla_decode_latent with its split scratch in the library's own device
    array (the C entry point allocates nothing; see include/mla_latent.h).
    Pass ``out_latent`` and ``lse`` to make the whole call allocation-free;
    otherwise they are allocated here with torch.  Returns (out_latent, lse)."""
    torch = _torch()
    what = "mla_decode_latent_noalloc"
    _need(q_lat, (torch.bfloat16,), what + " q_lat")
    _need(q_pe, (torch.bfloat16,), what + " q_pe")
    _need(kv_cache, (torch.bfloat16,), what + " kv_cache")
    _need(block_table, (torch.int32,), what + " block_table")
    _need(seqlens, (torch.int32,), what + " seqlens")
    _need(lse, (torch.float32,), what + " lse")
    B, T, H, r = q_lat.shape
    dr = q_pe.shape[3]
    num_blocks, page_size, _ = kv_cache.shape
    _shape(q_pe, (B, T, H, dr), what + " q_pe")
    _shape(kv_cache, (num_blocks, page_size, r + dr), what + " kv_cache")
    if block_table.dim() != 2 or block_table.shape[0] < B or seqlens.dim() != 1 or seqlens.shape[0] < B:
        raise ValueError(what + ": block_table [>=B, max_blocks] and seqlens [>=B] expected")
    _shape(out_latent, (B, T, H, r), what + " out_latent")
    _shape(lse, (B, T, H), what + " lse")
    if out_dtype is None:
        out_dtype = out_latent.dtype if out_latent is not None else torch.bfloat16
    elif out_latent is not None and out_latent.dtype != out_dtype:
        raise ValueError("out_latent's dtype differs from out_dtype")
    if out_latent is None:
        out_latent = torch.empty((B, T, H, r), dtype=out_dtype, device=q_lat.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q_lat.device)
    _check(load_library().mla_decode_latent_noalloc(
        _ptr(q_lat), _ptr(q_pe), _ptr(kv_cache), num_blocks, page_size, _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), B, T, H, r, dr, int(max_seqlen), float(softmax_scale), int(num_splits), _ptr(out_latent),
        _dtype_code(out_dtype), _ptr(lse), _stream(stream)), what)
    return out_latent, lse


def mla_merge_splits(part_out, part_lse, split_indptr, B, out_latent=None, lse=None,
                     out_dtype=None, stream=None):
    """Merge partials -> (out_latent [B,T,H,512], lse [B,T,H])."""
    torch = _torch()
    _need(part_lse, (torch.float32,), "mla_merge_splits part_lse")
    _need(split_indptr, (torch.int32,), "mla_merge_splits split_indptr")
    _need(lse, (torch.float32,), "mla_merge_splits lse")
    _, T, H, r = part_out.shape
    _shape(part_lse, (part_out.shape[0], T, H), "mla_merge_splits part_lse")
    _shape(split_indptr, (B + 1,), "mla_merge_splits split_indptr")
    _shape(out_latent, (B, T, H, r), "mla_merge_splits out_latent")
    _shape(lse, (B, T, H), "mla_merge_splits lse")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_latent is None:
        out_latent = torch.empty((B, T, H, r), dtype=out_dtype, device=part_out.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=part_out.device)
    _check(load_library().mla_merge_splits(_ptr(part_out), _dtype_code(part_out.dtype),
                                           _ptr(part_lse), _ptr(split_indptr), B, T, H, r,
                                           _ptr(out_latent), _dtype_code(out_latent.dtype),
                                           _ptr(lse), _stream(stream)), "mla_merge_splits")
    return out_latent, lse


def mla_unabsorb_out(latent, w_uv, out=None, stream=None):
    """latent [B,T,H,512] bf16/f32, w_uv [H,128,512] bf16 -> out [B,T,H,128] f32."""
    torch = _torch()
    _need(latent, (torch.bfloat16, torch.float32), "mla_unabsorb_out latent")
    _need(w_uv, (torch.bfloat16,), "mla_unabsorb_out w_uv")
    _need(out, (torch.float32,), "mla_unabsorb_out out")
    B, T, H, r = latent.shape
    dv = w_uv.shape[1]
    _shape(w_uv, (H, dv, r), "mla_unabsorb_out w_uv")
    _shape(out, (B, T, H, dv), "mla_unabsorb_out out")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=latent.device)
    _check(load_library().mla_unabsorb_out(_ptr(latent), _dtype_code(latent.dtype), _ptr(w_uv),
                                           _ptr(out), B, T, H, r, dv, _stream(stream)),
           "mla_unabsorb_out")
    return out


def mla_merge_unabsorb(part_out, part_lse, split_indptr, w_uv, B, out=None, lse=None, stream=None):
    """Merge of split partials and un-absorb in one kernel:
    part_out [*,T,H,512] f32/bf16, part_lse [*,T,H] f32, split_indptr [B+1] int32,
    w_uv [H,128,512] bf16 -> (out [B,T,H,128] f32, lse [B,T,H] f32)."""
    torch = _torch()
    _need(part_out, (torch.bfloat16, torch.float32), "mla_merge_unabsorb part_out")
    _need(part_lse, (torch.float32,), "mla_merge_unabsorb part_lse")
    _need(split_indptr, (torch.int32,), "mla_merge_unabsorb split_indptr")
    _need(w_uv, (torch.bfloat16,), "mla_merge_unabsorb w_uv")
    _need(out, (torch.float32,), "mla_merge_unabsorb out")
    _need(lse, (torch.float32,), "mla_merge_unabsorb lse")
    _, T, H, r = part_out.shape
    dv = w_uv.shape[1]
    _shape(part_lse, (part_out.shape[0], T, H), "mla_merge_unabsorb part_lse")
    _shape(split_indptr, (B + 1,), "mla_merge_unabsorb split_indptr")
    _shape(w_uv, (H, dv, r), "mla_merge_unabsorb w_uv")
    _shape(out, (B, T, H, dv), "mla_merge_unabsorb out")
    _shape(lse, (B, T, H), "mla_merge_unabsorb lse")
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=part_out.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=part_out.device)
    _check(load_library().mla_merge_unabsorb(_ptr(part_out), _dtype_code(part_out.dtype), _ptr(part_lse),
                                             _ptr(split_indptr), _ptr(w_uv), B, T, H, r, dv, _ptr(out),
                                             _ptr(lse), _stream(stream)), "mla_merge_unabsorb")
    return out, lse


def mla_append_cache(c_new, kpe_new, kv_cache, block_table, seqlens, stream=None):
    """Write the T new rows of every sequence at positions seqlens[b]-T+t of the
    paged cache (in place).  c_new [B,T,512] bf16, kpe_new [B,T,64] bf16."""
    torch = _torch()
    for t, n in ((c_new, "c_new"), (kpe_new, "kpe_new"), (kv_cache, "kv_cache")):
        _need(t, (torch.bfloat16,), "mla_append_cache " + n)
    _need(block_table, (torch.int32,), "mla_append_cache block_table")
    _need(seqlens, (torch.int32,), "mla_append_cache seqlens")
    B, T, r = c_new.shape
    dr = kpe_new.shape[2]
    num_blocks, page_size, _ = kv_cache.shape
    if tuple(kpe_new.shape[:2]) != (B, T) or seqlens.shape[0] < B or block_table.shape[0] < B:
        raise ValueError("mla_append_cache: c_new, kpe_new, seqlens and block_table disagree on B, T")
    _shape(kv_cache, (num_blocks, page_size, r + dr), "mla_append_cache kv_cache")
    _check(load_library().mla_append_cache(_ptr(c_new), _ptr(kpe_new), _ptr(kv_cache), num_blocks, page_size,
                                           _ptr(block_table), block_table.shape[1], _ptr(seqlens), B, T, r,
                                           dr, _stream(stream)), "mla_append_cache")
    return kv_cache


def mla_sparse_split_count(B, T, H, topk, num_splits=0) -> int:
    """Split count mla_decode_sparse uses (0 = automatic)."""
    sc = ctypes.c_int(0)
    _check(load_library().mla_sparse_split_count(B, T, H, topk, num_splits, ctypes.byref(sc)),
           "mla_sparse_split_count")
    return int(sc.value)


class SparseBuffers:
    """Caller-owned split partials of mla_decode_sparse (B*T*S rows)."""

    def __init__(self, B, T, H, topk, num_splits, device, part_dtype=None):
        torch = _torch()
        self.num_splits = mla_sparse_split_count(B, T, H, topk, num_splits)
        self.part_out = self.part_lse = self.split_indptr = None
        if self.num_splits > 1:
            n = max(B * T * self.num_splits, 1)
            self.part_out = torch.empty((n, H, R_LATENT), dtype=part_dtype or torch.float32, device=device)
            self.part_lse = torch.empty((n, H), dtype=torch.float32, device=device)
            self.split_indptr = torch.empty(B * T + 1, dtype=torch.int32, device=device)


def mla_decode_sparse(q_lat, q_pe, kv_cache, indices, topk_length, softmax_scale, num_splits=0,
                      out_dtype=None, buffers: Optional[SparseBuffers] = None, out_latent=None, lse=None,
                      merge=True, stream=None):
    """Sparse (top-k) latent attention (see include/mla_latent.h).

    indices [B,T,topk] int32 physical rows, topk_length [B] int32 or None.
    Returns (out_latent, lse); with more than one split and merge=False the
    partials stay in ``buffers`` and (None, None) is returned."""
    return _sparse(False, q_lat, q_pe, kv_cache, indices, topk_length, softmax_scale, num_splits, out_dtype,
                   buffers, out_latent, lse, merge, stream)


def mla_decode_sparse_fp8(q_lat, q_pe, kv_cache, indices, topk_length, softmax_scale, num_splits=0,
                          out_dtype=None, buffers: Optional[SparseBuffers] = None, out_latent=None, lse=None,
                          merge=True, stream=None):
    """mla_decode_sparse over FP8 rows: ``kv_cache`` is uint8 [num_blocks, P, 656]."""
    return _sparse(True, q_lat, q_pe, kv_cache, indices, topk_length, softmax_scale, num_splits, out_dtype,
                   buffers, out_latent, lse, merge, stream)


def _sparse(fp8, q_lat, q_pe, kv_cache, indices, topk_length, softmax_scale, num_splits, out_dtype, buffers,
            out_latent, lse, merge, stream):
    torch = _torch()
    _need(q_lat, (torch.bfloat16,), "mla_decode_sparse q_lat")
    _need(q_pe, (torch.bfloat16,), "mla_decode_sparse q_pe")
    _need(kv_cache, (torch.uint8,) if fp8 else (torch.bfloat16,), "mla_decode_sparse kv_cache")
    _need(indices, (torch.int32,), "mla_decode_sparse indices")
    _need(topk_length, (torch.int32,), "mla_decode_sparse topk_length")
    B, T, H, r = q_lat.shape
    dr = q_pe.shape[3]
    num_blocks, page_size, _ = kv_cache.shape
    topk = indices.shape[2]
    if tuple(indices.shape[:2]) != (B, T) or (topk_length is not None and topk_length.shape[0] < B):
        raise ValueError("mla_decode_sparse: indices / topk_length do not match q_lat")
    _shape(q_pe, (B, T, H, dr), "mla_decode_sparse q_pe")
    _shape(kv_cache, (num_blocks, page_size, 656 if fp8 else r + dr), "mla_decode_sparse kv_cache")
    _shape(out_latent, (B, T, H, r), "mla_decode_sparse out_latent")
    _shape(lse, (B, T, H), "mla_decode_sparse lse")
    if out_dtype is None:
        out_dtype = out_latent.dtype if out_latent is not None else torch.bfloat16
    elif out_latent is not None and out_latent.dtype != out_dtype:
        raise ValueError("out_latent's dtype differs from out_dtype")
    if buffers is None:
        buffers = SparseBuffers(B, T, H, topk, num_splits, q_lat.device)
    S = buffers.num_splits
    if S != mla_sparse_split_count(B, T, H, topk, num_splits):
        raise ValueError(f"mla_decode_sparse: buffers hold {S} splits, the call asks for "
                         f"{mla_sparse_split_count(B, T, H, topk, num_splits)}")
    if S > 1:
        rows = B * T * S
        _check_buffer(buffers.part_out, lambda s: len(s) == 3 and s[0] >= rows and s[1:] == (H, R_LATENT),
                      (torch.bfloat16, torch.float32), q_lat.device,
                      f"mla_decode_sparse: buffers.part_out must be [>= {rows}, {H}, {R_LATENT}] bf16/f32")
        _check_buffer(buffers.part_lse, lambda s: len(s) == 2 and s[0] >= rows and s[1] == H, (torch.float32,),
                      q_lat.device, f"mla_decode_sparse: buffers.part_lse must be [>= {rows}, {H}] f32")
        _check_buffer(buffers.split_indptr, lambda s: len(s) == 1 and s[0] >= B * T + 1, (torch.int32,),
                      q_lat.device, f"mla_decode_sparse: buffers.split_indptr must hold >= {B * T + 1} int32")
    want_out = S == 1 or merge
    if want_out and out_latent is None:
        out_latent = torch.empty((B, T, H, r), dtype=out_dtype, device=q_lat.device)
    if want_out and lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q_lat.device)
    split = S != 1
    lib = load_library()
    _check((lib.mla_decode_sparse_fp8 if fp8 else lib.mla_decode_sparse)(
        _ptr(q_lat), _ptr(q_pe), _ptr(kv_cache), num_blocks, page_size, _ptr(indices), topk,
        _ptr(topk_length), B, T, H, r, dr, float(softmax_scale), S,
        _ptr(buffers.part_out if split else None),
        _dtype_code(buffers.part_out.dtype) if split else MLA_F32,
        _ptr(buffers.part_lse if split else None), _ptr(buffers.split_indptr if split else None),
        _ptr(out_latent if want_out else None), _dtype_code(out_dtype),
        _ptr(lse if want_out else None), _stream(stream)), "mla_decode_sparse_fp8" if fp8 else "mla_decode_sparse")
    return (out_latent, lse) if want_out else (None, None)


def mla_normal_workspace_size(B, T, H, max_seqlen, chunk) -> int:
    nb = ctypes.c_size_t(0)
    _check(load_normal_library().mla_normal_workspace_size(B, T, H, max_seqlen, chunk, ctypes.byref(nb)),
           "mla_normal_workspace_size")
    return int(nb.value)


def mla_decode_normal(q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seqlens, max_seqlen, softmax_scale,
                      chunk=None, workspace=None, out=None, lse=None, stream=None):
    """Normal-path decode on the GPU (up-projected per-head K/V, chunked).

    Returns (out [B,T,H,128] f32, lse [B,T,H] f32).  ``chunk`` defaults to
    max_seqlen (one chunk)."""
    torch = _torch()
    for t, n in ((q_nope, "q_nope"), (q_pe, "q_pe"), (w_uk, "w_uk"), (w_uv, "w_uv"), (kv_cache, "kv_cache")):
        _need(t, (torch.bfloat16,), "mla_decode_normal " + n)
    _need(block_table, (torch.int32,), "mla_decode_normal block_table")
    _need(seqlens, (torch.int32,), "mla_decode_normal seqlens")
    B, T, H, dn = q_nope.shape
    dr = q_pe.shape[3]
    dv, r = w_uv.shape[1], w_uk.shape[2]
    num_blocks, page_size, _ = kv_cache.shape
    _shape(q_pe, (B, T, H, dr), "mla_decode_normal q_pe")
    _shape(w_uk, (H, dn, r), "mla_decode_normal w_uk")
    _shape(w_uv, (H, dv, r), "mla_decode_normal w_uv")
    _shape(kv_cache, (num_blocks, page_size, r + dr), "mla_decode_normal kv_cache")
    if block_table.shape[0] < B or seqlens.shape[0] < B:
        raise ValueError("mla_decode_normal: block_table and seqlens need a row per sequence")
    chunk = int(max_seqlen) if chunk is None else int(chunk)
    need = mla_normal_workspace_size(B, T, H, int(max_seqlen), chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q_nope.device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q_nope.device)
    _check(load_normal_library().mla_decode_normal(
        _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv), _ptr(kv_cache), num_blocks, page_size,
        _ptr(block_table), block_table.shape[1], _ptr(seqlens), B, T, H, dn, dr, dv, r, int(max_seqlen),
        float(softmax_scale), chunk, _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
        _stream(stream)), "mla_decode_normal")
    return out, lse


def mla_validate_inputs(block_table, seqlens, T, max_seqlen, page_size, num_blocks, stream=None):
    """Synchronous index check; returns the status code (0 = valid)."""
    B = seqlens.shape[0]
    return int(load_library().mla_validate_inputs(_ptr(block_table), block_table.shape[1],
                                                  _ptr(seqlens), B, T, int(max_seqlen), page_size,
                                                  num_blocks, _stream(stream)))


def softmax_scale(d_nope=D_NOPE, d_rope=D_ROPE) -> float:
    """1/sqrt(d_nope + d_rope): the original 192-wide key's scale ("MLA in full detail")."""
    return 1.0 / math.sqrt(d_nope + d_rope)


def absorbed_decode(q_nope, q_pe, w_uk, w_uv, kv_cache, block_table, seqlens, max_seqlen,
                    num_splits=1, buffers=None, latent_dtype=None, stream=None):
    """One decode step: absorb -> latent attention (-> merge) -> un-absorb.
    With 2 to 4 uniform splits and a bf16 latent the partials are bf16 and the
    merge and un-absorb run as one kernel (mla_merge_unabsorb), the faster form
    for that case; otherwise as mla_merge_splits (inside the decode call) and
    mla_unabsorb_out.

    Returns (out [B,T,H,128] f32, lse [B,T,H] f32)."""
    torch = _torch()
    q_lat = mla_absorb_q(q_nope, w_uk, stream=stream)
    if 2 <= num_splits <= 4 and latent_dtype in (None, torch.bfloat16):
        B, T, H = q_nope.shape[:3]
        if buffers is None:
            buffers = DecodeBuffers(B, T, H, max_seqlen, kv_cache.shape[1], num_splits, q_nope.device,
                                    part_dtype=torch.bfloat16)
        mla_decode_latent(q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen, softmax_scale(),
                          num_splits=num_splits, buffers=buffers, merge=False, stream=stream)
        return mla_merge_unabsorb(buffers.part_out, buffers.part_lse, buffers.split_indptr, w_uv, B,
                                  stream=stream)
    lat, lse = mla_decode_latent(q_lat, q_pe, kv_cache, block_table, seqlens, max_seqlen,
                                 softmax_scale(), num_splits=num_splits,
                                 out_dtype=latent_dtype or torch.bfloat16, buffers=buffers,
                                 stream=stream)
    out = mla_unabsorb_out(lat, w_uv, stream=stream)
    return out, lse


__all__ = [
    "MLA_BF16", "MLA_F32", "MLAError", "load_library", "load_normal_library", "status_string", "mla_status_string",
    "mla_absorb_q", "mla_decode_workspace_size", "mla_decode_latent", "mla_decode_latent_fp8",
    "mla_decode_latent_noalloc", "mla_merge_splits",
    "mla_unabsorb_out", "mla_merge_unabsorb", "mla_append_cache", "mla_sparse_split_count", "mla_decode_sparse",
    "mla_decode_sparse_fp8",
    "SparseBuffers",
    "mla_normal_workspace_size", "mla_decode_normal", "mla_validate_inputs", "DecodeBuffers", "softmax_scale",
    "absorbed_decode",
]
