"""C-ABI checks that need no GPU: the libraries load, export every entry point
their headers declare (include/mla_latent.h -> libmla_latent.so,
include/mla_normal.h -> libmla_normal.so), the decode library is free of
rocBLAS and of mutable state, and every entry point rejects bad host-side
arguments before any launch (the pointers passed here are never
dereferenced)."""
import ctypes
import functools
import os
import re

import pytest

import mla_latent_kv_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_latent.h")
NORMAL_HEADER = os.path.join(ROOT, "include", "mla_normal.h")

OK, NULL, ALIGN, SHAPE, UNSUP, WS = 0, -1, -2, -3, -4, -5


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not (os.path.exists(mk.LIB_PATH) and os.path.exists(mk.NORMAL_LIB_PATH)):
        from mla_latent_kv_amd import _build
        _build.build()
    return mk.load_library()


@pytest.fixture(scope="module")
def nlib(lib):
    return mk.load_normal_library()


def test_every_declared_symbol_is_exported(lib, nlib):
    names = declared_functions()
    assert {"mla_absorb_q", "mla_decode_latent", "mla_merge_splits", "mla_unabsorb_out"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    normal = set(declared_functions(NORMAL_HEADER)) - set(names)
    assert normal == {"mla_decode_normal", "mla_normal_workspace_size"}
    for n in normal:
        assert hasattr(nlib, n), n
        assert not hasattr(lib, n), f"{n} belongs to libmla_normal.so only"


def _elf(cmd, path):
    import shutil
    import subprocess
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    return subprocess.run([*cmd, path], check=True, capture_output=True, text=True).stdout


def test_decode_library_links_no_rocblas(lib):
    """libmla_latent.so depends on the HIP runtime only: no BLAS library (whose
    handles and workspaces allocate) behind any of its entry points."""
    needed = re.findall(r"NEEDED.*\[(.*)\]", _elf(["readelf", "-d"], mk.LIB_PATH))
    assert needed and not [n for n in needed if "blas" in n.lower()], needed
    assert any("rocblas" in n for n in re.findall(r"NEEDED.*\[(.*)\]", _elf(["readelf", "-d"], mk.NORMAL_LIB_PATH)))


def test_decode_library_keeps_no_state(lib):
    """No writable data of the library's own: the only writable symbols are the
    toolchain's (ELF bookkeeping, the HIP fat-binary registration handles), the
    host-side handles of the kernels, and the no-allocation entry point's
    device array (its host-side stand-in), per-device address table and their
    mutex.  A rocBLAS handle table, another mutex or a cached plan would show
    up here."""
    syms = _elf(["nm", "-C", "--defined-only"], mk.LIB_PATH).splitlines()
    own = []
    for line in syms:
        parts = line.split(maxsplit=2)
        if len(parts) < 3 or parts[1] not in "BbDdSs":
            continue
        name = parts[2]
        if name.startswith(("__", "_DYNAMIC", "_GLOBAL_OFFSET_TABLE_", "DW.ref.")):
            continue
        if re.fullmatch(r"mla::\w+_kernel(<.*>)?\(.*\)", name):   # kernel launch handles
            continue
        if name in NOALLOC_STATE:
            continue
        own.append(name)
    assert not own, own


NOALLOC_STATE = {"(anonymous namespace)::noalloc_scratch", "(anonymous namespace)::g_noalloc_ptr",
                 "(anonymous namespace)::g_noalloc_mu"}


def _file_scope_variables(src):
    """Declarations at namespace scope that are neither functions nor
    constants (a crude C++ scan: comments stripped, braces counted)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"^\s*#.*$", "", src, flags=re.M)
    depth, top, line = 0, [], ""
    scopes = []   # True for a namespace / extern "C" brace
    for ch in src:
        if ch == "{":
            head = " ".join(line.split())
            is_ns = head.startswith(("namespace", 'extern "C"')) and "(" not in head
            if all(scopes) and not is_ns:
                top.append(head)
            scopes.append(is_ns)
            line = ""
        elif ch == "}":
            scopes.pop()
            line = ""
        elif ch == ";":
            if all(scopes):
                top.append(" ".join(line.split()))
            line = ""
        else:
            line += ch
    out = []
    for d in top:
        if not d or "(" in d or d.startswith(("constexpr", "using", "typedef", "struct", "class", "enum",
                                               "template", "static_assert", "return")):
            continue
        if re.match(r"^(static\s+)?(const\s+)?[\w:<>,\*&\s]+\s+[\w\[\]\d]+\s*(=.*)?$", d) and \
                not re.match(r"^(static\s+)?const\s", d):
            out.append(d)
    return out


def test_file_scope_scan_flags_mutable_globals():
    """The scan below catches the kinds of state this library must not hold."""
    bad = """namespace { std::mutex g_mu; rocblas_handle g_blas[64] = {}; int counter = 0;
             constexpr int kX = 4; int f(int a) { int local = a; return local; } }
             extern "C" { int mla_x(void) { static int calls; return calls; } }"""
    assert _file_scope_variables(bad) == ["std::mutex g_mu", "rocblas_handle g_blas[64] =", "int counter = 0"]


def test_api_source_has_no_file_scope_state():
    """The ABI source itself (api.cpp: validation, sizing, launches) declares no
    file-scope variable other than constants."""
    src = open(os.path.join(ROOT, "mla_latent_kv_amd", "csrc", "api.cpp")).read()
    assert _file_scope_variables(src) == []


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = mk.status_string(code)
        assert s and s != "unknown status"
    assert mk.status_string(12345) == "unknown status"


P16 = ctypes.c_void_p(1 << 20)      # 16-byte aligned fake device address
P17 = ctypes.c_void_p((1 << 20) + 2)  # misaligned


def test_absorb_validation(lib):
    f = lib.mla_absorb_q
    assert f(P16, P16, P16, 2, 1, 128, 64, 512, None) == UNSUP     # d_nope != 128
    assert f(P16, P16, P16, 2, 1, 128, 128, 256, None) == UNSUP    # r != 512
    assert f(P16, P16, P16, 2, 1025, 128, 128, 512, None) == UNSUP  # T > 1024
    assert f(P16, P16, P16, 2, 1, 129, 128, 512, None) == UNSUP    # H > 128
    assert f(P16, P16, P16, 2, 0, 128, 128, 512, None) == SHAPE    # T < 1
    assert f(P16, P16, P16, -1, 1, 128, 128, 512, None) == SHAPE
    assert f(None, P16, P16, 2, 1, 128, 128, 512, None) == NULL
    assert f(P16, P17, P16, 2, 1, 128, 128, 512, None) == ALIGN
    assert f(None, None, None, 0, 1, 128, 128, 512, None) == OK    # empty batch: no-op


def test_unabsorb_validation(lib):
    f = lib.mla_unabsorb_out
    assert f(P16, 0, P16, P16, 2, 1, 128, 512, 64, None) == UNSUP
    assert f(P16, 7, P16, P16, 2, 1, 128, 512, 128, None) == UNSUP  # bad dtype
    assert f(P16, 0, None, P16, 2, 1, 128, 512, 128, None) == NULL
    assert f(P16, 1, P16, P17, 2, 1, 128, 512, 128, None) == ALIGN
    assert f(None, 0, None, None, 0, 1, 128, 512, 128, None) == OK


def _decode_any(lib, fp8=False, **kw):
    a = dict(q_lat=P16, q_pe=P16, kv=P16, nb=64, P=64, bt=P16, mb=64, sl=P16, B=2, T=1, H=128,
             r=512, dr=64, maxL=4096, scale=0.07, S=1, ws=None, wsb=0, po=None, pdt=1, pl=None,
             si=None, out=P16, odt=0, lse=None)
    a.update(kw)
    f = lib.mla_decode_latent_fp8 if fp8 else lib.mla_decode_latent
    return f(a["q_lat"], a["q_pe"], a["kv"], a["nb"], a["P"], a["bt"], a["mb"],
             a["sl"], a["B"], a["T"], a["H"], a["r"], a["dr"], a["maxL"],
             ctypes.c_float(a["scale"]), a["S"], a["ws"], a["wsb"], a["po"],
             a["pdt"], a["pl"], a["si"], a["out"], a["odt"], a["lse"], None)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_validation(lib, fp8):
    _decode = functools.partial(_decode_any, fp8=fp8)
    assert _decode(lib, r=256) == UNSUP
    assert _decode(lib, dr=32) == UNSUP
    assert _decode(lib, P=24) == UNSUP          # not a multiple of 16
    assert _decode(lib, P=2048) == UNSUP
    assert _decode(lib, T=1025) == UNSUP
    assert _decode(lib, odt=5) == UNSUP
    assert _decode(lib, pdt=3) == UNSUP
    assert _decode(lib, scale=0.0) == SHAPE
    assert _decode(lib, scale=float("nan")) == SHAPE
    assert _decode(lib, maxL=0, T=1) == SHAPE    # max_seqlen < T
    assert _decode(lib, mb=63) == SHAPE          # 4096 tokens need 64 pages of 64
    assert _decode(lib, nb=0) == SHAPE
    assert _decode(lib, S=-1) == SHAPE
    assert _decode(lib, q_lat=None) == NULL
    assert _decode(lib, kv=P17) == ALIGN
    assert _decode(lib, out=None) == NULL        # unsplit needs out_latent
    assert _decode(lib, S=4) == WS               # split without partial buffers
    need = ctypes.c_size_t(0)
    ms = ctypes.c_int(0)
    assert lib.mla_decode_workspace_size(2, 1, 128, 512, 4096, 64, 4, ctypes.byref(need),
                                         ctypes.byref(ms)) == OK
    assert ms.value == 8 and need.value == 0       # uniform splits keep no work list
    assert _decode(lib, S=4, po=P16, pl=P16, si=None) == WS
    assert _decode(lib, S=4, po=P17, pl=P16, si=P16) == ALIGN
    assert _decode(lib, S=4, po=P17, pdt=0, pl=P16, si=P16) == ALIGN
    assert _decode(lib, B=0, q_lat=None, out=None) == OK


def test_workspace_size(lib):
    need = ctypes.c_size_t(123)
    ms = ctypes.c_int(7)
    assert lib.mla_decode_workspace_size(64, 1, 128, 512, 4096, 64, 1, ctypes.byref(need),
                                         ctypes.byref(ms)) == OK
    assert need.value == 0 and ms.value == 0
    assert lib.mla_decode_workspace_size(4, 1, 128, 512, 131072, 64, 64, ctypes.byref(need),
                                         ctypes.byref(ms)) == OK
    assert ms.value == 256
    assert lib.mla_decode_workspace_size(4, 1, 128, 512, 131072, 64, 64, None, ctypes.byref(ms)) == NULL
    assert lib.mla_decode_workspace_size(4, 1, 128, 256, 131072, 64, 64, ctypes.byref(need),
                                         ctypes.byref(ms)) == UNSUP


def test_merge_validation(lib):
    f = lib.mla_merge_splits
    assert f(P16, 1, P16, P16, 2, 1, 128, 256, P16, 0, None, None) == UNSUP
    assert f(None, 1, P16, P16, 2, 1, 128, 512, P16, 0, None, None) == NULL
    assert f(P16, 1, P16, P16, 2, 1, 128, 512, P17, 0, None, None) == ALIGN
    assert f(P16, 1, P16, P16, 2, 1, 128, 512, P16, 9, None, None) == UNSUP
    assert f(P16, 2, P16, P16, 2, 1, 128, 512, P16, 0, None, None) == UNSUP   # bad partial dtype
    assert f(None, 0, None, None, 0, 1, 128, 512, None, 0, None, None) == OK


def test_merge_unabsorb_validation(lib):
    f = lib.mla_merge_unabsorb
    assert f(P16, 0, P16, P16, P16, 2, 1, 128, 256, 128, P16, None, None) == UNSUP   # r
    assert f(P16, 0, P16, P16, P16, 2, 1, 128, 512, 64, P16, None, None) == UNSUP    # d_V
    assert f(P16, 2, P16, P16, P16, 2, 1, 128, 512, 128, P16, None, None) == UNSUP   # partial dtype
    assert f(P16, 0, P16, P16, P16, 2, 1, 129, 512, 128, P16, None, None) == UNSUP   # H
    assert f(None, 0, P16, P16, P16, 2, 1, 128, 512, 128, P16, None, None) == NULL
    assert f(P16, 0, P16, P16, P17, 2, 1, 128, 512, 128, P16, None, None) == ALIGN   # w_uv
    assert f(P16, 0, P16, P16, P16, 2, 1, 128, 512, 128, P17, None, None) == ALIGN   # out
    assert f(None, 0, None, None, None, 0, 1, 128, 512, 128, None, None, None) == OK  # B = 0: no-op


def test_binding_names_match_abi():
    for n in ("mla_absorb_q", "mla_decode_latent", "mla_decode_latent_fp8", "mla_merge_splits",
              "mla_unabsorb_out", "mla_merge_unabsorb", "mla_append_cache",
              "mla_decode_sparse", "mla_sparse_split_count", "mla_decode_normal", "mla_normal_workspace_size",
              "load_normal_library",
              "mla_decode_workspace_size", "mla_validate_inputs", "mla_status_string"):
        assert callable(getattr(mk, n))


def _append(lib, **kw):
    a = dict(c=P16, k=P16, kv=P16, nb=64, P=64, bt=P16, mb=64, sl=P16, B=2, T=1, r=512, dr=64)
    a.update(kw)
    return lib.mla_append_cache(a["c"], a["k"], a["kv"], a["nb"], a["P"], a["bt"], a["mb"], a["sl"],
                                a["B"], a["T"], a["r"], a["dr"], None)


def test_append_validation(lib):
    assert _append(lib, r=256) == UNSUP
    assert _append(lib, dr=32) == UNSUP
    assert _append(lib, P=24) == UNSUP
    assert _append(lib, P=2048) == UNSUP
    assert _append(lib, T=1025) == UNSUP
    assert _append(lib, T=0) == SHAPE
    assert _append(lib, B=-1) == SHAPE
    assert _append(lib, nb=0) == SHAPE
    assert _append(lib, mb=0) == SHAPE
    assert _append(lib, c=None) == NULL
    assert _append(lib, kv=P17) == ALIGN
    assert _append(lib, bt=ctypes.c_void_p((1 << 20) + 2)) == ALIGN
    assert _append(lib, B=1 << 22, T=8) == UNSUP     # more rows than one launch covers
    assert _append(lib, B=0, c=None, k=None, kv=None, bt=None, sl=None) == OK


def _sparse(lib, **kw):
    a = dict(q=P16, qp=P16, kv=P16, nb=64, P=64, idx=P16, topk=2048, tl=None, B=2, T=1, H=128, r=512,
             dr=64, scale=0.07, S=1, po=None, pdt=1, pl=None, si=None, out=P16, odt=0, lse=None)
    a.update(kw)
    return lib.mla_decode_sparse(a["q"], a["qp"], a["kv"], a["nb"], a["P"], a["idx"], a["topk"], a["tl"],
                                 a["B"], a["T"], a["H"], a["r"], a["dr"], ctypes.c_float(a["scale"]),
                                 a["S"], a["po"], a["pdt"], a["pl"], a["si"], a["out"], a["odt"], a["lse"],
                                 None)


def test_sparse_validation(lib):
    assert _sparse(lib, r=256) == UNSUP
    assert _sparse(lib, dr=32) == UNSUP
    assert _sparse(lib, T=1025) == UNSUP
    assert _sparse(lib, H=129) == UNSUP
    assert _sparse(lib, P=24) == UNSUP
    assert _sparse(lib, odt=4) == UNSUP
    assert _sparse(lib, topk=0) == SHAPE
    assert _sparse(lib, nb=0) == SHAPE
    assert _sparse(lib, S=-1) == SHAPE
    assert _sparse(lib, scale=-1.0) == SHAPE
    assert _sparse(lib, nb=1 << 23, P=1024) == UNSUP      # more than 2^32 - 1 rows
    assert _sparse(lib, q=None) == NULL
    assert _sparse(lib, idx=None) == NULL
    assert _sparse(lib, idx=ctypes.c_void_p((1 << 20) + 2)) == ALIGN
    assert _sparse(lib, tl=ctypes.c_void_p((1 << 20) + 2)) == ALIGN
    assert _sparse(lib, out=None) == NULL                  # one split needs out_latent
    assert _sparse(lib, S=4) == WS                         # split without partial buffers
    assert _sparse(lib, S=4, po=P17, pl=P16, si=P16) == ALIGN
    assert _sparse(lib, B=0, q=None, out=None, idx=None) == OK


def test_sparse_split_count(lib):
    sc = ctypes.c_int(0)
    assert lib.mla_sparse_split_count(64, 1, 128, 2048, 4, ctypes.byref(sc)) == OK and sc.value == 4
    assert lib.mla_sparse_split_count(0, 1, 128, 2048, 0, ctypes.byref(sc)) == OK and sc.value == 1
    assert lib.mla_sparse_split_count(64, 1, 128, 0, 0, ctypes.byref(sc)) == SHAPE
    assert lib.mla_sparse_split_count(64, 1, 128, 16, 0, None) == NULL


def _normal(lib, **kw):
    a = dict(qn=P16, qp=P16, wk=P16, wv=P16, kv=P16, nb=64, P=64, bt=P16, mb=64, sl=P16, B=2, T=1, H=128,
             dn=128, dr=64, dv=128, r=512, maxL=4096, scale=0.07, chunk=1024, ws=P16, wsb=1 << 40, out=P16,
             lse=None)
    a.update(kw)
    return lib.mla_decode_normal(a["qn"], a["qp"], a["wk"], a["wv"], a["kv"], a["nb"], a["P"], a["bt"], a["mb"],
                                 a["sl"], a["B"], a["T"], a["H"], a["dn"], a["dr"], a["dv"], a["r"], a["maxL"],
                                 ctypes.c_float(a["scale"]), a["chunk"], a["ws"], ctypes.c_size_t(a["wsb"]),
                                 a["out"], a["lse"], None)


def test_normal_validation(nlib):
    lib = nlib
    assert _normal(lib, dn=64) == UNSUP
    assert _normal(lib, r=256) == UNSUP
    assert _normal(lib, T=1025) == UNSUP
    assert _normal(lib, P=24) == UNSUP
    assert _normal(lib, chunk=0) == SHAPE
    assert _normal(lib, maxL=0) == SHAPE
    assert _normal(lib, mb=63) == SHAPE
    assert _normal(lib, scale=0.0) == SHAPE
    assert _normal(lib, ws=None) == WS
    assert _normal(lib, wsb=1000) == WS
    assert _normal(lib, qn=P17) == ALIGN
    assert _normal(lib, out=None) == NULL
    assert _normal(lib, B=1 << 16, chunk=1 << 9) == UNSUP      # B * chunk > 2^24
    assert _normal(lib, B=0, qn=None, out=None, ws=None) == OK


def test_normal_workspace_size(nlib):
    lib = nlib
    nb = ctypes.c_size_t(0)
    assert lib.mla_normal_workspace_size(4, 1, 128, 4096, 4096, ctypes.byref(nb)) == OK
    one = nb.value
    # latent + rope + K + V, each rounded to 256 bytes; no carried state with one chunk
    assert one == 4 * 4096 * (512 + 64 + 2 * 128 * 128) * 2
    assert lib.mla_normal_workspace_size(4, 1, 128, 4096, 1024, ctypes.byref(nb)) == OK
    assert nb.value == one // 4 + 4 * 128 * 128 * 4 + 2 * (4 * 128 * 4)   # + output, max and sum state
    assert lib.mla_normal_workspace_size(4, 1, 128, 4096, 1024, None) == NULL


def test_binding_takes_the_output_dtype_from_out_latent():
    """A caller-provided out_latent fixes the output dtype; a conflicting
    out_dtype is rejected before any call (CPU tensors: nothing is launched)."""
    import torch
    q = torch.zeros((1, 1, 1, 512), dtype=torch.bfloat16)
    qp = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16)
    kv = torch.zeros((1, 16, 576), dtype=torch.bfloat16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    out = torch.zeros((1, 1, 1, 512), dtype=torch.float32)
    with pytest.raises(ValueError):
        mk.mla_decode_latent(q, qp, kv, bt, sl, 1, 0.07, out_latent=out, out_dtype=torch.bfloat16)


def test_binding_rejects_misread_tensors():
    """Element types the C ABI would misread, and non-contiguous views, raise
    in the binding (CPU tensors: nothing is launched)."""
    import torch
    q = torch.zeros((1, 1, 1, 512), dtype=torch.bfloat16)
    qp = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16)
    kv = torch.zeros((1, 16, 576), dtype=torch.bfloat16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        mk.mla_decode_latent(q.float(), qp, kv, bt, sl, 1, 0.07)                 # fp32 query
    with pytest.raises(ValueError):
        mk.mla_decode_latent(q, qp, kv, bt.long(), sl, 1, 0.07)                  # int64 table
    with pytest.raises(ValueError):
        mk.mla_decode_latent_fp8(q, qp, kv, bt, sl, 1, 0.07)                     # bf16 rows to the FP8 entry
    wide = torch.zeros((1, 1, 1, 1024), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mk.mla_decode_latent(wide[..., ::2], qp, kv, bt, sl, 1, 0.07)            # strided view
    with pytest.raises(ValueError):
        mk.mla_absorb_q(torch.zeros((1, 1, 1, 128)), torch.zeros((1, 128, 512), dtype=torch.bfloat16))


def test_binding_rejects_shape_mismatches():
    """Sizes the kernels index by must agree across tensors (CPU tensors:
    nothing is launched)."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros((2, 1, 4, 512), dtype=bf)
    kv = torch.zeros((1, 16, 576), dtype=bf)
    bt = torch.zeros((2, 1), dtype=torch.int32)
    sl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        mk.mla_decode_latent(q, torch.zeros((2, 1, 3, 64), dtype=bf), kv, bt, sl, 1, 0.07)   # q_pe heads
    with pytest.raises(ValueError):
        mk.mla_decode_latent(q, torch.zeros((2, 1, 4, 64), dtype=bf), kv, bt[:1], sl, 1, 0.07)  # table rows
    with pytest.raises(ValueError):
        mk.mla_unabsorb_out(q, torch.zeros((3, 128, 512), dtype=bf))                           # w_uv heads
    po = torch.zeros((8, 1, 4, 512), dtype=bf)
    pl = torch.zeros((8, 1, 4))
    ind = torch.zeros(3, dtype=torch.int32)
    w_uv = torch.zeros((4, 128, 512), dtype=bf)
    with pytest.raises(ValueError):
        mk.mla_merge_unabsorb(po, pl[:7], ind, w_uv, 2)                                         # lse rows
    with pytest.raises(ValueError):
        mk.mla_merge_unabsorb(po, pl, ind[:2], w_uv, 2)                                         # split table
    with pytest.raises(ValueError):
        mk.mla_merge_unabsorb(po, pl, ind, w_uv[:3], 2)                                         # w_uv heads
    with pytest.raises(ValueError):
        mk.mla_merge_unabsorb(po, pl, ind, w_uv, 2, out=torch.zeros((2, 1, 4, 64)))             # out width
    with pytest.raises(ValueError):
        mk.mla_merge_unabsorb(po, pl.double(), ind, w_uv, 2)                                    # lse dtype
    with pytest.raises(ValueError):
        mk.mla_absorb_q(torch.zeros((2, 1, 4, 128), dtype=bf), torch.zeros((4, 128, 512), dtype=bf),
                        q_lat=torch.zeros((2, 1, 4, 256), dtype=bf))


def test_binding_rejects_host_tensors():
    """A host tensor never reaches a kernel (it would be a device memory fault)."""
    import torch
    bf = torch.bfloat16
    with pytest.raises(ValueError, match="device"):
        mk.mla_absorb_q(torch.zeros((1, 1, 1, 128), dtype=bf), torch.zeros((1, 128, 512), dtype=bf))


def _decode_inputs(B=2, T=1, H=8, L=256, P=64):
    import torch
    bf = torch.bfloat16
    nb = B * ((L + P - 1) // P)
    return dict(q_lat=torch.zeros((B, T, H, 512), dtype=bf), q_pe=torch.zeros((B, T, H, 64), dtype=bf),
                kv_cache=torch.zeros((nb, P, 576), dtype=bf),
                block_table=torch.zeros((B, nb // B), dtype=torch.int32),
                seqlens=torch.full((B,), L, dtype=torch.int32), max_seqlen=L)


def _call_decode(inp, S, buffers):
    return mk.mla_decode_latent(inp["q_lat"], inp["q_pe"], inp["kv_cache"], inp["block_table"], inp["seqlens"],
                                inp["max_seqlen"], 0.07, num_splits=S, buffers=buffers, merge=False)


@pytest.mark.parametrize("built_for", [dict(S=2), dict(B=1), dict(T=1, H=4), dict(part="shape")])
def test_binding_rejects_decode_buffers_of_another_call(lib, built_for):
    """A DecodeBuffers built for fewer splits, sequences or heads than the call
    it is passed to would be written past its end by the kernels (the C ABI
    sees no buffer sizes): the binding refuses it (CPU tensors: nothing is
    launched either way)."""
    import torch
    inp = _decode_inputs(B=2, T=2, H=8)
    B, T, H = 2, 2, 8
    S = 4
    kw = dict(B=B, T=T, H=H, S=S)
    kw.update({k: v for k, v in built_for.items() if k != "part"})
    buf = mk.DecodeBuffers(kw["B"], kw["T"], kw["H"], 256, 64, kw["S"], "cpu")
    if built_for.get("part") == "shape":
        buf.part_lse = torch.empty((buf.part_lse.shape[0], T, H + 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="buffers"):
        _call_decode(inp, S, buf)


def test_binding_accepts_matching_decode_buffers(lib):
    """The same check passes buffers that fit (the call then stops at the
    host-tensor check, before the C ABI)."""
    inp = _decode_inputs(B=2, T=2, H=8)
    for built_S in (4, 8):   # more splits than needed is also large enough
        buf = mk.DecodeBuffers(2, 2, 8, 256, 64, built_S, "cpu")
        with pytest.raises(ValueError, match="device"):
            _call_decode(inp, 4, buf)


def test_binding_rejects_sparse_buffers_of_another_call(lib):
    import torch
    bf = torch.bfloat16
    B, T, H, topk = 2, 1, 8, 512
    q = torch.zeros((B, T, H, 512), dtype=bf)
    qp = torch.zeros((B, T, H, 64), dtype=bf)
    kv = torch.zeros((16, 64, 576), dtype=bf)
    idx = torch.zeros((B, T, topk), dtype=torch.int32)
    with pytest.raises(ValueError, match="splits"):
        mk.mla_decode_sparse(q, qp, kv, idx, None, 0.07, num_splits=4,
                             buffers=mk.SparseBuffers(B, T, H, topk, 2, "cpu"))
    small = mk.SparseBuffers(1, T, H, topk, 4, "cpu")      # built for one sequence
    with pytest.raises(ValueError, match="buffers"):
        mk.mla_decode_sparse(q, qp, kv, idx, None, 0.07, num_splits=4, buffers=small)
    ok = mk.SparseBuffers(B, T, H, topk, 4, "cpu")
    with pytest.raises(ValueError, match="device"):
        mk.mla_decode_sparse(q, qp, kv, idx, None, 0.07, num_splits=4, buffers=ok)


def test_noalloc_rejects_what_exceeds_its_array(lib):
    """mla_decode_latent_noalloc refuses, before any device call, a split whose
    scratch would not fit in its 64 MiB array, and needs an output."""
    f = lib.mla_decode_latent_noalloc

    def call(B, T, H, maxL, S, out=P16):
        return f(P16, P16, P16, 1 << 14, 64, P16, (maxL + 63) // 64, P16, B, T, H, 512, 64, maxL,
                 ctypes.c_float(0.07), S, out, 0, None, None)
    # 64 sequences x 64 splits x 8 x 128 query rows of bf16 partials: 4 GiB
    assert call(64, 8, 128, 8192, 64) == WS
    # 128 rows x 512 splits of one sequence: 64 MiB of partials plus the rest
    assert call(1, 1, 128, 1 << 20, 512) == WS
    assert call(2, 1, 128, 4096, 4, out=None) == NULL
    assert call(0, 1, 128, 4096, 4) == OK             # empty batch: nothing to do
