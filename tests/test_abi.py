"""The C-ABI library loads, exports every symbol include/qas.h declares, and
rejects bad arguments before touching the device (no compute calls here)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qas.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qas_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def qas():
    import query_aware_sparse_amd
    return query_aware_sparse_amd


def test_library_exports_every_declared_symbol(qas):
    names = _declared()
    assert "qas_decode_layer" in names and len(names) >= 9
    lib = ctypes.CDLL(qas.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the binding exposes the compute entry points under the same names
    for n in names:
        if n not in ("qas_status_string", "qas_last_error", "qas_version"):
            assert hasattr(qas, n), n


def test_status_strings_and_version(qas):
    assert qas.lib.qas_status_string(0) == b"ok"
    assert qas.lib.qas_status_string(5) == b"workspace too small"
    assert qas.version().startswith("qas")


def _cache(qas, **kw):
    c = qas.qas_cache(16, 128, 8, 64, qas.QAS_F16, 0, 1, 1, 1, 0, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _batch(qas, **kw):
    b = qas.qas_batch(2, 10, 6, 0, 8, 8, 8)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


def test_validation_happens_before_any_launch(qas):
    lib = qas.lib
    byref = ctypes.byref
    c, b = _cache(qas), _batch(qas)
    # NULL cache
    assert lib.qas_score_pages(None, byref(b), 8, 1, 32, 8, None) == 1
    # head_dim not supported
    assert lib.qas_score_pages(byref(_cache(qas, head_dim=96)), byref(b), 8, 1, 32, 8,
                               None) == 4
    # page size not a power of two
    assert lib.qas_score_pages(byref(_cache(qas, page_size=12)), byref(b), 8, 1, 32, 8,
                               None) == 2
    # H_q not a multiple of H_kv
    assert lib.qas_score_pages(byref(c), byref(b), 8, 1, 30, 8, None) == 2
    # q dtype differs from kv dtype
    assert lib.qas_score_pages(byref(c), byref(b), 8, 2, 32, 8, None) == 3
    assert b"q_dtype" in lib.qas_last_error()
    # workspace too small
    need = lib.qas_workspace_bytes(2, byref(c), byref(b), 32, 64)
    assert need > 0
    assert lib.qas_decode_layer(byref(c), byref(b), 8, 1, 32, 64, 0.1, None, None, None,
                                8, None, 8, need - 1, None) == 5
    # workspace large enough but not 16-byte aligned (checked before any launch)
    assert lib.qas_decode_layer(byref(c), byref(b), 8, 1, 32, 64, 0.1, None, None, None,
                                8, None, 8, need, None) == 5
    assert b"aligned" in lib.qas_last_error()
    # top-k: k < 1
    assert lib.qas_topk_pages(8, byref(b), 8, 16, 0, 8, None, None) == 2
    # sparse decode: sel_stride < sel_len
    assert lib.qas_sparse_decode(byref(c), byref(b), 8, 1, 32, 8, 4, 5, 0.1, 8, None, 8,
                                 1 << 20, None) == 2
    # append: only one of k_new / v_new for decode layer
    assert lib.qas_decode_layer(byref(c), byref(b), 8, 1, 32, 64, 0.1, 8, None, None, 8,
                                None, 8, need, None) == 1
    # batch with max_pages > total_pages
    assert lib.qas_score_pages(byref(c), byref(_batch(qas, max_pages=11)), 8, 1, 32, 8,
                               None) == 2


def test_fp8_writer_validation(qas):
    """qas_append_fp8 checks its cache, dtypes and sizes before any launch."""
    lib, byref = qas.lib, ctypes.byref
    fp8 = _cache(qas, kv_dtype=qas.QAS_FP8_E4M3, page_size=64, k_scale=8, v_scale=8)
    b = _batch(qas)
    args = (8, 16, 16, 8, 8)          # new_indptr, total_new, max_new, k_new, v_new
    assert lib.qas_append_fp8(None, byref(b), *args, qas.QAS_F32, None) == 1
    # not an fp8 cache
    assert lib.qas_append_fp8(byref(_cache(qas)), byref(b), *args, qas.QAS_F32, None) == 3
    # unsupported input dtype, head size, page size
    assert lib.qas_append_fp8(byref(fp8), byref(b), *args, qas.QAS_FP8_E4M3, None) == 4
    assert lib.qas_append_fp8(byref(_cache(qas, kv_dtype=qas.QAS_FP8_E4M3, page_size=16,
                                           k_scale=8, v_scale=8)),
                              byref(b), *args, qas.QAS_F32, None) == 4
    assert lib.qas_append_fp8(byref(_cache(qas, kv_dtype=qas.QAS_FP8_E4M3, page_size=64,
                                           head_dim=64, k_scale=8, v_scale=8)),
                              byref(b), *args, qas.QAS_BF16, None) == 4
    # scales missing
    assert lib.qas_append_fp8(byref(_cache(qas, kv_dtype=qas.QAS_FP8_E4M3, page_size=32)),
                              byref(b), *args, qas.QAS_F16, None) == 1
    # inconsistent counts, missing rows
    assert lib.qas_append_fp8(byref(fp8), byref(b), 8, 4, 16, 8, 8, qas.QAS_F32, None) == 2
    assert lib.qas_append_fp8(byref(fp8), byref(b), 8, 16, 16, None, 8, qas.QAS_F32, None) == 1
    # nothing to write is a no-op
    assert lib.qas_append_fp8(byref(fp8), byref(b), 8, 0, 0, None, None, qas.QAS_F32, None) == 0


def test_workspace_sizes_are_consistent(qas):
    lib = qas.lib
    c, b = _cache(qas), _batch(qas)
    sd = lib.qas_workspace_bytes(1, ctypes.byref(c), ctypes.byref(b), 32, 64)
    dl = lib.qas_workspace_bytes(2, ctypes.byref(c), ctypes.byref(b), 32, 64)
    assert 0 < sd < dl
    assert sd % 256 == 0 and dl % 256 == 0
    assert lib.qas_workspace_bytes(9, ctypes.byref(c), ctypes.byref(b), 32, 64) == 0


def test_selection_capacity_and_select_validation(qas):
    """List capacity for the top-k joined with fixed sink / local pages, and
    argument checks of qas_select_pages / qas_decode_layer_mixed (no launch)."""
    from ctypes import byref
    lib = qas.lib
    assert qas.qas_selection_capacity(256, 16, 0, 0) == 256
    # 4 sink tokens -> 1 page; 512 local tokens -> up to 32 + 1 pages (unaligned window)
    assert qas.qas_selection_capacity(95, 16, 4, 512) == 95 + 1 + 33
    assert qas.qas_selection_capacity(10, 16, 17, 1) == 10 + 2 + 2
    assert qas.qas_selection_capacity(0, 16, 0, 0) == 0
    assert qas.qas_selection_capacity(4, 16, -1, 0) == 0
    b = _batch(qas)
    # stride below the capacity, negative window: shape errors before any launch
    assert lib.qas_select_pages(8, byref(b), 8, 16, 4, 4, 32, 8, 4, None, None) == 2
    assert b"sel_stride" in lib.qas_last_error()
    assert lib.qas_select_pages(8, byref(b), 8, 16, 4, -1, 0, 8, 16, None, None) == 2
    c = _cache(qas)
    assert lib.qas_decode_layer_mixed(byref(c), byref(b), 8, 1, 32, 64, 0, -5, 0.1, None, None,
                                      None, 8, None, 8, 1 << 30, None) == 2
    # the mixed layer needs the workspace of its list capacity
    cap = qas.qas_selection_capacity(64, 16, 4, 512)
    need = lib.qas_workspace_bytes(2, byref(c), byref(b), 32, cap)
    assert need >= lib.qas_workspace_bytes(2, byref(c), byref(b), 32, 64)
    assert lib.qas_decode_layer_mixed(byref(c), byref(b), 8, 1, 32, 64, 4, 512, 0.1, None, None,
                                      None, 8, None, 8, need - 1, None) == 5


def test_next_row_workspace_sizes(qas):
    """Workspace sizes of the draft-position and exact top-R calls (no launch):
    0 for invalid arguments, 256-byte granular, growing with the draft count
    and with R; the position call's size is the decode layer's over
    B * gamma rows."""
    from ctypes import byref
    lib = qas.lib
    c, b = _cache(qas), _batch(qas)
    # draft positions: gamma rows per request
    p1 = qas.qas_positions_workspace_bytes(c, b, 32, 1, 64)
    p4 = qas.qas_positions_workspace_bytes(c, b, 32, 4, 64)
    rows4 = _batch(qas, batch=b.batch * 4)
    assert p1 == lib.qas_workspace_bytes(2, byref(c), byref(b), 32, 64)
    assert p4 == lib.qas_workspace_bytes(2, byref(c), byref(rows4), 32, 64)
    assert 0 < p1 < p4 and p4 % 256 == 0
    assert qas.qas_positions_workspace_bytes(c, b, 32, 0, 64) == 0
    assert qas.qas_positions_workspace_bytes(c, _batch(qas, batch=0), 32, 4, 64) == 0
    # exact top-R
    t1 = qas.qas_exact_top_r_workspace_bytes(c, b, 32, 1)
    t64 = qas.qas_exact_top_r_workspace_bytes(c, b, 32, 64)
    assert 0 < t1 < t64 and t1 % 256 == 0 and t64 % 256 == 0
    assert qas.qas_exact_top_r_workspace_bytes(c, b, 32, 0) == 0
    assert qas.qas_exact_top_r_workspace_bytes(c, b, 0, 64) == 0
    assert qas.qas_exact_top_r_workspace_bytes(_cache(qas, page_size=12), b, 32, 64) == 0
    # more query heads, more workspace
    assert qas.qas_exact_top_r_workspace_bytes(c, b, 64, 64) > t64


def _prototypes():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    out = {}
    for ret, name, args in re.findall(
            r"([A-Za-z_][\w\s\*]*?)\b(qas_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        params = [] if args.strip() in ("", "void") else [p.strip() for p in args.split(",")]
        out[name] = (ret.strip(), params)
    return out


def _ctype_of(decl):
    """The ctypes type a C parameter or return type must be marshalled as."""
    if "*" in decl or decl.split()[0] == "hipStream_t":
        return "ptr"
    words = decl.replace("const", "").split()
    base = words[0]
    return {"int32_t": "i32", "int": "i32", "qas_status": "i32", "float": "f32",
            "size_t": "size"}[base]


def test_binding_signatures_match_the_header(qas):
    """Every function the header declares has a ctypes signature in the binding
    with the same number of parameters and matching widths (a pointer passed
    without one would be truncated to a C int)."""
    import ctypes
    kinds = {ctypes.c_void_p: "ptr", ctypes.c_char_p: "ptr", ctypes.c_int32: "i32",
             ctypes.c_float: "f32", ctypes.c_size_t: "size"}
    protos = _prototypes()
    assert set(protos) == set(qas._SIGNATURES), set(protos) ^ set(qas._SIGNATURES)
    for name, (ret, params) in protos.items():
        res, args = qas._SIGNATURES[name]
        assert len(args) == len(params), (name, len(args), len(params))
        for i, (p, a) in enumerate(zip(params, args)):
            assert kinds[a] == _ctype_of(p), (name, i, p, a)
        assert kinds[res] == _ctype_of(ret), (name, ret, res)
