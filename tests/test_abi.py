"""Host-side checks of the C ABI: the library loads, exports every function include/bsa.h
declares, and validates arguments before launching anything (no GPU needed: every call here
returns an error status before any HIP work)."""
import ctypes
import os
import re

import pytest

import long_context_attention_sparse_amd as bsa
from long_context_attention_sparse_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_\w+|bsfa_\w+|vs_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bd.load()


def test_exports_match_header(lib):
    declared = _header_functions()
    assert set(declared) == set(bd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(5):
        assert lib.bsa_status_string(code)
    assert lib.bsa_status_string(99) == b"unknown status"


def _struct_fields(name):
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} " + name + ";", text).group(1)
    fields = []
    for decl in filter(None, (d.strip() for d in body.split(";"))):
        # "[const] type[*] a, b" -> ["a", "b"]
        names = re.sub(r"^(const\s+)?\w+\s*\*?\s*", "", decl)
        fields += [x.strip() for x in names.split(",")]
    return fields


def test_struct_layouts_match_header():
    assert _struct_fields("bsa_problem") == [f for f, _ in bd._Problem._fields_]
    assert _struct_fields("bsa_tensor") == [f for f, _ in bd._Tensor._fields_]


def _prob(**kw):
    base = dict(B=1, Hq=4, Hkv=2, Sq=1, Sk=256, D=128, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=0,
                max_seqlen_k=0, softmax_scale=0.0, causal=0, softcap=0.0)
    base.update(kw)
    return bd._Problem(**base)


def _t(ptr=16, dtype=0, sb=256 * 2 * 128, ss=2 * 128, sh=128):
    return bd._Tensor(ptr, dtype, sb, ss, sh)


def _fwd(lib, prob, q=None, k=None, v=None, o=None, pat=None, ws=None, ws_bytes=0):
    q = q or _t(sb=4 * 128, ss=4 * 128)
    k = k or _t()
    v = v or _t()
    o = o or _t(sb=4 * 128, ss=4 * 128)
    return lib.bsa_fwd(ctypes.byref(prob), q, k, v, ctypes.byref(pat) if pat else None, o, None, ws, ws_bytes, None)


def test_fwd_argument_errors(lib):
    assert lib.bsa_fwd(None, _t(), _t(), _t(), None, _t(), None, None, 0, None) == bd.BSA_ERR_INVALID_ARG
    assert _fwd(lib, _prob(Hq=3, Hkv=2)) == bd.BSA_ERR_INVALID_ARG                # Hq % Hkv
    assert _fwd(lib, _prob(B=0)) == bd.BSA_ERR_INVALID_ARG
    assert _fwd(lib, _prob(D=96)) == bd.BSA_ERR_UNSUPPORTED                       # head dim
    assert _fwd(lib, _prob(D=64, Sq=256)) == bd.BSA_ERR_UNSUPPORTED               # D 64 off the decode path
    assert _fwd(lib, _prob(softcap=-1.0)) == bd.BSA_ERR_INVALID_ARG               # softcap < 0
    assert _fwd(lib, _prob(softcap=float("nan"))) == bd.BSA_ERR_INVALID_ARG
    assert _fwd(lib, _prob(softcap=float("inf"))) == bd.BSA_ERR_INVALID_ARG
    assert _fwd(lib, _prob(), q=_t(ptr=0)) == bd.BSA_ERR_INVALID_ARG              # null tensor
    assert _fwd(lib, _prob(), k=_t(dtype=1)) == bd.BSA_ERR_UNSUPPORTED            # f32 inputs
    assert _fwd(lib, _prob(), q=_t(ptr=18)) == bd.BSA_ERR_INVALID_ARG             # misaligned rows
    assert _fwd(lib, _prob(), o=_t(dtype=7)) == bd.BSA_ERR_INVALID_ARG            # output dtype
    assert _fwd(lib, _prob(), k=_t(ss=1 << 25)) == bd.BSA_ERR_UNSUPPORTED          # 64 MB token stride
    assert _fwd(lib, _prob(), v=_t(ss=-128)) == bd.BSA_ERR_UNSUPPORTED             # negative token stride
    bad_kind = bd._Pattern(9, 2, 64, 64, 4, 0, 16, 16, None, None, 0, 0, 0)
    assert _fwd(lib, _prob(), q=_t(ss=1 << 24), pat=bad_kind) == bd.BSA_ERR_INVALID_ARG  # 32 MB passes, the
                                                                                    # pattern check fails


def test_pattern_errors(lib):
    cnt = ctypes.c_int32(0)
    idx = (ctypes.c_int32 * 4)()
    addr = ctypes.addressof
    pat = bd._Pattern(1, 2, 128, 96, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert _fwd(lib, _prob(), pat=pat) == bd.BSA_ERR_UNSUPPORTED                  # block_N
    pat = bd._Pattern(1, 3, 128, 64, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert _fwd(lib, _prob(), pat=pat) == bd.BSA_ERR_INVALID_ARG                  # list heads
    pat = bd._Pattern(1, 2, 128, 128, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert _fwd(lib, _prob(Sk=320), pat=pat) == bd.BSA_ERR_INVALID_ARG            # Sk % block_N
    pat = bd._Pattern(2, 4, 128, 64, 4, 4, addr(cnt), addr(idx), addr(cnt), addr(idx), 0, 0, 0)
    assert _fwd(lib, _prob(causal=0), pat=pat) == bd.BSA_ERR_UNSUPPORTED          # VS block_M > block_N
    pat = bd._Pattern(9, 2, 64, 64, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert _fwd(lib, _prob(), pat=pat) == bd.BSA_ERR_INVALID_ARG                  # kind


def test_workspace_errors(lib):
    prob = _prob(B=4, Hq=8, Hkv=2, Sk=4096)
    need = lib.bsa_workspace_size(ctypes.byref(prob), None)
    assert need > 0                                                               # split-KV decode needs scratch
    assert _fwd(lib, prob) == bd.BSA_ERR_WORKSPACE
    assert _fwd(lib, prob, ws=16, ws_bytes=need - 1) == bd.BSA_ERR_WORKSPACE


def test_combine_and_partials_errors(lib):
    assert lib.bsa_combine(0, 1, 1, 1, 128, 16, 16, _t(), None, None) == bd.BSA_ERR_INVALID_ARG
    assert lib.bsa_combine(2, 1, 1, 1, 80, 16, 16, _t(), None, None) == bd.BSA_ERR_UNSUPPORTED
    prob = _prob()
    assert lib.bsa_fwd_partials(ctypes.byref(prob), _t(), _t(), _t(), None, 1, None, 16, None) == bd.BSA_ERR_INVALID_ARG
    cu = ctypes.c_int32(0)
    varlen = _prob(cu_seqlens_q=ctypes.addressof(cu), cu_seqlens_k=ctypes.addressof(cu), max_seqlen_q=4, max_seqlen_k=4)
    assert lib.bsa_fwd_partials(ctypes.byref(varlen), _t(), _t(), _t(), None, 1, 16, 16, None) == bd.BSA_ERR_UNSUPPORTED
    # partial counts: dense entries are 64-key blocks; E <= 0 picks the split size
    assert lib.bsa_num_partials(ctypes.byref(prob), None, 1) == 4
    assert lib.bsa_num_partials(ctypes.byref(prob), None, 3) == 2
    assert lib.bsa_num_partials(ctypes.byref(_prob(Hq=3)), None, 1) == -1


def test_gated_and_vs_convert_errors(lib):
    prob = _prob(Hq=2, Hkv=2, Sq=256, Sk=256, causal=1)
    T = 16
    q = _t(sb=256 * 2 * 128, ss=2 * 128)
    assert lib.bsa_fwd_gated(ctypes.byref(prob), q, _t(), _t(), None, 128, 128, 0, q, None, None, None, None) \
        == bd.BSA_ERR_INVALID_ARG
    assert lib.bsa_fwd_gated(ctypes.byref(prob), q, _t(), _t(), T, 64, 64, 0, q, None, None, None, None) \
        == bd.BSA_ERR_UNSUPPORTED
    for bad in (2, -1):                                                                 # skipped: 0 or 1
        assert lib.bsa_fwd_gated(ctypes.byref(prob), q, _t(), _t(), T, 128, 128, bad, q, None, None, None, None) \
            == bd.BSA_ERR_INVALID_ARG
    cal = lib.bsfa_calibrate
    assert cal(ctypes.byref(prob), q, _t(), 0, T, T, None) == bd.BSA_ERR_INVALID_ARG         # k_keep < 1
    assert cal(ctypes.byref(prob), q, _t(), 2, None, T, None) == bd.BSA_ERR_INVALID_ARG      # no tile_max
    assert cal(ctypes.byref(prob), q, _t(), 2, T, None, None) == bd.BSA_ERR_INVALID_ARG      # no T
    assert cal(ctypes.byref(_prob(Hq=2, Hkv=2, Sq=256, Sk=256, causal=0)), q, _t(), 2, T, T, None) \
        == bd.BSA_ERR_UNSUPPORTED                                                            # not causal
    assert cal(ctypes.byref(_prob(Hq=2, Hkv=2, Sq=200, Sk=200, causal=1)), q, _t(), 2, T, T, None) \
        == bd.BSA_ERR_UNSUPPORTED                                                            # S % 128
    assert cal(ctypes.byref(_prob(Hq=2, Hkv=2, Sq=4097 * 128, Sk=4097 * 128, causal=1)), q, _t(), 2, T, T,
               None) == bd.BSA_ERR_UNSUPPORTED                                               # rows too long
    # selected attention
    sp = _prob(Hq=4, Hkv=2, Sq=256, Sk=256, causal=1)
    qs = _t(sb=256 * 4 * 128, ss=4 * 128)
    ws = lib.bsa_selected_workspace_size(ctypes.byref(sp), 0, 8, 64)
    assert ws > 8 * 256 * 4 * 128 * 4                                # the float32 partials alone
    assert lib.bsa_selected_workspace_size(ctypes.byref(sp), 0, 8, 128) == 0
    fs = lib.bsa_fwd_selected
    assert fs(ctypes.byref(sp), qs, _t(), _t(), None, 0, 8, 64, qs, None, 256, ws, None) == bd.BSA_ERR_INVALID_ARG
    assert fs(ctypes.byref(sp), qs, _t(), _t(), 16, 0, 0, 64, qs, None, 256, ws, None) == bd.BSA_ERR_INVALID_ARG
    assert fs(ctypes.byref(sp), qs, _t(), _t(), 16, 0, 8, 32, qs, None, 256, ws, None) == bd.BSA_ERR_UNSUPPORTED
    assert fs(ctypes.byref(sp), qs, _t(), _t(), 16, 0, 8, 64, qs, None, 256, ws - 1, None) == bd.BSA_ERR_WORKSPACE
    assert fs(ctypes.byref(sp), qs, _t(), _t(), 16, 0, 8, 64, qs, None, 16, ws, None) == bd.BSA_ERR_WORKSPACE
    assert fs(ctypes.byref(_prob(Hq=32, Hkv=1, Sq=256, Sk=256, causal=1)), _t(sb=256 * 32 * 128, ss=32 * 128),
              _t(), _t(), 16, 0, 8, 64, _t(sb=256 * 32 * 128, ss=32 * 128), None, 256, ws, None) \
        == bd.BSA_ERR_UNSUPPORTED                                                            # group of 32
    # backward
    bp = _prob(Hq=4, Hkv=2, Sq=256, Sk=256, causal=1)
    wsb = lib.bsa_bwd_workspace_size(ctypes.byref(bp), None)
    assert wsb >= 4 * 256 * 4                                          # the row dots
    assert lib.bsa_bwd_workspace_size(ctypes.byref(_prob(Hq=4, Hkv=2, Sq=256, Sk=256, causal=1, softcap=5.0)),
                                      None) == wsb                                    # softcap: same layout
    cnt = ctypes.c_int32(0)
    idx = (ctypes.c_int32 * 4)()
    many = bd._Pattern(1, 4096, 128, 128, 4, 0, ctypes.addressof(cnt), ctypes.addressof(idx), None, None, 0, 0, 0)
    assert lib.bsa_bwd_workspace_size(ctypes.byref(_prob(Hq=4096, Hkv=2, Sq=256, Sk=256, causal=1)),
                                      ctypes.byref(many)) == 0                       # 2^12 query heads
    bw = lib.bsa_bwd
    assert bw(ctypes.byref(bp), qs, _t(), _t(), None, qs, None, qs, 16, 16, 16, 256, wsb, None) \
        == bd.BSA_ERR_INVALID_ARG                                                            # no lse
    assert bw(ctypes.byref(bp), qs, _t(), _t(), None, qs, 16, qs, None, 16, 16, 256, wsb, None) \
        == bd.BSA_ERR_INVALID_ARG                                                            # no dq
    assert bw(ctypes.byref(bp), qs, _t(), _t(), None, qs, 16, qs, 16, 16, 16, 256, wsb - 1, None) \
        == bd.BSA_ERR_WORKSPACE
    assert bw(ctypes.byref(_prob(Hq=4, Hkv=2, Sq=256, Sk=256, causal=1, D=64)), qs, _t(), _t(), None, qs, 16, qs,
              16, 16, 16, 256, wsb, None) == bd.BSA_ERR_UNSUPPORTED                          # head dim 64
    sc = _prob(Hq=2, Hkv=2, Sq=256, Sk=256, causal=1, softcap=30.0)
    assert lib.bsa_fwd_gated(ctypes.byref(sc), q, _t(), _t(), T, 128, 128, 0, q, None, None, None, None) \
        == bd.BSA_ERR_UNSUPPORTED
    nc = _prob(Hq=2, Hkv=2, Sq=256, Sk=256, causal=0)
    assert lib.bsa_fwd_gated(ctypes.byref(nc), q, _t(), _t(), T, 128, 128, 0, q, None, None, None, None) \
        == bd.BSA_ERR_UNSUPPORTED
    x = 16
    assert lib.vs_convert_indexes(x, x, x, x, 1, 1, 4, 4, 256, 64, 64, 0, x, x, x, x, None) == bd.BSA_ERR_UNSUPPORTED
    assert lib.vs_convert_indexes(x, x, x, x, 1, 1, 4, 4, 256, 128, 64, 1, x, x, x, x, None) == bd.BSA_ERR_UNSUPPORTED
    assert lib.vs_convert_indexes(None, x, x, x, 1, 1, 4, 4, 256, 64, 64, 1, x, x, x, x, None) == bd.BSA_ERR_INVALID_ARG
    assert lib.vs_convert_indexes(x, x, x, x, 0, 1, 4, 4, 256, 64, 64, 1, x, x, x, x, None) == bd.BSA_ERR_INVALID_ARG
    mh = lib.vs_convert_indexes_mergehead
    assert mh(x, x, x, x, None, x, 1, 1, 4, 4, 256, 64, 64, 1, x, x, x, x, None) == bd.BSA_ERR_INVALID_ARG
    assert mh(x, x, x, x, x, None, 1, 1, 4, 4, 256, 64, 64, 1, x, x, x, x, None) == bd.BSA_ERR_INVALID_ARG
    assert mh(x, x, x, x, x, x, 1, 1, 4, 4, 256, 64, 64, 0, x, x, x, x, None) == bd.BSA_ERR_UNSUPPORTED
    assert mh(x, x, x, x, x, x, 0, 1, 4, 4, 256, 64, 64, 1, x, x, x, x, None) == bd.BSA_ERR_INVALID_ARG


def test_check_pattern_errors(lib):
    cnt = ctypes.c_int32(0)
    idx = (ctypes.c_int32 * 4)()
    res = (ctypes.c_int32 * 3)()
    addr = ctypes.addressof
    ok = bd._Pattern(1, 2, 128, 64, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    prob = _prob()
    chk = lib.bsa_check_pattern
    assert chk(None, ctypes.byref(ok), addr(res), None) == bd.BSA_ERR_INVALID_ARG
    assert chk(ctypes.byref(prob), None, addr(res), None) == bd.BSA_ERR_INVALID_ARG           # no pattern
    assert chk(ctypes.byref(prob), ctypes.byref(ok), None, None) == bd.BSA_ERR_INVALID_ARG     # no result
    assert chk(ctypes.byref(prob), ctypes.byref(ok), addr(res) + 2, None) == bd.BSA_ERR_INVALID_ARG  # misaligned
    assert chk(ctypes.byref(_prob(Hq=3, Hkv=2)), ctypes.byref(ok), addr(res), None) == bd.BSA_ERR_INVALID_ARG
    dense = bd._Pattern(0, 2, 128, 64, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert chk(ctypes.byref(prob), ctypes.byref(dense), addr(res), None) == bd.BSA_ERR_INVALID_ARG
    bad_n = bd._Pattern(1, 2, 128, 96, 4, 0, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert chk(ctypes.byref(prob), ctypes.byref(bad_n), addr(res), None) == bd.BSA_ERR_UNSUPPORTED
    vs_nocols = bd._Pattern(2, 2, 64, 64, 4, 4, addr(cnt), addr(idx), None, None, 0, 0, 0)
    assert chk(ctypes.byref(prob), ctypes.byref(vs_nocols), addr(res), None) == bd.BSA_ERR_INVALID_ARG
