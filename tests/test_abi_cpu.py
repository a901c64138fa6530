"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/flexmi.h, and rejects each kind of invalid argument with
its status code before any HIP call is made (the pointers below are fake
16-byte-aligned addresses that are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import programmable_block_sparse_amd as pbs
from programmable_block_sparse_amd import flex_block_mask, flex_mask_params, flex_score_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flexmi.h")

FAKE = 0x10000   # aligned, never dereferenced
OK, NULL, SHAPE, GQA, BLOCKMASK, UNSUPPORTED, LAYOUT, WORKSPACE, HIP, PARAM = range(10)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pbs.library_path()):
        pytest.skip("libflexmi.so not built")
    return pbs.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flex_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(pbs.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pbs.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (flex_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    names = ["FLEX_OK", "FLEX_ERR_NULL", "FLEX_ERR_SHAPE", "FLEX_ERR_GQA", "FLEX_ERR_BLOCKMASK",
             "FLEX_ERR_UNSUPPORTED", "FLEX_ERR_LAYOUT", "FLEX_ERR_WORKSPACE", "FLEX_ERR_HIP", "FLEX_ERR_PARAM"]
    for code, name in enumerate(names):
        assert pbs.flex_status_string(code) == name
    assert pbs.flex_status_string(99) == "FLEX_ERR_UNKNOWN"


def _bm(L, S, qb, kb, B=1, H=1):
    c = flex_block_mask()
    c.B, c.H, c.q_block, c.kv_block = B, H, qb, kb
    c.num_q_blocks, c.num_kv_blocks = -(-L // qb), -(-S // kb)
    c.kv_num_blocks = c.kv_indices = c.full_kv_num_blocks = c.full_kv_indices = FAKE
    return c


def _mask(kind="causal", q_offset=0, window=0, sinks=0, doc=None, doc_len=0):
    m = flex_mask_params()
    m.kind, m.q_offset, m.window, m.sinks = pbs.MASK_KINDS[kind], q_offset, window, sinks
    m.doc_id, m.doc_len = doc, doc_len
    return m


def _score(kind="none", cap=0.0, alibi_m=8.0):
    s = flex_score_params()
    s.kind, s.cap, s.alibi_m = pbs.SCORE_KINDS[kind], cap, alibi_m
    return s


def build(lib, mask, L, S, bm):
    return lib.flex_blockmask_build(ctypes.byref(mask) if mask is not None else None, L, S,
                                    ctypes.byref(bm) if bm is not None else None, None)


def test_builder_rejects(lib):
    L = S = 256
    assert build(lib, None, L, S, _bm(L, S, 64, 64)) == NULL
    assert build(lib, _mask(), L, S, None) == NULL
    bad = _bm(L, S, 64, 64); bad.kv_indices = None
    assert build(lib, _mask(), L, S, bad) == NULL
    assert build(lib, _mask(), 0, S, _bm(1, S, 64, 64)) == SHAPE
    assert build(lib, _mask(), L, 1 << 30, _bm(L, 1 << 20, 64, 64)) == SHAPE
    small = _bm(L, S, 64, 64); small.num_q_blocks = 3
    assert build(lib, _mask(), L, S, small) == BLOCKMASK
    assert "too small" in pbs.flex_last_error()
    large = _bm(L, S, 64, 64); large.num_kv_blocks = 5
    assert build(lib, _mask(), L, S, large) == BLOCKMASK
    assert "too large" in pbs.flex_last_error()
    assert build(lib, _mask(), L, S, _bm(L, S, 2048, 64)) == BLOCKMASK
    assert build(lib, _mask(), L, S, _bm(L, S, 64, 64, B=0)) == BLOCKMASK
    m = _mask(); m.kind = 7
    assert build(lib, m, L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("causal_window_sinks", window=0), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("causal_window_sinks", window=4, sinks=-1), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("doc_causal", doc=None), L, S, _bm(L, S, 64, 64)) == NULL
    assert build(lib, _mask("doc_causal", doc=FAKE, doc_len=S - 1), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("doc_causal", doc=FAKE, doc_len=S, q_offset=-1), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("doc_causal", doc=FAKE, doc_len=S, q_offset=5), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask("doc_causal", doc=FAKE, doc_len=1 << 29), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask(q_offset=1 << 30), L, S, _bm(L, S, 64, 64)) == PARAM
    assert build(lib, _mask(), 64, 64 * 70000, _bm(64, 64 * 70000, 64, 64)) == UNSUPPORTED
    assert build(lib, _mask(), 70000, 64, _bm(70000, 64, 1, 64)) == UNSUPPORTED
    assert build(lib, _mask(), 64, 64, _bm(64, 64, 64, 64, B=300, H=300)) == UNSUPPORTED


class Fwd:
    """Valid argument set for flex_attn_fwd; tests change one thing at a time."""

    def __init__(self, dtype=1, B=2, Hq=4, Hkv=2, L=256, S=256, D=64, qb=128, kb=64):
        self.q = self.k = self.v = self.out = FAKE
        self.lse = FAKE
        self.dtype, self.B, self.Hq, self.Hkv, self.L, self.S, self.D = dtype, B, Hq, Hkv, L, S, D
        self.qs = [Hq * L * D, L * D, D]
        self.ks = [Hkv * S * D, S * D, D]
        self.vs = list(self.ks)
        self.scale = 0.0
        self.score = _score("softcap", cap=30.0)
        self.mask = _mask("causal", q_offset=S - L)
        self.bm = _bm(L, S, qb, kb)
        self.ws, self.ws_bytes = None, 0

    def call(self, lib):
        a3 = lambda x: None if x is None else (ctypes.c_int64 * 3)(*x)
        ref = lambda x: None if x is None else ctypes.byref(x)
        return lib.flex_attn_fwd(self.q, self.k, self.v, self.dtype, self.B, self.Hq, self.Hkv, self.L, self.S,
                                 self.D, a3(self.qs), a3(self.ks), a3(self.vs), ctypes.c_float(self.scale),
                                 ref(self.score), ref(self.mask), ref(self.bm), self.out, self.lse, self.ws,
                                 self.ws_bytes, None)


@pytest.mark.parametrize("change,code", [
    (lambda f: setattr(f, "q", None), NULL),
    (lambda f: setattr(f, "out", None), NULL),
    (lambda f: setattr(f, "ks", None), NULL),
    (lambda f: setattr(f, "score", None), NULL),
    (lambda f: setattr(f, "mask", None), NULL),
    (lambda f: setattr(f, "bm", None), NULL),
    (lambda f: setattr(f.bm, "full_kv_indices", None), NULL),
    (lambda f: setattr(f, "B", 0), SHAPE),
    (lambda f: setattr(f, "L", -3), SHAPE),
    (lambda f: setattr(f, "Hkv", 3), GQA),
    (lambda f: setattr(f, "dtype", 2), UNSUPPORTED),
    (lambda f: setattr(f, "D", 96), UNSUPPORTED),
    (lambda f: setattr(f.bm, "num_q_blocks", 1), BLOCKMASK),
    (lambda f: setattr(f.bm, "num_kv_blocks", 8), BLOCKMASK),
    (lambda f: setattr(f.bm, "B", 3), BLOCKMASK),
    (lambda f: setattr(f.bm, "H", 2), BLOCKMASK),
    (lambda f: (setattr(f.bm, "q_block", 48), setattr(f.bm, "num_q_blocks", 6)), UNSUPPORTED),
    (lambda f: (setattr(f.bm, "kv_block", 32), setattr(f.bm, "num_kv_blocks", 8)), UNSUPPORTED),
    (lambda f: setattr(f, "q", FAKE + 8), LAYOUT),
    (lambda f: setattr(f, "out", FAKE + 4), LAYOUT),
    (lambda f: setattr(f, "lse", FAKE + 2), LAYOUT),
    (lambda f: setattr(f, "qs", [1 << 20, 1 << 14, 66]), LAYOUT),
    (lambda f: setattr(f, "ks", [-64, 64, 64]), LAYOUT),
    (lambda f: setattr(f, "score", _score("softcap", cap=0.0)), PARAM),
    (lambda f: setattr(f, "score", _score("softcap_alibi", cap=float("inf"))), PARAM),
    (lambda f: setattr(f.score, "kind", 5), PARAM),
    (lambda f: setattr(f.mask, "kind", -1), PARAM),
    (lambda f: setattr(f, "mask", _mask("causal_window_sinks", window=0)), PARAM),
    (lambda f: setattr(f, "mask", _mask("doc_causal", doc=None)), NULL),
    (lambda f: setattr(f, "mask", _mask("doc_causal", doc=FAKE, doc_len=100)), PARAM),
    (lambda f: setattr(f, "mask", _mask("doc_causal", doc=FAKE + 2, doc_len=256)), LAYOUT),
    (lambda f: setattr(f, "scale", float("inf")), PARAM),
])
def test_fwd_rejects(lib, change, code):
    f = Fwd()
    change(f)
    assert f.call(lib) == code, pbs.flex_last_error()
    assert pbs.flex_last_error() != ""


def test_fp32_alignment_unit_is_four_elements(lib):
    f = Fwd(dtype=0)
    f.qs = [f.Hq * f.L * 68, f.L * 68, 68]        # 68 floats = 272 bytes: aligned for fp32 ...
    f.q = FAKE + 16
    f.mask = _mask("causal_window_sinks", window=0)  # ... so the first failure is the mask
    assert f.call(lib) == PARAM
    f.qs = [f.Hq * f.L * 66, f.L * 66, 66]
    assert f.call(lib) == LAYOUT


def _program(*clauses, q_offset=0, doc=None, doc_len=0):
    m = _mask("program", q_offset=q_offset, doc=doc, doc_len=doc_len)
    m.n_clauses = len(clauses)
    for i, c in enumerate(clauses):
        m.clause[i].n = len(c)
        for j, (name, arg) in enumerate(c):
            m.clause[i].lit[j].kind = pbs.PREDICATES[name] if isinstance(name, str) else name
            m.clause[i].lit[j].arg = arg
    return m


def test_program_mask_validation(lib):
    L = S = 256
    ok = _program([("causal", 0)], [("window", 64), ("kv_lt", 4)])
    bm = _bm(L, S, 64, 64)
    # valid programs pass validation and fail only at the (absent) GPU launch
    assert build(lib, ok, L, S, bm) in (0, HIP)
    assert build(lib, _program(), L, S, bm) == PARAM                                   # no clause
    five = _program(*[[("causal", 0)]] * 4)
    five.n_clauses = 5
    assert build(lib, five, L, S, bm) == PARAM                                         # too many clauses
    empty = _program([("causal", 0)])
    empty.clause[0].n = 0
    assert build(lib, empty, L, S, bm) == PARAM                                        # empty clause
    three = _program([("causal", 0)])
    three.clause[0].n = 3
    assert build(lib, three, L, S, bm) == PARAM                                        # too many predicates
    assert build(lib, _program([(9, 0)]), L, S, bm) == PARAM                           # unknown predicate
    for name, arg in (("window", 0), ("chunk", 0), ("stride", 0), ("kv_lt", -1), ("head_lt", -2)):
        assert build(lib, _program([(name, arg)]), L, S, bm) == PARAM, name
    assert build(lib, _program([("doc", 0)]), L, S, bm) == NULL                        # doc predicate, no ids
    assert build(lib, _program([("doc", 0)], doc=FAKE, doc_len=S - 1), L, S, bm) == PARAM
    assert build(lib, _program([("doc", 0)], doc=FAKE, doc_len=S, q_offset=-1), L, S, bm) == PARAM


def test_fwd_program_and_score_rules(lib):
    f = Fwd()
    f.mask = _program([("causal", 0)], [("head_lt", 2), ("window", 32)], q_offset=f.S - f.L)
    assert f.call(lib) == BLOCKMASK                     # reads the head but the block mask is broadcast
    assert "head" in pbs.flex_last_error()
    f = Fwd()
    f.score = _score("alibi", alibi_m=float("nan"))
    assert f.call(lib) == PARAM
    f = Fwd()
    f.score = _score("alibi", cap=0.0)                   # no cap needed for the uncapped ALiBi
    assert f.call(lib) in (0, HIP)


def test_aux_entry_point_checks_max_scores_alignment(lib):
    f = Fwd()
    a3 = lambda x: (ctypes.c_int64 * 3)(*x)
    call = lambda ms: lib.flex_attn_fwd_aux(f.q, f.k, f.v, f.dtype, f.B, f.Hq, f.Hkv, f.L, f.S, f.D, a3(f.qs),
                                             a3(f.ks), a3(f.vs), ctypes.c_float(0.0), ctypes.byref(f.score),
                                             ctypes.byref(f.mask), ctypes.byref(f.bm), f.out, f.lse, ms, None, 0,
                                             None)
    assert call(FAKE + 2) == LAYOUT
    assert call(None) in (0, HIP)


def test_workspace_query_rejects_bad_shapes(lib):
    bm = _bm(256, 256, 128, 64)
    assert lib.flex_attn_fwd_workspace_bytes(1, 2, 4, 3, 256, 256, 64, ctypes.byref(bm)) == 0
    assert lib.flex_attn_fwd_workspace_bytes(1, 2, 4, 2, 256, 256, 96, ctypes.byref(bm)) == 0
    assert lib.flex_attn_fwd_workspace_bytes(1, 2, 4, 2, 256, 256, 64, None) == 0


def _bmq(L, S, qb, kb, B=1, H=1):
    c = pbs.flex_block_mask_q()
    c.B, c.H, c.q_block, c.kv_block = B, H, qb, kb
    c.num_q_blocks, c.num_kv_blocks = -(-L // qb), -(-S // kb)
    c.q_num_blocks = c.q_indices = c.full_q_num_blocks = c.full_q_indices = FAKE
    return c


class Bwd(Fwd):
    """Valid argument set for flex_attn_bwd; tests change one thing at a time."""

    def __init__(self, **kw):
        super().__init__(**kw)
        self.dout = self.dq = self.dk = self.dv = FAKE
        self.bmq = _bmq(self.L, self.S, self.bm.q_block, self.bm.kv_block)
        self.ws = FAKE
        self.ws_bytes = 2 * self.B * self.Hq * (-(-self.L // 128) * 128) * 4    # columns too short to share

    def call(self, lib):
        a3 = lambda x: None if x is None else (ctypes.c_int64 * 3)(*x)
        ref = lambda x: None if x is None else ctypes.byref(x)
        return lib.flex_attn_bwd(self.q, self.k, self.v, self.out, self.dout, self.lse, self.dtype, self.B, self.Hq,
                                 self.Hkv, self.L, self.S, self.D, a3(self.qs), a3(self.ks), a3(self.vs),
                                 ctypes.c_float(self.scale), ref(self.score), ref(self.mask), ref(self.bm),
                                 ref(self.bmq), self.dq, self.dk, self.dv, self.ws, self.ws_bytes, None)


@pytest.mark.parametrize("change,code", [
    (lambda f: setattr(f, "dout", None), NULL),
    (lambda f: setattr(f, "lse", None), NULL),
    (lambda f: setattr(f, "dk", None), NULL),
    (lambda f: setattr(f, "bmq", None), NULL),
    (lambda f: setattr(f.bmq, "full_q_indices", None), NULL),
    (lambda f: setattr(f, "Hkv", 3), GQA),
    (lambda f: setattr(f.bmq, "num_kv_blocks", 3), BLOCKMASK),
    (lambda f: setattr(f.bmq, "H", 4), BLOCKMASK),
    (lambda f: (setattr(f.bm, "q_block", 32), setattr(f.bm, "num_q_blocks", 8),
                setattr(f.bmq, "q_block", 32), setattr(f.bmq, "num_q_blocks", 8)), UNSUPPORTED),
    (lambda f: setattr(f, "dq", FAKE + 8), LAYOUT),
    (lambda f: setattr(f, "dv", FAKE + 2), LAYOUT),
    (lambda f: setattr(f, "ws", None), WORKSPACE),
    (lambda f: setattr(f, "ws_bytes", f.ws_bytes - 4), WORKSPACE),
    (lambda f: setattr(f, "ws", FAKE + 4), LAYOUT),
    (lambda f: setattr(f, "scale", float("nan")), PARAM),
    (lambda f: setattr(f, "mask", _mask("causal_window_sinks", window=0)), PARAM),
])
def test_bwd_rejects(lib, change, code):
    f = Bwd()
    change(f)
    assert f.call(lib) == code, pbs.flex_last_error()
    assert pbs.flex_last_error() != ""


def test_bwd_valid_call_reaches_the_launch(lib):
    for kw in ({}, {"dtype": 0, "D": 128}, {"L": 100, "S": 300}):
        f = Bwd(**kw)
        assert f.call(lib) in (OK, HIP), pbs.flex_last_error()


def test_bwd_workspace_bytes(lib):
    ws = lambda B, Hq, Hkv, L, S, D, bm, dtype=1: lib.flex_attn_bwd_workspace_bytes(dtype, B, Hq, Hkv, L, S, D,
                                                                                    ctypes.byref(bm))
    # two float32 per (batch, query head, row), rows padded to a multiple of 128
    assert ws(2, 3, 3, 100, 100, 64, _bm(100, 100, 128, 64)) == 2 * 2 * 3 * 128 * 4
    assert ws(1, 1, 1, 129, 129, 64, _bm(129, 129, 64, 64)) == 2 * 256 * 4
    # columns of up to 4 * 64 * 2 = 512 Q-side tiles may be shared by up to four
    # workgroups: four float32 (dk, dv) partials per 64-key column
    L = S = 8192
    cols = 2 * 2 * (S // 64)
    assert ws(2, 8, 2, L, S, 128, _bm(L, S, 128, 64)) == 2 * 2 * 8 * L * 4 + 4 * cols * 2 * 64 * 128 * 4
    assert ws(0, 1, 1, 10, 10, 64, _bm(10, 10, 64, 64)) == 0
    assert ws(1, 1, 1, 0, 10, 64, _bm(10, 10, 64, 64)) == 0
    assert ws(1, 4, 3, 10, 10, 64, _bm(10, 10, 64, 64)) == 0              # not a GQA ratio
    assert ws(1, 1, 1, 10, 10, 96, _bm(10, 10, 64, 64)) == 0              # head dim
    assert ws(1, 1, 1, 10, 10, 64, _bm(10, 10, 32, 64)) == 0              # q_block
    assert lib.flex_attn_bwd_workspace_bytes(1, 1, 1, 1, 10, 10, 64, None) == 0


def test_transpose_rejects(lib):
    bm, bmq = _bm(256, 300, 128, 64), _bmq(256, 300, 128, 64)
    call = lambda a, b: lib.flex_blockmask_transpose(None if a is None else ctypes.byref(a),
                                                     None if b is None else ctypes.byref(b), None)
    assert call(bm, bmq) in (OK, HIP)
    assert call(None, bmq) == NULL
    assert call(bm, None) == NULL
    bmq.q_indices = None
    assert call(bm, bmq) == NULL
    bmq = _bmq(256, 300, 128, 64)
    bmq.num_q_blocks = 3
    assert call(bm, bmq) == BLOCKMASK
    bmq = _bmq(256, 300, 128, 64, B=2)
    assert call(bm, bmq) == BLOCKMASK


def test_blockmask_utilities_reject(lib):
    bm = _bm(256, 300, 128, 64, B=2, H=3)
    ref = lambda x: None if x is None else ctypes.byref(x)
    assert lib.flex_blockmask_to_dense(ref(bm), FAKE, None) in (OK, HIP)
    assert lib.flex_blockmask_to_dense(None, FAKE, None) == NULL
    assert lib.flex_blockmask_to_dense(ref(bm), None, None) == NULL
    assert lib.flex_blockmask_grid(ref(bm), 0, 4, FAKE, None) == SHAPE
    assert lib.flex_blockmask_grid(ref(bm), 2, 2, FAKE, None) in (OK, HIP)
    assert lib.flex_blockmask_sparsity(ref(bm), FAKE + 4, None) == LAYOUT
    assert lib.flex_blockmask_sparsity(ref(bm), FAKE, None) in (OK, HIP)
    big = _bm(64, 64 * 70000, 64, 64)
    assert lib.flex_blockmask_to_dense(ref(big), FAKE, None) == UNSUPPORTED
    # slicing: ranges inside the dims and non-empty, out dims equal to the ranges
    r = lambda *v: (ctypes.c_int32 * 6)(*v)
    out = _bm(128, 300, 128, 64, B=1, H=2)
    assert lib.flex_blockmask_slice(ref(bm), r(1, 2, 1, 3, 1, 2), ref(out), None) in (OK, HIP)
    assert lib.flex_blockmask_slice(ref(bm), r(1, 2, 1, 3, 1, 3), ref(out), None) == BLOCKMASK   # rows past nQB
    assert lib.flex_blockmask_slice(ref(bm), r(1, 1, 1, 3, 1, 2), ref(out), None) == BLOCKMASK   # empty range
    assert lib.flex_blockmask_slice(ref(bm), r(0, 2, 1, 3, 1, 2), ref(out), None) == BLOCKMASK   # out B differs
    assert lib.flex_blockmask_slice(ref(bm), None, ref(out), None) == NULL
    # cropping: only to fewer blocks, out dims for the new lengths
    adj = _bm(200, 100, 128, 64, B=2, H=3)
    assert lib.flex_blockmask_adjust(ref(bm), 200, 100, ref(adj), None) in (OK, HIP)
    assert lib.flex_blockmask_adjust(ref(bm), 200, 400, ref(_bm(200, 400, 128, 64, B=2, H=3)), None) == BLOCKMASK
    assert lib.flex_blockmask_adjust(ref(bm), 0, 100, ref(adj), None) == SHAPE
    assert lib.flex_blockmask_adjust(ref(bm), 200, 100, ref(_bm(200, 100, 128, 64)), None) == BLOCKMASK


def test_paged_forward_rejects(lib):
    f = Fwd(L=16, S=1000, qb=16)
    a3 = lambda x: (ctypes.c_int64 * 3)(*x)
    pages = pbs.flex_kv_pages()
    pages.page_table, pages.page_size, pages.max_pages, pages.num_pages = FAKE, 64, 16, 40

    def call(pg):
        return lib.flex_attn_fwd_paged(f.q, f.k, f.v, f.dtype, f.B, f.Hq, f.Hkv, f.L, f.S, f.D, a3(f.qs),
                                       a3([64 * 64 * 2, 64 * 64, 64]), a3([64 * 64 * 2, 64 * 64, 64]),
                                       ctypes.c_float(0.0), ctypes.byref(f.score), ctypes.byref(f.mask),
                                       ctypes.byref(f.bm), None if pg is None else ctypes.byref(pg), f.out, f.lse,
                                       None, None, 0, None)
    assert call(pages) in (OK, HIP), pbs.flex_last_error()
    assert call(None) == NULL
    for field, bad, code in (("page_size", 48, PARAM), ("page_size", 96, PARAM), ("page_size", 32, PARAM),
                             ("max_pages", 15, PARAM), ("num_pages", 0, PARAM), ("page_table", None, NULL),
                             ("page_table", FAKE + 2, LAYOUT)):
        pg = pbs.flex_kv_pages()
        pg.page_table, pg.page_size, pg.max_pages, pg.num_pages = FAKE, 64, 16, 40
        setattr(pg, field, bad)
        assert call(pg) == code, (field, bad, pbs.flex_last_error())


def test_paged_backward_rejects(lib):
    """flex_attn_bwd_paged: the backward's checks plus the page geometry."""
    f = Bwd(L=128, S=1000, qb=64)
    a3 = lambda x: (ctypes.c_int64 * 3)(*x)
    ref = lambda x: None if x is None else ctypes.byref(x)

    def call(pg, bmq=f.bmq):
        return lib.flex_attn_bwd_paged(f.q, f.k, f.v, ref(pg), f.out, f.dout, f.lse, f.dtype, f.B, f.Hq, f.Hkv, f.L,
                                       f.S, f.D, a3(f.qs), a3([64 * 64 * 2, 64 * 64, 64]),
                                       a3([64 * 64 * 2, 64 * 64, 64]), ctypes.c_float(0.0), ref(f.score),
                                       ref(f.mask), ref(f.bm), ref(bmq), f.dq, f.dk, f.dv, f.ws, f.ws_bytes, None)
    pages = pbs.flex_kv_pages()
    pages.page_table, pages.page_size, pages.max_pages, pages.num_pages = FAKE, 64, 16, 40
    assert call(pages) in (OK, HIP), pbs.flex_last_error()
    assert call(None) == NULL
    assert call(pages, bmq=None) == NULL
    for field, bad, code in (("page_size", 48, PARAM), ("page_size", 32, PARAM), ("max_pages", 15, PARAM),
                             ("num_pages", 0, PARAM), ("page_table", None, NULL), ("page_table", FAKE + 2, LAYOUT)):
        pg = pbs.flex_kv_pages()
        pg.page_table, pg.page_size, pg.max_pages, pg.num_pages = FAKE, 64, 16, 40
        setattr(pg, field, bad)
        assert call(pg) == code, (field, bad, pbs.flex_last_error())


def test_per_batch_arrays_need_per_batch_block_mask(lib):
    f = Fwd()
    f.mask.kv_lens = FAKE
    assert f.call(lib) == BLOCKMASK                       # block mask B=1 but two batches
    f.bm.B = f.B
    assert f.call(lib) in (OK, HIP)
    f.mask.q_offsets = FAKE + 2
    assert f.call(lib) == LAYOUT
    b = Bwd()
    b.mask.kv_lens = FAKE
    assert b.call(lib) == BLOCKMASK                       # the backward checks the same
    b.bm.B = b.bmq.B = b.B
    assert b.call(lib) in (OK, HIP), pbs.flex_last_error()
    b.mask.q_offsets = FAKE + 2
    assert b.call(lib) == LAYOUT


def test_binding_rejects_host_tensors_before_any_launch():
    """The binding checks every tensor it marshals (device, dtype, exact shape,
    contiguity) and raises ValueError before a pointer reaches the library:
    host tensors here, where no GPU exists, must never be passed on."""
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    bm = pbs.BlockMask(i32(1, 1, 1), i32(1, 1, 1, 1), i32(1, 1, 1), i32(1, 1, 1, 1), 64, 64, 64, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        pbs.flex_attn_fwd(q, k, k, block_mask=bm)
    with pytest.raises(ValueError, match="GPU tensor"):
        pbs.flex_attn_fwd_paged(q, k, k, i32(1, 1), S=64, block_mask=bm)
    with pytest.raises(ValueError):
        pbs.flex_attn_bwd(q, k, k, q, q, torch.zeros((1, 2, 64)), block_mask=bm, block_mask_q=None)
    with pytest.raises(ValueError, match="must be on"):
        bm.to_c()
    with pytest.raises(ValueError, match="must be on"):
        pbs.flex_blockmask_build(pbs.MaskSpec(kind="causal"), 64, 64, 64, 64, out=bm)
    # wrong shapes are caught whatever the device
    bad = pbs.BlockMask(i32(1, 1, 2), i32(1, 1, 1, 1), i32(1, 1, 1), i32(1, 1, 1, 1), 64, 64, 64, 64)
    with pytest.raises(ValueError, match="shape|must be on"):
        bad._validate(torch.device("cpu"))


def test_noalloc_entry_point_checks(lib):
    """flex_attn_fwd_noalloc takes flex_attn_fwd's checks, and refuses before
    any HIP call a call whose split-KV partials exceed its scratch array."""
    lib.flex_attn_fwd_noalloc.restype = ctypes.c_int
    a3 = lambda x: (ctypes.c_int64 * 3)(*x)

    def call(f):
        return lib.flex_attn_fwd_noalloc(f.q, f.k, f.v, f.dtype, f.B, f.Hq, f.Hkv, f.L, f.S, f.D, a3(f.qs), a3(f.ks),
                                         a3(f.vs), ctypes.c_float(f.scale), ctypes.byref(f.score),
                                         ctypes.byref(f.mask), ctypes.byref(f.bm), f.out, f.lse, None)
    f = Fwd()
    f.q = None
    assert call(f) == NULL
    f = Fwd(Hq=4, Hkv=1)
    f.bm.num_kv_blocks = 3
    assert call(f) == BLOCKMASK
    # 1000 (batch, K/V head) units of 64 packed rows: one split each, 125*32*16 rows of
    # (128 + 4) floats = 33.8 MB of partials, above the 32 MiB array
    f = Fwd(B=125, Hq=32, Hkv=8, L=16, S=2048, D=128, qb=16)
    need = lib.flex_attn_fwd_workspace_bytes(f.dtype, f.B, f.Hq, f.Hkv, f.L, f.S, f.D, ctypes.byref(f.bm))
    assert need > 32 << 20
    assert call(f) == WORKSPACE
    assert "scratch" in pbs.flex_last_error()
