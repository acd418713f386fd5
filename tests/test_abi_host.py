"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call.  No GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tokengate.h")


def _declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_four_hot_path_calls():
    syms = _declared_symbols()
    for s in ("tg_gate_score", "tg_topk_select", "tg_gather_kept", "tg_keybias_attn_prefill"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    from learned_token_pruning_05_amd import _lib
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for s in _declared_symbols():
        assert hasattr(raw, s), s
        assert s in _lib.SIGNATURES, s


def test_status_strings(lib):
    from learned_token_pruning_05_amd import _lib
    assert _lib.status_string(0) == "TG_OK"
    assert _lib.status_string(3) == "TG_ERR_WORKSPACE"
    assert _lib.status_string(99) == "TG_ERR_UNKNOWN"


def test_kept_counts_matches_definition(lib):
    from learned_token_pruning_05_amd import _lib
    for w in workloads.all_configs() + [workloads.custom([5, 1, 9, 0], [2, 1, 0, 0], [1, 7, 3, 0])]:
        got = _lib.tg_kept_counts(w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc_arr)
        want = oracle.kept_counts(w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc_arr)
        assert got.tolist() == want.tolist(), w.name


@pytest.mark.parametrize("bad", [
    dict(doc_end=[6]),          # span beyond the sequence
    dict(doc_begin=[3], doc_end=[2]),
    dict(k_doc=[-1]),
    dict(cu=[1, 6]),            # cu_seqlens[0] != 0
])
def test_kept_counts_rejects(lib, bad):
    from learned_token_pruning_05_amd import _lib
    args = dict(cu=[0, 5], doc_begin=[0], doc_end=[3], k_doc=[1])
    args.update(bad)
    with pytest.raises(_lib.TokenGateError):
        _lib.tg_kept_counts(args["cu"], args["doc_begin"], args["doc_end"], args["k_doc"])


# Raw calls with NULL / fake pointers: every one must fail validation and
# return before any HIP call, so no device memory is touched.
FAKE = ctypes.c_void_p(0x1000)     # 16-B aligned, never dereferenced
MIS = ctypes.c_void_p(0x1004)      # misaligned


def test_gate_validation(lib):
    L = lib
    E, U = 1, 2
    g = lambda **kw: L.tg_gate_score(*[kw.get(k, v) for k, v in [
        ("x", FAKE), ("dt", 1), ("n", 10), ("d", 2048), ("stride", 2048), ("w1", FAKE), ("b1", None),
        ("w2", FAKE), ("b2", 0.0), ("dh", 256), ("out", FAKE), ("st", None)]])
    assert g(n=-1) == E
    assert g(dt=7) == E
    assert g(d=2047) == E
    assert g(stride=1024) == E
    assert g(b2=float("nan")) == E
    assert g(x=None) == E
    assert g(x=MIS) == E
    assert g(w2=None) == E
    assert g(dh=100) == U
    assert g(d=2056, stride=2056) == U           # bf16 path needs d_model % 64 == 0
    assert g(d=2080, stride=2080) == U
    assert g(stride=1 << 23) == U                # 32-bit per-workgroup offsets
    assert g(dt=0, d=4096, stride=4096) == U     # fp32 path limit
    assert g(n=0) == 0                          # empty: no launch


def test_topk_validation(lib):
    L = lib
    t = lambda **kw: L.tg_topk_select(*[kw.get(k, v) for k, v in [
        ("s", FAKE), ("ns", 1), ("n", 10), ("mx", 10), ("cu", FAKE), ("b", FAKE), ("e", FAKE), ("k", FAKE),
        ("ck", FAKE), ("out", FAKE), ("ws", None), ("wsb", 0), ("st", None)]])
    assert t(ns=-1) == 1
    assert t(n=-5) == 1
    assert t(n=2 ** 31) == 1
    assert t(cu=None) == 1
    assert t(out=None) == 1
    assert t(s=None) == 1
    assert t(mx=11) == 1                         # longer than the whole batch
    assert t(n=2 ** 23, mx=2 ** 23) == 2          # beyond the 4 Mi grid limit
    assert t(n=2 ** 22 + 1, mx=2 ** 22 + 1) == 2  # one token past it
    need = L.tg_topk_workspace_bytes(1, 10, 10)
    assert need > 0
    assert t(ws=None, wsb=need) == 3
    assert t(ws=FAKE, wsb=need - 1) == 3
    assert t(ws=ctypes.c_void_p(0x1010), wsb=need) == 3   # not 256-byte aligned
    assert t(ns=0) == 0


def test_gather_validation(lib):
    L = lib
    t = lambda **kw: L.tg_gather_kept(*[kw.get(k, v) for k, v in [
        ("x", FAKE), ("dt", 1), ("d", 2048), ("stride", 2048), ("s", FAKE), ("ki", FAKE), ("m", 10),
        ("ns", 1), ("cu", FAKE), ("ck", FAKE), ("xk", FAKE), ("sk", FAKE), ("pk", FAKE), ("st", None)]])
    assert t(m=-1) == 1
    assert t(d=12, stride=12) == 1
    assert t(x=MIS) == 1
    assert t(xk=None) == 1
    assert t(s=None) == 1          # scores_kept requested without scores
    assert t(cu=None) == 1         # positions requested without metadata
    assert t(m=0) == 0


def test_attn_validation(lib):
    L = lib
    need = L.tg_attn_workspace_bytes(1, 100, 8, 128)
    assert need > 100 * 8 * 128 * 2 * 2
    a = lambda **kw: L.tg_keybias_attn_prefill(*[kw.get(k, v) for k, v in [
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("qs", 2048), ("kvs", 1024), ("ks", FAKE), ("g", FAKE),
        ("tau", 0.9), ("pos", FAKE), ("ck", FAKE), ("ns", 1), ("m", 100), ("mx", 100), ("hq", 16),
        ("hkv", 8), ("d", 128), ("rb", 1e6), ("out", FAKE), ("lse", None), ("ws", FAKE), ("wsb", need),
        ("st", None)]])
    assert a(tau=0.0) == 1
    assert a(tau=-1.0) == 1
    assert a(tau=float("inf")) == 1
    assert a(rb=float("nan")) == 1
    assert a(hq=12) == 1               # not a multiple of Hkv
    assert a(d=96) == 2                # unsupported head_dim
    assert a(hq=24, qs=3072) == 2      # group size 3
    assert a(qs=1000) == 1             # stride too small
    assert a(kvs=1028) == 1            # stride not a multiple of 8
    assert a(mx=101) == 1              # longer than the total
    assert a(q=None) == 1
    assert a(v=MIS) == 1
    assert a(wsb=need - 1) == 3        # workspace too small
    assert a(ws=ctypes.c_void_p(0x1010)) == 3   # workspace not 256-B aligned
    assert a(m=0) == 0


def test_attn_prepare_forward_validation(lib):
    L = lib
    need = L.tg_attn_workspace_bytes(1, 100, 8, 128)
    p = lambda **kw: L.tg_attn_prepare(*[kw.get(k, v) for k, v in [
        ("k", FAKE), ("v", FAKE), ("kvs", 1024), ("ks", FAKE), ("pos", FAKE), ("ck", FAKE), ("ns", 1),
        ("m", 100), ("hkv", 8), ("d", 128), ("rb", 1e6), ("ws", FAKE), ("wsb", need), ("st", None)]])
    assert p(rb=float("inf")) == 1
    assert p(d=80) == 2
    assert p(kvs=1000) == 1            # below Hkv * D
    assert p(hkv=0) == 1
    assert p(k=None) == 1
    assert p(pos=None) == 1
    assert p(v=MIS) == 1
    assert p(ns=0) == 1                # kept tokens but no sequence
    assert p(wsb=need - 1) == 3
    assert p(m=0) == 0
    f = lambda **kw: L.tg_attn_forward(*[kw.get(k, v) for k, v in [
        ("q", FAKE), ("qs", 2048), ("g", FAKE), ("tau", 0.9), ("ck", FAKE), ("ns", 1), ("m", 100), ("mx", 100),
        ("hq", 16), ("hkv", 8), ("d", 128), ("rb", 1e6), ("out", FAKE), ("lse", None), ("ws", FAKE),
        ("wsb", need), ("st", None)]])
    assert f(tau=0.0) == 1
    assert f(hq=12) == 1
    assert f(hq=24, qs=3072) == 2
    assert f(qs=2040) == 1
    assert f(mx=101) == 1
    assert f(g=None) == 1
    assert f(out=MIS) == 1
    assert f(ws=ctypes.c_void_p(0x1010)) == 3
    assert f(wsb=need - 1) == 3
    assert f(m=0) == 0


def test_attn_decode_validation(lib):
    L = lib
    cache = L.tg_attn_workspace_bytes(1, 100, 8, 128)
    need = L.tg_attn_decode_workspace_bytes(1, 100, 16, 128)
    assert need >= 2 * 16 * 128 * 4 and L.tg_attn_decode_workspace_bytes(1, 100, 16, 96) == 0
    a = lambda **kw: L.tg_attn_decode(*[kw.get(k, v) for k, v in [
        ("q", FAKE), ("qs", 2048), ("qp", FAKE), ("g", FAKE), ("tau", 0.9), ("pos", FAKE), ("ck", FAKE),
        ("ns", 1), ("m", 100), ("mx", 100), ("hq", 16), ("hkv", 8), ("d", 128), ("rb", 1e6), ("cache", FAKE),
        ("cb", cache), ("out", FAKE), ("lse", None), ("ws", FAKE), ("wsb", need), ("st", None)]])
    assert a(tau=0.0) == 1
    assert a(rb=float("nan")) == 1
    assert a(hq=12) == 1               # not a multiple of Hkv
    assert a(d=96) == 2                # unsupported head_dim
    assert a(hq=24, qs=3072) == 2      # group size 3
    assert a(qs=2000) == 1             # stride below Hq * D
    assert a(mx=101) == 1              # longer than the total
    assert a(mx=0) == 1                # kept keys but no length
    assert a(q=None) == 1
    assert a(qp=None) == 1
    assert a(pos=None) == 1
    assert a(cb=cache - 1) == 3        # cache smaller than the prepared layout
    assert a(cache=ctypes.c_void_p(0x1010)) == 3
    assert a(wsb=need - 1) == 3
    assert a(ws=ctypes.c_void_p(0x1010)) == 3
    assert a(ns=0) == 1                # kept keys but no sequence
    assert a(ns=0, m=0, mx=0) == 0     # nothing to do, nothing launched


def test_attn_gate_grads_validation(lib):
    L = lib
    cache = L.tg_attn_workspace_bytes(1, 100, 8, 128)
    need = L.tg_attn_gate_grads_workspace_bytes(1, 100, 100, 16, 128)
    assert need >= 2 * 16 * 100 * (128 + 16) * 2 + 16 * 100 * 4
    assert L.tg_attn_gate_grads_workspace_bytes(1, 100, 100, 16, 96) == 0
    a = lambda **kw: L.tg_attn_gate_grads(*[kw.get(k, v) for k, v in [
        ("q", FAKE), ("qs", 2048), ("v", FAKE), ("kvs", 1024), ("s", FAKE), ("g", FAKE), ("tau", 0.9),
        ("ck", FAKE), ("ns", 1), ("m", 100), ("mx", 100), ("hq", 16), ("hkv", 8), ("d", 128), ("rb", 1e6),
        ("out", FAKE), ("lse", FAKE), ("do", FAKE), ("dos", 2048), ("cache", FAKE), ("cb", cache),
        ("dsc", FAKE), ("dg", FAKE), ("dt", FAKE), ("ws", FAKE), ("wsb", need), ("st", None)]])
    assert a(tau=0.0) == 1
    assert a(tau=float("inf")) == 1
    assert a(rb=float("nan")) == 1
    assert a(hq=12) == 1               # not a multiple of Hkv
    assert a(d=96) == 2                # unsupported head_dim
    assert a(hq=24, qs=3072, dos=3072) == 2   # group size 3
    assert a(qs=2000) == 1             # stride below Hq * D
    assert a(kvs=1000) == 1
    assert a(dos=2040) == 1
    assert a(dos=2052) == 1            # not a multiple of 8
    assert a(mx=101) == 1              # longer than the total
    assert a(mx=0) == 1                # kept keys but no length
    for name in ("q", "v", "s", "g", "ck", "out", "lse", "do", "dsc", "dg", "dt"):
        assert a(**{name: None}) == 1, name
    assert a(q=ctypes.c_void_p(0x1008)) == 1   # not 16-B aligned
    assert a(do=ctypes.c_void_p(0x1008)) == 1
    assert a(cb=cache - 1) == 3        # cache smaller than the prepared layout
    assert a(cache=ctypes.c_void_p(0x1010)) == 3
    assert a(wsb=need - 1) == 3
    assert a(ws=ctypes.c_void_p(0x1010)) == 3
    assert a(m=0, mx=0, dg=None) == 1  # the zero gradients still need somewhere to go
    assert a(ns=0) == 1                # kept tokens but no sequence


def test_random_k_validation(lib):
    L = lib
    need = L.tg_random_k_workspace_bytes(2, 1000, 600)
    assert need >= 1000 * 4 + L.tg_topk_workspace_bytes(2, 1000, 600)
    a = lambda **kw: L.tg_random_k_select(*[kw.get(k, v) for k, v in [
        ("seed", 5), ("ns", 2), ("n", 1000), ("mx", 600), ("cu", FAKE), ("db", FAKE), ("de", FAKE), ("kd", FAKE),
        ("ck", FAKE), ("out", FAKE), ("ws", FAKE), ("wsb", need), ("st", None)]])
    assert a(n=-1) == 1
    assert a(mx=1001) == 1            # longer than the total
    assert a(cu=None) == 1
    assert a(out=None) == 1
    assert a(wsb=need - 1) == 3
    assert a(ws=ctypes.c_void_p(0x1010)) == 3
    assert a(ns=0) == 0
    assert a(n=0, mx=0) == 0


def test_library_has_no_undefined_internal_symbols(lib):
    """Every kernel stub must be defined: an undefined tg:: symbol only shows
    up when the library is loaded for real."""
    import subprocess
    from learned_token_pruning_05_amd import _lib
    out = subprocess.run(["nm", "-D", _lib.LIB_PATH], capture_output=True, text=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "_ZN2tg" in l]
    assert not undefined, undefined[:3]


def test_random_budgets_host_bit_exact(lib):
    """tg_random_budgets (host code) against oracle.random_budgets, bit-exact, for
    seeds up to 2^64 - 1 and spans up to 2^31 - 2; and its validation."""
    import oracle
    from learned_token_pruning_05_amd import _lib
    db = np.array([0, 5, 0, 3, 0, 100, 7], dtype=np.int32)
    de = np.array([9, 5, 1, 40003, 2 ** 31 - 2, 130916, 8], dtype=np.int32)
    for seed in (0, 1, 12345, 2 ** 63, 2 ** 64 - 1):
        np.testing.assert_array_equal(_lib.tg_random_budgets(seed, db, de), oracle.random_budgets(seed, db, de))
    assert lib.tg_random_budgets(1, -1, None, None, None) == 1
    bad = np.array([5], dtype=np.int32)
    good = np.array([4], dtype=np.int32)
    out = np.zeros(1, dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.tg_random_budgets(1, 1, p(bad), p(good), p(out)) == 1   # end before begin
    assert lib.tg_random_budgets(1, 1, p(good), p(bad), None) == 1
    assert lib.tg_random_budgets(1, 0, None, None, None) == 0


def test_gated_select_validation(lib):
    """The fused front-half call validates all three stages before launching: an
    error in any stage's arguments returns that stage's status."""
    L = lib
    need = L.tg_topk_workspace_bytes(1, 4096, 4096)
    a = lambda **kw: L.tg_gated_select(*[kw.get(k, v) for k, v in [
        ("x", FAKE), ("dt", 1), ("n", 4096), ("d", 2048), ("xs", 2048), ("w1", FAKE), ("b1", None), ("w2", FAKE),
        ("b2", 0.0), ("dh", 256), ("ns", 1), ("mx", 4096), ("cu", FAKE), ("db", FAKE), ("de", FAKE), ("kd", FAKE),
        ("ck", FAKE), ("m", 1000), ("sc", FAKE), ("ki", FAKE), ("xk", FAKE), ("sk", FAKE), ("pk", FAKE),
        ("ws", FAKE), ("wsb", need), ("st", None)]])
    assert a(d=100) == 1                  # gate: d_model not a multiple of 8
    assert a(dh=100) == 2                 # gate: unsupported hidden width
    assert a(b2=float("nan")) == 1
    assert a(mx=4097) == 1                # top-K: longer than the total
    assert a(kd=None) == 1
    assert a(wsb=need - 1) == 3           # top-K workspace
    assert a(xk=None) == 1                # gather output
    assert a(xk=ctypes.c_void_p(0x1008)) == 1
    assert a(m=-1) == 1
    assert a(n=0, mx=0, m=0) == 0         # nothing to do, nothing launched


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so,
    before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_binding_rejects_bad_tensors(lib):
    """The Python binding checks device, dtype, rank and size of every tensor
    argument before the C call, so a host tensor, a wrong dtype or a short
    buffer raises instead of reaching a kernel as a bad pointer.  (CPU tensors
    only: every call here is refused before any GPU work.)"""
    import torch
    from learned_token_pruning_05_amd import _lib as tg
    x = torch.zeros(8, 64, dtype=torch.bfloat16)
    w1 = torch.zeros(64, 64, dtype=torch.bfloat16)
    w2 = torch.zeros(64)
    with pytest.raises(ValueError, match="GPU device"):
        tg.tg_gate_score(x, w1, None, w2, 0.0)
    with pytest.raises(TypeError, match="must be a torch tensor"):
        tg.tg_gate_score(np.zeros((8, 64), np.float32), w1, None, w2, 0.0)
    i32 = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU device"):
        tg.tg_topk_select(torch.zeros(8), i32, i32[:1], i32[:1], i32[:1], i32, 2, 8)
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU device"):
        tg.tg_keybias_attn_prefill(q, q, q, torch.zeros(4), torch.ones(2), 0.9, torch.zeros(4, dtype=torch.int32),
                                   i32, 4)
    with pytest.raises(TypeError):
        tg.tg_attn_prepare(q.float(), q.float(), torch.zeros(4), torch.zeros(4, dtype=torch.int32), i32)
    with pytest.raises(ValueError, match="GPU device"):
        tg.tg_attn_gate_grads(q, q, torch.zeros(4), torch.ones(2), 0.9, i32, 4, q, torch.zeros(2, 4), q,
                              torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU device"):
        tg.tg_gather_kept(x, None, torch.zeros(2, dtype=torch.int32), i32, i32)



def test_binding_check_rules():
    """_req, the binding's per-tensor check: dtype and rank are checked first,
    then the device, then size and contiguity (host tensors; no GPU needed)."""
    import torch
    from learned_token_pruning_05_amd import _lib as tg
    t = torch.zeros(4, 8)
    with pytest.raises(TypeError, match="torch.int32"):
        tg._req(t, "t", torch.int32)
    with pytest.raises(ValueError, match="dimensions"):
        tg._req(t, "t", torch.float32, dim=1)
    with pytest.raises(ValueError, match="GPU device"):
        tg._req(t, "t", torch.float32, dim=2)
    tg._req(None, "t", optional=True)
    with pytest.raises(ValueError, match="required"):
        tg._req(None, "t")
