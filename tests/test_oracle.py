"""Pins for the CPU oracle against things other than itself: library routines
(torch fp64 linear/silu/SDPA), hand-worked fixtures, closed forms, brute force
and invariants.  No GPU."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(v):
    return float(v) if not isinstance(v, str) else float(v.replace("nan", "nan"))


# ---------------------------------------------------------------- gate ----
def test_gate_matches_torch_linear_silu():
    r = np.random.default_rng(11)
    x = r.standard_normal((37, 24))
    w1 = r.standard_normal((10, 24)) * 0.3
    b1 = r.standard_normal(10)
    w2 = r.standard_normal(10)
    b2 = 0.37
    got = oracle.gate_score(x, w1, b1, w2, b2, chunk_rows=8)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    ref = F.linear(F.silu(F.linear(t(x), t(w1), t(b1))), t(w2)[None, :]).squeeze(1) + b2
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_gate_matches_scalar_loop():
    """The gate written out token by token and unit by unit in plain Python
    floats (math.exp, no arrays): s = b2 + sum_n w2_n a_n / (1 + exp(-a_n)),
    a_n = b1_n + sum_k W1_nk x_k."""
    r = np.random.default_rng(13)
    x = r.standard_normal((9, 7))
    w1 = r.standard_normal((5, 7)) * 0.4
    b1 = r.standard_normal(5) * 0.2
    w2 = r.standard_normal(5)
    b2 = -0.3
    ref = []
    for t in range(x.shape[0]):
        acc = b2
        for n in range(w1.shape[0]):
            a = float(b1[n])
            for kk in range(x.shape[1]):
                a += float(w1[n, kk]) * float(x[t, kk])
            acc += float(w2[n]) * a / (1.0 + math.exp(-a))
        ref.append(acc)
    np.testing.assert_allclose(oracle.gate_score(x, w1, b1, w2, b2), ref, rtol=1e-13, atol=1e-14)


def test_gate_closed_forms():
    r = np.random.default_rng(12)
    w1 = r.standard_normal((6, 5))
    b1 = np.array([0.0, 1.0, -1.0, 2.0, -3.0, 0.5])
    w2 = r.standard_normal(6)
    # x = 0 -> s = w2 . SiLU(b1) + b2, with sigmoid(1) = 0.7310585786300049 (table value)
    s = oracle.gate_score(np.zeros((3, 5)), w1, b1, w2, -0.25)
    sig = {0.0: 0.5, 1.0: 0.7310585786300049, -1.0: 0.2689414213699951,
           2.0: 0.8807970779778823, -3.0: 0.04742587317756678, 0.5: 0.6224593312018546}
    want = sum(w2[i] * b1[i] * sig[b1[i]] for i in range(6)) - 0.25
    np.testing.assert_allclose(s, want, rtol=1e-14)
    # W1 = 0 and b1 = 0 -> SiLU(0) = 0 -> s = b2 exactly
    s0 = oracle.gate_score(r.standard_normal((4, 5)), np.zeros((6, 5)), None, w2, 1.5)
    assert np.all(s0 == 1.5)


def test_silu_limits():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    assert np.isfinite(oracle.silu(np.array([-1000.0]))).all()


def test_gate_workload_shapes():
    w = workloads.tiny()
    g = w.gate_inputs()
    s = oracle.gate_score(g["x_f"], g["w1_f"], g["b1_f"], g["w2_f"], g["b2"])
    assert s.shape == (512,) and np.isfinite(s).all()
    assert s.std() > 1e-3


# --------------------------------------------------------------- top-K ----
def _brute_keep(scores, k):
    """Python sorted() on (nan flag, -score, index): the selection rule read
    from the pages plus the tie / special-value readings."""
    n = len(scores)
    keyf = lambda i: (1, 0.0, i) if math.isnan(scores[i]) else (0, -scores[i], i)
    return sorted(sorted(range(n), key=keyf)[:min(k, n)])


def _beats(a, sa, b, sb):
    """Pairwise: does token a rank strictly before token b?"""
    if math.isnan(sa) or math.isnan(sb):
        if math.isnan(sa) and math.isnan(sb):
            return a < b
        return math.isnan(sb)
    if sa != sb:
        return sa > sb
    return a < b


def test_topk_golden_hand_example():
    g = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    s = np.array([float(v) for v in g["scores"]], dtype=np.float32)
    for c in g["cases"]:
        kept, cu = oracle.topk_select(s, [0, 8], [g["doc_begin"]], [g["doc_end"]], [c["k_doc"]])
        assert kept.tolist() == c["kept"], c


def test_topk_exhaustive_tiny():
    vals = [-math.inf, -1.0, -0.0, 0.0, 1.0, math.nan]
    for n in range(1, 6):
        for combo in itertools.product(vals, repeat=n):
            s = np.array(combo, dtype=np.float32)
            for k in range(0, n + 2):
                kept, _ = oracle.topk_select(s, [0, n], [0], [n], [k])
                assert kept.tolist() == _brute_keep(list(combo), k), (combo, k)


def test_topk_random_against_pairwise_dominance():
    r = np.random.default_rng(3)
    for trial in range(300):
        n = int(r.integers(1, 40))
        q = int(r.integers(0, n + 1))
        nd = n - q
        pool = np.array([-2.0, -1.0, 0.0, -0.0, 1.0, 3.0, np.inf, -np.inf, np.nan], dtype=np.float32)
        s = np.where(r.random(n) < 0.5, r.choice(pool, n), r.standard_normal(n)).astype(np.float32)
        k = int(r.integers(0, nd + 3))
        kept, cu = oracle.topk_select(s, [0, n], [0], [nd], [k])
        kept = kept.tolist()
        assert kept == sorted(kept)
        assert len(kept) == min(k, nd) + q == cu[-1]
        assert set(range(nd, n)) <= set(kept)          # question always kept
        kd = [i for i in kept if i < nd]
        pr = [i for i in range(nd) if i not in kept]
        for a in kd:                                   # every kept doc token beats every pruned one
            for b in pr:
                assert _beats(a, float(s[a]), b, float(s[b]))
        # idempotence: reselecting the kept document tokens with the same budget keeps all
        sub = s[kd]
        k2, _ = oracle.topk_select(sub, [0, len(kd)], [0], [len(kd)], [min(k, nd)])
        assert k2.tolist() == list(range(len(kd)))


def test_topk_doc_span_in_middle_and_varlen():
    r = np.random.default_rng(5)
    lens, spans, ks = [9, 1, 14, 0, 6], [(2, 7), (0, 1), (3, 10), (0, 0), (0, 6)], [2, 0, 100, 4, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    s = r.standard_normal(cu[-1]).astype(np.float32)
    kept, ck = oracle.topk_select(s, cu, [a for a, _ in spans], [b for _, b in spans], ks)
    parts = []
    for i, n in enumerate(lens):
        a, b = spans[i]
        local = _brute_keep([float(v) for v in s[cu[i] + a:cu[i] + b]], ks[i])
        keep = sorted([a + j for j in local] + list(range(0, a)) + list(range(b, n)))
        parts += [cu[i] + j for j in keep]
        assert ck[i + 1] - ck[i] == len(keep)
    assert kept.tolist() == parts


def test_topk_rejects_bad_metadata():
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros(4, np.float32), [0, 4], [0], [5], [1])
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros(4, np.float32), [0, 4], [0], [4], [-1])


def test_topk_planted_ties_cut_inside_group():
    w = workloads.custom([3000, 2000], [100, 50], [240, 160], tie_frac=0.05)
    s = w.topk_scores()
    kept, ck = oracle.topk_select(s, w.cu_seqlens, w.doc_begin, w.doc_end, w.k_doc)
    for i in range(2):
        a, nd = int(w.cu_seqlens[i]), int(w.doc_end[i])
        doc = s[a:a + nd]
        vals, cnt = np.unique(doc, return_counts=True)
        t = vals[np.argmax(cnt)]
        kd = kept[(kept >= a) & (kept < a + nd)] - a
        tied_kept = np.sort(kd[doc[kd] == t])
        tied_all = np.nonzero(doc == t)[0]
        assert 0 < tied_kept.size < tied_all.size          # the cut falls inside the tie group
        assert (tied_kept == tied_all[:tied_kept.size]).all()  # lowest indices win


# -------------------------------------------------------------- gather ----
def test_gather_definition():
    r = np.random.default_rng(8)
    cu = np.array([0, 5, 12])
    x = r.standard_normal((12, 3))
    s = r.standard_normal(12).astype(np.float32)
    kept = np.array([1, 3, 4, 5, 6, 11])
    ck = np.array([0, 3, 6])
    xk, sk, pk = oracle.gather_kept(x, s, kept, cu, ck)
    assert (xk == x[kept]).all() and (sk == s[kept]).all()
    assert pk.tolist() == [1, 3, 4, 0, 1, 6]


# ---------------------------------------------------------------- RoPE ----
def _rope_complex(x, pos, base):
    """Independent form: channels (m, m + D/2) as one complex number times e^{i pos w_m}."""
    d = x.shape[-1]
    h = d // 2
    w = np.array([base ** (-(2.0 * m) / d) for m in range(h)])
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_golden_and_complex_form():
    g = json.load(open(os.path.join(GOLD, "rope_hand.json")))
    got = oracle.rope(np.array(g["x"])[None, None, :], np.array([g["pos"]]), g["base"])[0, 0]
    np.testing.assert_allclose(got, g["out"], rtol=0, atol=1e-15)
    r = np.random.default_rng(9)
    x = r.standard_normal((20, 3, 16))
    pos = r.integers(0, 200000, 20)
    np.testing.assert_allclose(oracle.rope(x, pos, 1e6), _rope_complex(x, pos, 1e6), atol=1e-12)


def test_rope_invariants():
    r = np.random.default_rng(10)
    q = r.standard_normal((1, 1, 64))
    k = r.standard_normal((1, 1, 64))
    np.testing.assert_array_equal(oracle.rope(q, [0], 1e6), q)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, [12345], 1e6)), np.linalg.norm(q), rtol=1e-14)
    dot = lambda p1, p2: float((oracle.rope(q, [p1], 1e6) * oracle.rope(k, [p2], 1e6)).sum())
    assert abs(dot(100, 40) - dot(100 + 777, 40 + 777)) < 1e-10


# ----------------------------------------------------------- attention ----
def _sdpa_ref(q, k, v, pos, gain, tau, s, base, keep_mask=None):
    """torch fp64 SDPA with a float mask: g_h * s_j on kept keys, -inf on pruned
    keys and on keys at later positions; K/V repeated per q head."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    if base:
        q, k = _rope_complex(q, pos, base), _rope_complex(k, pos, base)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    qt = t(q).permute(1, 0, 2)
    kt = t(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    vt = t(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    pos = np.asarray(pos)
    allowed = pos[None, :] <= pos[:, None]
    if keep_mask is not None:
        allowed = allowed & keep_mask[None, :]
    mask = torch.full((hq, n, n), -math.inf, dtype=torch.float64)
    bias = t(np.asarray(gain, dtype=np.float64)[:, None] * np.asarray(s, dtype=np.float64)[None, :])
    al = torch.from_numpy(allowed)
    for h in range(hq):
        mask[h][al] = bias[h][None, :].expand(n, n)[al]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=1.0 / (math.sqrt(d) * tau))
    return o.permute(1, 0, 2).numpy()


def test_attention_golden_two_tokens():
    g = json.load(open(os.path.join(GOLD, "attn_two_tokens.json")))
    a = lambda key: np.array(g[key], dtype=np.float64)[:, None, :]
    out, lse = oracle.keybias_attention(a("q"), a("k"), a("v"), np.array(g["s"]), np.array([g["gain"]]),
                                        g["tau"], np.array([0, 1]), [0, 2], rope_base=0)
    np.testing.assert_allclose(out[:, 0, :], g["out"], atol=1e-15)
    np.testing.assert_allclose(lse[0], g["lse"], atol=1e-15)


def test_attention_reduces_to_causal_sdpa():
    """g = 0, tau = 1, nothing pruned: plain causal GQA attention (is_causal SDPA)."""
    r = np.random.default_rng(21)
    n, hq, hkv, d = 37, 4, 2, 16
    q, k, v = (r.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    out, _ = oracle.keybias_attention(q, k, v, r.standard_normal(n), np.zeros(hq), 1.0,
                                      np.arange(n), [0, n], rope_base=0)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(t(q), t(k).repeat_interleave(2, 0), t(v).repeat_interleave(2, 0),
                                         is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("base", [0.0, 1e6, 100.0])
def test_attention_pruning_equals_masking(base):
    """Key-bias attention on the compacted set == full-length attention with
    pruned keys masked out, at the kept query rows (pins gather, positions,
    RoPE on original positions, causality, bias sign, per-head gain, tau)."""
    r = np.random.default_rng(22)
    n, hq, hkv, d = 60, 6, 2, 8
    q, k, v = (r.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(n).astype(np.float32)
    gain = r.uniform(0.5, 2, hq)
    tau = 0.83
    kept, ck = oracle.topk_select(s, [0, n], [0], [48], [17])
    qk, sk, pk = oracle.gather_kept(q, s, kept, [0, n], ck)
    kk = k[kept]
    vk = v[kept]
    out, _ = oracle.keybias_attention(qk, kk, vk, sk, gain, tau, pk, ck, rope_base=base)
    keep = np.zeros(n, dtype=bool)
    keep[kept] = True
    ref = _sdpa_ref(q, k, v, np.arange(n), gain, tau, s, base, keep_mask=keep)
    np.testing.assert_allclose(out, ref[kept], atol=1e-11)


def test_attention_shift_invariance_and_tau_placement():
    r = np.random.default_rng(23)
    n, hq, hkv, d = 30, 2, 1, 8
    q, k, v = (r.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(n)
    g = np.array([0.7, 1.9])
    pos = np.sort(r.choice(1000, n, replace=False))
    o1, l1 = oracle.keybias_attention(q, k, v, s, g, 0.9, pos, [0, n])
    o2, l2 = oracle.keybias_attention(q, k, v, s + 3.25, g, 0.9, pos, [0, n])
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, (g * 3.25)[:, None] * np.ones((1, n)), atol=1e-12)
    o3, _ = oracle.keybias_attention(q / 0.9, k, v, s, g, 1.0, pos, [0, n])
    np.testing.assert_allclose(o1, o3, atol=1e-12)


def test_attention_gqa_and_varlen():
    r = np.random.default_rng(24)
    lens = [5, 1, 13, 8]
    ck = np.concatenate([[0], np.cumsum(lens)])
    m, hq, hkv, d = ck[-1], 8, 2, 16
    q, k, v = (r.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(m)
    g = r.uniform(0.5, 2, hq)
    pos = np.concatenate([np.sort(r.choice(50, L, replace=False)) for L in lens])
    out, lse = oracle.keybias_attention(q, k, v, s, g, 0.95, pos, ck)
    # GQA == MHA with repeat-interleaved K/V
    o_mha, _ = oracle.keybias_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), s, g, 0.95, pos, ck)
    np.testing.assert_allclose(out, o_mha, atol=1e-12)
    # varlen == concatenation of per-sequence calls
    for i in range(len(lens)):
        a, b = ck[i], ck[i + 1]
        oi, li = oracle.keybias_attention(q[a:b], k[a:b], v[a:b], s[a:b], g, 0.95, pos[a:b], [0, b - a])
        np.testing.assert_allclose(out[a:b], oi, atol=1e-12)
        np.testing.assert_allclose(lse[:, a:b], li, atol=1e-12)


def test_attention_closed_forms_and_lse():
    r = np.random.default_rng(25)
    n, d = 12, 8
    k = r.standard_normal((n, 1, d))
    v = r.standard_normal((n, 1, d))
    q = r.standard_normal((n, 1, d))
    s = r.standard_normal(n)
    out, lse = oracle.keybias_attention(q, k, v, s, np.array([1.3]), 0.8, np.arange(n), [0, n])
    np.testing.assert_allclose(out[0, 0], v[0, 0], atol=1e-14)            # row 0 sees only itself
    o0, _ = oracle.keybias_attention(np.zeros_like(q), k, v, s, np.array([0.0]), 1.0, np.arange(n), [0, n])
    means = np.cumsum(v[:, 0], axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o0[:, 0], means, atol=1e-13)              # uniform weights
    qr, kr = _rope_complex(q, np.arange(n), 1e6), _rope_complex(k, np.arange(n), 1e6)
    logits = torch.from_numpy((qr[:, 0] @ kr[:, 0].T) / (math.sqrt(d) * 0.8) + 1.3 * s[None, :])
    logits = logits.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse[0], torch.logsumexp(logits, 1).numpy(), atol=1e-12)


def test_attention_rows_subset():
    r = np.random.default_rng(26)
    n, hq, hkv, d = 40, 2, 1, 8
    q, k, v = (r.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(n)
    full, _ = oracle.keybias_attention(q, k, v, s, np.ones(hq), 1.0, np.arange(n), [0, n])
    part, _ = oracle.keybias_attention(q, k, v, s, np.ones(hq), 1.0, np.arange(n), [0, n], rows=[0, 7, 39])
    np.testing.assert_array_equal(part[[0, 7, 39]], full[[0, 7, 39]])
    assert np.isnan(part[1]).all()


def test_attention_rejects_bad_params():
    z = np.zeros((2, 2, 4))
    with pytest.raises(ValueError):
        oracle.keybias_attention(z, z[:, :1], z[:, :1], np.zeros(2), np.ones(2), 0.0, [0, 1], [0, 2])
    with pytest.raises(ValueError):
        oracle.keybias_attention(np.zeros((2, 3, 4)), z, z, np.zeros(2), np.ones(3), 1.0, [0, 1], [0, 2])


# ------------------------------------------------------------------ decode ----
def _decode_case(seed, lens, hq, hkv, d):
    r = np.random.default_rng(seed)
    ck = np.concatenate([[0], np.cumsum(lens)])
    m = int(ck[-1])
    q, k, v = (r.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(m)
    g = r.uniform(0.5, 2, hq)
    pos = np.concatenate([np.sort(r.choice(4000, L, replace=False)) for L in lens])
    return q, k, v, s, g, pos, ck


@pytest.mark.parametrize("base", [0.0, 1e6])
def test_decode_equals_prefill_row(base):
    """A query placed at a kept token's position, with that token's q, sees the
    same keys as that token's prefill row (keys after it masked), so decode ==
    the prefill oracle's row: pins the position mask, RoPE at the query
    position, bias, gain, tau and GQA against the independently pinned prefill."""
    q, k, v, s, g, pos, ck = _decode_case(31, [9, 1, 17, 6], 8, 2, 16)
    full_o, full_l = oracle.keybias_attention(q, k, v, s, g, 0.87, pos, ck, rope_base=base)
    r = np.random.default_rng(5)
    for trial in range(3):
        rows = np.array([r.integers(ck[i], ck[i + 1]) if trial else ck[i + 1] - 1 for i in range(len(ck) - 1)])
        o, l = oracle.keybias_decode(q[rows], pos[rows], k, v, s, g, 0.87, pos, ck, rope_base=base)
        np.testing.assert_allclose(o, full_o[rows], atol=1e-12)
        np.testing.assert_allclose(l, full_l[:, rows], atol=1e-12)


def test_decode_closed_forms_and_empty():
    q, k, v, s, g, pos, ck = _decode_case(32, [7, 12], 2, 1, 8)
    qp = np.array([pos[ck[1] - 1] + 50, pos[ck[1] + 4]])      # all of seq 0; first 5 keys of seq 1
    o, l = oracle.keybias_decode(np.zeros((2, 2, 8)), qp, k, v, s, np.zeros(2), 1.0, pos, ck)
    np.testing.assert_allclose(o[0, :, :], np.broadcast_to(v[0:7, 0].mean(0), (2, 8)), atol=1e-14)
    np.testing.assert_allclose(o[1, :, :], np.broadcast_to(v[7:12, 0].mean(0), (2, 8)), atol=1e-14)
    np.testing.assert_allclose(l, np.log([[7, 5], [7, 5]]), atol=1e-14)
    # a query before every key sees nothing: O = 0, LSE = -inf
    o, l = oracle.keybias_decode(q[[0, 7]], np.array([pos[0] - 1, pos[7] - 1]), k, v, s, g, 1.0, pos, ck)
    assert not o.any() and np.all(l == -np.inf)


def test_decode_shift_invariance():
    q, k, v, s, g, pos, ck = _decode_case(33, [11, 4], 4, 2, 8)
    qp = pos[[10, 14]] + 3
    o1, l1 = oracle.keybias_decode(q[[3, 12]], qp, k, v, s, g, 0.9, pos, ck)
    o2, l2 = oracle.keybias_decode(q[[3, 12]], qp, k, v, s - 1.5, g, 0.9, pos, ck)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1 - l2, (g * 1.5)[:, None] * np.ones((1, 2)), atol=1e-12)


# -------------------------------------------------------------- random-K ----
def test_splitmix64_reference_outputs():
    """SplitMix64 seeded with 0 (Steele, Lea and Flood 2014; Vigna's reference
    implementation) starts 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4, 0x06c45d188009454f."""
    got = oracle.splitmix64(0, 3)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # counter-based: output i of seed s is output 0 of seed s + i * increment
    g = 0x9E3779B97F4A7C15
    a = oracle.splitmix64(12345, 6)
    for i in range(6):
        assert int(oracle.splitmix64((12345 + i * g) % 2 ** 64, 1)[0]) == int(a[i])


def test_random_scores_encode_30_bit_draws_in_order():
    """Each score is a positive normal float whose bit pattern is 2^23 plus the
    top 30 bits of the pinned SplitMix64 output, so the scores sort exactly
    like those draws (checked on values, not on the encoding)."""
    s = oracle.random_scores(7, 5000)
    raw = oracle.splitmix64(7, 5000) >> np.uint64(34)
    assert s.dtype == np.float32 and np.all(np.isfinite(s))
    assert np.all(s >= np.float32(2.0 ** -126)) and np.all(s < np.float32(4.0))
    np.testing.assert_array_equal(s.view(np.uint32).astype(np.uint64) - (1 << 23), raw)
    np.testing.assert_array_equal(np.argsort(s.astype(np.float64), kind="stable"), np.argsort(raw, kind="stable"))
    # the draws' leading bits stay in the encoding's leading bits: the top 11
    # bits of 5000 encoded scores take hundreds of distinct values
    assert len(np.unique(s.view(np.uint32) >> 21)) > 400


def test_random_k_budget_question_and_determinism():
    cu = [0, 300, 350, 1000]
    db, de, kd = [0, 0, 0], [280, 50, 600], [40, 60, 0]     # budgets: partial, above n_doc, zero
    kept, ck = oracle.random_k_select(9, cu, db, de, kd)
    np.testing.assert_array_equal(ck, oracle.kept_counts(cu, db, de, kd))
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        ks = kept[ck[i]:ck[i + 1]] - a
        assert np.all(np.diff(ks) > 0)
        assert set(range(de[i], b - a)) <= set(ks.tolist())          # question always kept
        assert np.sum(ks < de[i]) == min(kd[i], de[i] - db[i])
    k2, _ = oracle.random_k_select(9, cu, db, de, kd)
    np.testing.assert_array_equal(kept, k2)
    k3, _ = oracle.random_k_select(10, cu, db, de, kd)
    assert not np.array_equal(kept, k3)


def test_random_k_uniform_over_seeds():
    """Each document token is kept with frequency K / n_doc over seeds (binomial
    bound at ~5 sigma per token), and pairs of tokens are not correlated."""
    n_doc, k, seeds = 40, 10, 2000
    cnt = np.zeros(n_doc)
    pair = 0
    for sd in range(seeds):
        kept, _ = oracle.random_k_select(sd, [0, n_doc + 4], [0], [n_doc], [k])
        doc = kept[kept < n_doc]
        cnt[doc] += 1
        pair += (0 in doc) and (1 in doc)
    p = k / n_doc
    assert np.all(np.abs(cnt / seeds - p) <= 5 * np.sqrt(p * (1 - p) / seeds))
    pp = k * (k - 1) / (n_doc * (n_doc - 1))                        # without-replacement pair rate
    assert abs(pair / seeds - pp) <= 5 * np.sqrt(pp * (1 - pp) / seeds)


# ------------------------------------------------------- gate-side gradients ----
def _grad_case(seed, lens, hq, hkv, d):
    r = np.random.default_rng(seed)
    ck = np.concatenate([[0], np.cumsum(lens)])
    m = int(ck[-1])
    q, k, v = (r.standard_normal((m, h, d)) for h in (hq, hkv, hkv))
    s = r.standard_normal(m)
    g = r.uniform(0.5, 2, hq)
    pos = np.concatenate([np.sort(r.choice(300, L, replace=False)) for L in lens])
    d_out = r.standard_normal((m, hq, d))
    return q, k, v, s, g, pos, ck, d_out


@pytest.mark.parametrize("base", [0.0, 1e6])
def test_gate_grads_match_finite_differences(base):
    """Central differences of L = sum(dO * O) from the (independently pinned)
    forward oracle, for every s_j, every g_h and tau."""
    q, k, v, s, g, pos, ck, d_out = _grad_case(51, [6, 1, 9], 4, 2, 8)
    tau = 0.9
    loss = lambda s_, g_, t_: float((d_out * oracle.keybias_attention(q, k, v, s_, g_, t_, pos, ck,
                                                                      rope_base=base)[0]).sum())
    ds, dg, dtau = oracle.keybias_attention_gate_grads(q, k, v, s, g, tau, pos, ck, d_out, rope_base=base)
    h = 1e-5
    fd_s = np.array([(loss(s + h * e, g, tau) - loss(s - h * e, g, tau)) / (2 * h) for e in np.eye(len(s))])
    fd_g = np.array([(loss(s, g + h * e, tau) - loss(s, g - h * e, tau)) / (2 * h) for e in np.eye(len(g))])
    fd_t = (loss(s, g, tau + h) - loss(s, g, tau - h)) / (2 * h)
    np.testing.assert_allclose(ds, fd_s, atol=1e-7)
    np.testing.assert_allclose(dg, fd_g, atol=1e-7)
    assert abs(dtau - fd_t) <= 1e-7


def test_gate_grads_closed_forms():
    q, k, v, s, g, pos, ck, d_out = _grad_case(52, [10, 7], 4, 1, 16)
    ds, dg, dtau = oracle.keybias_attention_gate_grads(q, k, v, s, g, 0.8, pos, ck, d_out)
    # softmax rows sum to one: sum_j dS_ij = 0, so the scores' gradient sums to zero per sequence
    for i in range(len(ck) - 1):
        assert abs(ds[ck[i]:ck[i + 1]].sum()) <= 1e-10
    # no gain: the loss does not see the scores
    ds0, _, _ = oracle.keybias_attention_gate_grads(q, k, v, s, np.zeros(4), 0.8, pos, ck, d_out)
    assert np.abs(ds0).max() == 0.0
    # (q, tau) -> (c q, c tau) leaves the forward unchanged, so c dL/dtau(c q, c tau) = dL/dtau(q, tau)
    _, _, dt2 = oracle.keybias_attention_gate_grads(2.0 * q, k, v, s, g, 1.6, pos, ck, d_out)
    assert abs(2.0 * dt2 - dtau) <= 1e-10 * max(1.0, abs(dtau))


def test_gate_grad_scales_bound_and_closed_form():
    """The condition scales bound the gradients (triangle inequality) and have a
    closed form for one-key sequences: P = 1, Delta = dP, so dS = 0 while each
    scale term is 2 |<dO, v>| times |g_h|, |s_j| or |<q, k>| / (sqrt(D) tau^2)
    (rotation at one shared position keeps the inner product)."""
    q, k, v, s, g, pos, ck, d_out = _grad_case(53, [9, 5, 12], 4, 2, 8)
    tau = 0.85
    ds, dg, dtau, (ms, mg, mt) = oracle.keybias_attention_gate_grads(q, k, v, s, g, tau, pos, ck, d_out,
                                                                     scales=True)
    assert np.all(np.abs(ds) <= ms + 1e-12) and np.all(np.abs(dg) <= mg + 1e-12) and abs(dtau) <= mt + 1e-12
    assert np.all(ms > 0) and np.all(mg > 0) and mt > 0
    r = oracle.keybias_attention_gate_grads(q, k, v, s, g, tau, pos, ck, 3.0 * d_out, scales=True)
    np.testing.assert_allclose(r[3][0], 3.0 * ms, rtol=1e-12)
    # one key per sequence
    q1, k1, v1, s1, g1, _, _, do1 = _grad_case(54, [1, 1, 1], 4, 2, 8)
    pos1 = np.array([5, 0, 299])
    ck1 = np.arange(4)
    ds1, dg1, dt1, (ms1, mg1, mt1) = oracle.keybias_attention_gate_grads(q1, k1, v1, s1, g1, tau, pos1, ck1, do1,
                                                                         scales=True)
    assert np.abs(ds1).max() <= 1e-12 and np.abs(dg1).max() <= 1e-12 and abs(dt1) <= 1e-12
    dp = np.stack([[do1[j, h] @ v1[j, h // 2] for h in range(4)] for j in range(3)])      # [key, head]
    qk = np.stack([[q1[j, h] @ k1[j, h // 2] for h in range(4)] for j in range(3)])
    np.testing.assert_allclose(ms1, (2 * np.abs(dp) * np.abs(g1)[None, :]).sum(1), rtol=1e-12)
    np.testing.assert_allclose(mg1, (2 * np.abs(dp) * np.abs(s1)[:, None]).sum(0), rtol=1e-12)
    np.testing.assert_allclose(mt1, (2 * np.abs(dp) * np.abs(qk)).sum() / (np.sqrt(8) * tau ** 2), rtol=1e-10)


def test_gate_grads_at_stored_forward_reduces_and_scales():
    """At the exact forward outputs the stored-forward backward is the
    finite-difference-pinned gradient; a constant c added to one head's lse
    scales every term of that head by exp(-c) (P = exp(l - lse)), and the other
    heads' terms are untouched."""
    q, k, v, s, g, pos, ck, d_out = _grad_case(55, [11, 1, 6], 4, 2, 8)
    tau = 0.87
    for base in (0.0, 1e6):
        out, lse = oracle.keybias_attention(q, k, v, s, g, tau, pos, ck, rope_base=base)
        ref = oracle.keybias_attention_gate_grads(q, k, v, s, g, tau, pos, ck, d_out, rope_base=base)
        got = oracle.keybias_attention_gate_grads_at(q, k, v, s, g, tau, pos, ck, d_out, out, lse, rope_base=base)
        np.testing.assert_allclose(got[0], ref[0], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(got[1], ref[1], rtol=1e-9, atol=1e-12)
        assert abs(got[2] - ref[2]) <= 1e-9 * max(1.0, abs(ref[2]))
    out, lse = oracle.keybias_attention(q, k, v, s, g, tau, pos, ck)
    base_dg = oracle.keybias_attention_gate_grads_at(q, k, v, s, g, tau, pos, ck, d_out, out, lse)[1]
    lse2 = lse.copy()
    lse2[2] += 0.7
    dg2 = oracle.keybias_attention_gate_grads_at(q, k, v, s, g, tau, pos, ck, d_out, out, lse2)[1]
    np.testing.assert_allclose(dg2[2], base_dg[2] * math.exp(-0.7), rtol=1e-12)
    np.testing.assert_allclose(np.delete(dg2, 2), np.delete(base_dg, 2), rtol=1e-12)


def test_gate_grads_at_one_key_closed_form():
    """One key per sequence with lse = its own logit (P = 1) and an arbitrary
    stored output u: dS = <dO, v - u>, so dL/ds = sum_h g_h dS_h,
    dL/dg_h = sum_j s_j dS_hj and dL/dtau = -sum dS <q, k> / (sqrt(D) tau^2)
    (rotation at one shared position keeps the inner product)."""
    q, k, v, s, g, _, _, d_out = _grad_case(56, [1, 1, 1], 4, 2, 8)
    pos = np.array([7, 0, 250])
    ck = np.arange(4)
    tau = 0.93
    u = np.random.default_rng(57).standard_normal(q.shape)
    qk = np.stack([[q[j, h] @ k[j, h // 2] for h in range(4)] for j in range(3)]) / (np.sqrt(8) * tau)
    lse = (qk + g[None, :] * s[:, None]).T                                     # [head, key]
    dsm = np.stack([[d_out[j, h] @ (v[j, h // 2] - u[j, h]) for h in range(4)] for j in range(3)])
    ds, dg, dt = oracle.keybias_attention_gate_grads_at(q, k, v, s, g, tau, pos, ck, d_out, u, lse)
    np.testing.assert_allclose(ds, (dsm * g[None, :]).sum(1), rtol=1e-12)
    np.testing.assert_allclose(dg, (dsm * s[:, None]).sum(0), rtol=1e-12)
    assert abs(dt - float(-(dsm * qk).sum() / tau)) <= 1e-12 * max(1.0, abs(dt))


# ------------------------------------------------------ random-budget sampling ----
def test_random_budgets_range_and_uniformity():
    """Budgets lie in {0..n_doc}; over seeds every value is drawn with frequency
    1/(n_doc+1) (binomial bound at ~5 sigma), both ends included; an empty
    document gets 0; the same seed gives the same budgets, another seed others."""
    db = np.array([0, 5, 0, 3])
    de = np.array([9, 5, 1, 40003])
    seeds = 3000
    cnt = np.zeros(10)
    ends = [0, 0]
    for sd in range(seeds):
        k = oracle.random_budgets(sd, db, de)
        assert k.dtype == np.int32 and np.all(k >= 0) and np.all(k <= de - db)
        assert k[1] == 0
        cnt[k[0]] += 1
        ends[0] += k[2] == 0
        ends[1] += k[2] == 1
    p = 1 / 10
    assert np.all(np.abs(cnt / seeds - p) <= 5 * np.sqrt(p * (1 - p) / seeds))
    assert abs(ends[0] / seeds - 0.5) <= 5 * np.sqrt(0.25 / seeds)
    np.testing.assert_array_equal(oracle.random_budgets(77, db, de), oracle.random_budgets(77, db, de))
    big = [oracle.random_budgets(sd, db, de)[3] for sd in range(400)]
    assert len(set(big)) >= 390                         # 40001 values: almost never equal
    assert abs(np.mean(big) / 40000 - 0.5) <= 5 * np.sqrt(1 / 12 / 400)
    with pytest.raises(ValueError):
        oracle.random_budgets(0, [3], [2])
