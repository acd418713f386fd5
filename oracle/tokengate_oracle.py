"""TokenGate pruned-prefill oracle: plain, slow, obviously correct CPU reference.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
imports nothing from the product path.

Everything is computed in float64 with numpy.  There is no blocking, fusion or
reordering beyond what each definition states, apart from chunking the gate
over rows and the attention over (sequence, head, 512 query rows), which does
not change any result.

Sources.  The method is described by the TokenGate news pages:
  [ES] "Investigadores de Stanford y UC Berkeley Presentan TokenGate: La
       Atención con Compuertas por Token Hace el Prefill de Contexto Largo
       Hasta 11.3x Más Rápido" (spke.com, Spanish edition of the MarkTechPost
       article).
  [GR] "TokenGate: το μοντέλο που διαβάζει στα πεταχτά μακριά κείμενα…"
       (mainews.gr).
  [RU] "Researchers from Stanford and UC Berkeley introduce TokenGate"
       (aikraft.ru), section "Техническая реализация".
The pages leave several details open; the readings used here are stated in
each function's docstring.

Parity status per function:
  gate_score          pinned (torch fp64 linear+silu, closed forms, scalar loop)
  topk_select         pinned (brute-force sort, exhaustive tiny cases, invariants)
  splitmix64          pinned (published reference outputs for seed 0)
  random_budgets      pinned (range, full and empty budgets reached, uniform
                      frequencies over seeds, determinism)
  random_k_select     pinned (budget and question invariants, determinism, selection
                      frequencies uniform over seeds)
  gather_kept         pinned (definition, invariants)
  rope                pinned (complex-rotation form, norm and relative-position
                      invariants)
  keybias_attention   pinned (textbook causal SDPA reduction, shift invariance,
                      pruning == masking, tau placement, GQA, varlen, closed forms)
  keybias_attention_gate_grads
                      pinned (central finite differences of the forward, closed
                      forms: g = 0 gives ds = 0, sum_j ds_j = 0, tau scaling);
                      its condition scales pinned by the triangle inequality
                      and the one-key closed form
  keybias_attention_gate_grads_at
                      pinned (equals keybias_attention_gate_grads at the exact
                      forward outputs; a constant added to a head's lse scales
                      that head's terms by exp(-c); one-key closed form with an
                      arbitrary stored output)
  keybias_decode      pinned (equals the prefill row of a kept token placed at its
                      position, closed forms, no-visible-key case, shift invariance)
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


# ----------------------------------------------------------------------------
# Step 1: gate MLP score
# ----------------------------------------------------------------------------
def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)), evaluated in float64."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def gate_score(x, w1, b1, w2, b2, chunk_rows: int = 8192) -> np.ndarray:
    """Score every token from its layer-L residual with a small two-layer MLP.

    [ES] section "¿Cómo funciona la poda de tokens aprendida de TokenGate?"
    (gate module phase): an MLP maps each token's post-attention residual at
    the gate layer to one score.  [GR] section "Πώς αποφασίζει τι θα
    κρατήσει": the gate scores every token.

    Reading (the pages only say "small MLP"): two layers with SiLU between,
        s_t = w2 . SiLU(W1 x_t + b1) + b2,
    W1 in nn.Linear layout [d_hid, d_model].  Every token is scored, document
    and question alike.  No squashing is applied to the output.

    x: [N, d_model]; w1: [d_hid, d_model]; b1: [d_hid] or None; w2: [d_hid];
    b2: scalar.  Returns float64 [N].
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    d_hid = w1.shape[0]
    b1 = np.zeros(d_hid) if b1 is None else np.asarray(b1, dtype=np.float64)
    out = np.empty(x.shape[0], dtype=np.float64)
    for r0 in range(0, x.shape[0], chunk_rows):
        a = x[r0:r0 + chunk_rows] @ w1.T + b1
        out[r0:r0 + chunk_rows] = silu(a) @ w2 + float(b2)
    return out


# ----------------------------------------------------------------------------
# Step 2: top-K selection, question always kept
# ----------------------------------------------------------------------------
def kept_counts(cu_seqlens, doc_begin, doc_end, k_doc) -> np.ndarray:
    """Kept tokens per sequence: min(K_s, n_doc_s) + (n_s - n_doc_s).

    [ES] "¿Cómo funciona…?": only the document part of the prompt can be
    pruned and the question never is.  K_s counts document tokens; a budget
    larger than the document keeps all of it, K_s = 0 keeps none of it.
    Returns cu_kept [S+1] (int64).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    s = len(cu) - 1
    cu_kept = np.zeros(s + 1, dtype=np.int64)
    for i in range(s):
        n = cu[i + 1] - cu[i]
        n_doc = int(doc_end[i]) - int(doc_begin[i])
        if not (0 <= doc_begin[i] <= doc_end[i] <= n) or k_doc[i] < 0:
            raise ValueError(f"sequence {i}: bad document span or budget")
        cu_kept[i + 1] = cu_kept[i] + min(int(k_doc[i]), n_doc) + (n - n_doc)
    return cu_kept


def _doc_order(scores_doc: np.ndarray) -> np.ndarray:
    """Positions of document tokens in selection order.

    Order: higher score first; equal scores by lower index first.  Real
    comparisons are used, so -0.0 equals +0.0 and +-inf order as usual.  NaN
    scores rank below every number, -inf included, and among themselves by
    index.  (The pages fix no rule for ties or special values; lowest index
    wins is the reading adopted here.)
    """
    s = np.asarray(scores_doc, dtype=np.float64)
    idx = np.arange(s.shape[0])
    nan = np.isnan(s)
    num_idx = idx[~nan]
    num_s = s[~nan]
    # lexsort: last key is primary -> primary = -score ascending, then index.
    order = num_idx[np.lexsort((num_idx, -num_s))]
    return np.concatenate([order, idx[nan]])


def topk_select(scores, cu_seqlens, doc_begin, doc_end, k_doc):
    """Keep the K highest-scoring document tokens plus every other token.

    [ES] "¿Cómo funciona…?": a top-K selector keeps the highest-scoring
    tokens; only the document is prunable, the question is never pruned.
    [GR] "Πώς αποφασίζει…": only the best-scored tokens stay, and the
    question always stays whole.

    scores: float32 (or float64) [N_tot], the array given to the selector;
    cu_seqlens: [S+1]; doc_begin/doc_end: [S], in-sequence document span
    [doc_begin, doc_end); k_doc: [S] document budget.
    Tokens outside the document span are always kept.  Kept global indices are
    returned in ascending order within each sequence, sequences in order.
    Returns (kept_idx int64 [M_tot], cu_kept int64 [S+1]).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    sc = np.asarray(scores)
    cu_kept = kept_counts(cu, doc_begin, doc_end, k_doc)
    parts = []
    for i in range(len(cu) - 1):
        start, n = int(cu[i]), int(cu[i + 1] - cu[i])
        db, de = int(doc_begin[i]), int(doc_end[i])
        k_eff = min(int(k_doc[i]), de - db)
        order = _doc_order(sc[start + db:start + de])
        kept_doc = order[:k_eff] + db
        nondoc = np.concatenate([np.arange(0, db), np.arange(de, n)])
        local = np.sort(np.concatenate([kept_doc, nondoc]).astype(np.int64))
        parts.append(local + start)
    kept = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    assert kept.shape[0] == cu_kept[-1]
    return kept, cu_kept


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n outputs of SplitMix64 seeded with `seed` (uint64).

    SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014; the 64-bit finalizer of Vigna's reference
    implementation): the state advances by the golden-ratio increment
    0x9E3779B97F4A7C15 and each state is mixed by two xor-shift-multiply
    rounds and a final xor-shift.  Output i depends only on seed + (i+1)
    increments, so it is a counter-based generator.
    """
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (np.arange(1, n + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15))
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def random_scores(seed: int, n: int) -> np.ndarray:
    """Random scores for n tokens, one independent uniform 30-bit draw each: the
    top 30 bits d_t of SplitMix64 output t (t = global token index), encoded as
    the positive normal fp32 whose bit pattern is 2^23 + d_t.  Positive floats
    order like their bit patterns, so the scores order exactly like the draws;
    only that order matters to the selector."""
    d = (splitmix64(seed, n) >> np.uint64(34)).astype(np.uint32)
    return (d + np.uint32(1 << 23)).view(np.float32)


def random_budgets(seed, doc_begin, doc_end):
    """Random-budget sampling for the training schedule ([ES] "¿Qué es la
    atención…?": each step averages a full-context loss and a loss at a random
    token budget, so one gate serves every budget).

    Reading (the pages name no distribution): sequence s draws its document
    budget uniformly from {0, 1, ..., n_doc_s}, where 0 keeps only the question
    and n_doc_s is the full context.  The draw uses SplitMix64 output s for
    `seed`: with u = its top 53 bits, K_s = floor(u (n_doc_s + 1) / 2^53),
    computed exactly in integers.  Returns int32 [S].
    """
    db = np.asarray(doc_begin, dtype=np.int64)
    de = np.asarray(doc_end, dtype=np.int64)
    if np.any(de < db):
        raise ValueError("doc_end < doc_begin")
    z = splitmix64(seed, len(db))
    out = np.empty(len(db), dtype=np.int32)
    for i in range(len(db)):
        u = int(z[i]) >> 11
        out[i] = (u * (int(de[i] - db[i]) + 1)) >> 53
    return out


def random_k_select(seed, cu_seqlens, doc_begin, doc_end, k_doc):
    """Random-K selector mode ([RU] "Техническая реализация" and the ablation the
    pages report: random token selection on the co-adapted backbone).

    Reading: the same budget and the same always-kept question as the learned
    selector, but the K_eff document tokens of each sequence are a seeded
    uniform random subset: the selector of topk_select applied to
    random_scores(seed, N_tot) instead of the gate's scores (30-bit draws, so
    equal draws are possible and keep the lower index, as for gate scores).
    Returns (kept_idx, cu_kept) as topk_select does.
    """
    n = int(np.asarray(cu_seqlens)[-1])
    return topk_select(random_scores(seed, n), cu_seqlens, doc_begin, doc_end, k_doc)


# ----------------------------------------------------------------------------
# Step 3: compaction of the kept set
# ----------------------------------------------------------------------------
def gather_kept(x, scores, kept_idx, cu_seqlens, cu_kept):
    """Compact kept residuals, scores and original positions.

    [ES] "¿Cómo funciona…?" (pruned forward phase): layers above the gate see
    only the kept tokens and never create KV entries for pruned ones, so every
    downstream tensor is sized by the kept count.

    pos_kept[m] = kept_idx[m] - cu_seqlens[seq(m)], the token's original
    position inside its sequence.  Returns (x_kept, s_kept, pos_kept int64).
    """
    kept_idx = np.asarray(kept_idx, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    ck = np.asarray(cu_kept, dtype=np.int64)
    pos = np.empty_like(kept_idx)
    for i in range(len(ck) - 1):
        pos[ck[i]:ck[i + 1]] = kept_idx[ck[i]:ck[i + 1]] - cu[i]
    return np.asarray(x)[kept_idx], np.asarray(scores)[kept_idx], pos


# ----------------------------------------------------------------------------
# Step 4: token-gated (key-bias) causal GQA attention over the kept set
# ----------------------------------------------------------------------------
def rope(x, pos, base: float) -> np.ndarray:
    """Rotary position embedding on original positions, float64.

    The pages say nothing about positions.  Reading: rotate-half pairing of
    channel m with channel m + D/2, angle pos * base^(-2m/D), m in [0, D/2).
    x: [M, H, D]; pos: [M].  base <= 0 means no rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    if base is None or base <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    m = np.arange(half, dtype=np.float64)
    inv_freq = base ** (-2.0 * m / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def keybias_attention(q, k, v, s_kept, gain, tau, pos, cu_kept,
                      rope_base: float = 1e6, rows=None, block_rows: int = 512):
    """Token-gated causal attention over the kept set.

    [ES] "¿Qué es la atención con control de acceso por tokens…?": each kept
    token's gate score becomes a bias on the attention logits of the layers
    above the gate; a learnable per-head gain scales it and a learnable
    temperature corrects for each query seeing fewer keys.  [RU] "Техническая
    реализация" describes the same router-style bias.

    Reading of the formula (the pages do not print it):
        l_ij = <R(q_i, pos_i), R(k_j, pos_j)> / (sqrt(D) * tau) + g_h * s_j
    over keys j of the same sequence with pos_j <= pos_i (self included);
    O_i = sum_j softmax_j(l_ij) v_j;  LSE_i = log sum_j exp(l_ij).
    GQA: q head h reads kv head h // (Hq / Hkv).  g has one value per q head,
    tau is one scalar.  Every kept key is biased, question keys included.

    q: [M, Hq, D]; k, v: [M, Hkv, D]; s_kept: [M]; gain: [Hq]; pos: [M];
    cu_kept: [S+1].  rows: optional iterable of kept-row indices to evaluate
    (others are left NaN).  Returns (O [M, Hq, D] float64, LSE [Hq, M] float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s_kept = np.asarray(s_kept, dtype=np.float64)
    gain = np.asarray(gain, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    ck = np.asarray(cu_kept, dtype=np.int64)
    m_tot, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if not (tau > 0 and math.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    grp = hq // hkv
    scale = 1.0 / (math.sqrt(d) * float(tau))
    out = np.full((m_tot, hq, d), np.nan)
    lse = np.full((hq, m_tot), np.nan)
    want = np.zeros(m_tot, dtype=bool)
    if rows is None:
        want[:] = True
    else:
        want[np.asarray(list(rows), dtype=np.int64)] = True
    for si in range(len(ck) - 1):
        a, b = int(ck[si]), int(ck[si + 1])
        if a == b or not want[a:b].any():
            continue
        p = pos[a:b]
        qr = rope(q[a:b], p, rope_base)
        kr = rope(k[a:b], p, rope_base)
        vs = v[a:b]
        sel = np.nonzero(want[a:b])[0]
        for h in range(hq):
            hk = h // grp
            bias = gain[h] * s_kept[a:b]
            for r0 in range(0, sel.shape[0], block_rows):
                ri = sel[r0:r0 + block_rows]
                logit = (qr[ri, h, :] @ kr[:, hk, :].T) * scale + bias[None, :]
                mask = p[None, :] > p[ri][:, None]
                logit[mask] = -np.inf
                mx = logit.max(axis=1, keepdims=True)
                e = np.exp(logit - mx)
                den = e.sum(axis=1, keepdims=True)
                out[a + ri, h, :] = (e @ vs[:, hk, :]) / den
                lse[h, a + ri] = (mx + np.log(den))[:, 0]
    return out, lse


def keybias_attention_gate_grads(q, k, v, s_kept, gain, tau, pos, cu_kept, d_out, rope_base: float = 1e6,
                                 scales: bool = False):
    """Gradients of a loss L through token-gated attention with respect to the
    gate-side parameters: the kept keys' scores s_j, the per-head gains g_h and
    the temperature tau, given dL/dO ([ES] "¿Qué es la atención…?": the gain and
    the temperature are learned, and the bias is how the loss reaches the gate's
    scores during training).

    From the forward definition (keybias_attention), per sequence and q head h:
        P_ij = softmax_j(l_ij),  dP_ij = <dO_i, v_j>,  Delta_i = sum_j P_ij dP_ij,
        dS_ij = P_ij (dP_ij - Delta_i)      (= dL/dl_ij)
    and with l_ij = <q~_i, k~_j> / (sqrt(D) tau) + g_h s_j:
        dL/ds_j  = sum_h g_h sum_i dS_hij
        dL/dg_h  = sum_ij s_j dS_hij
        dL/dtau  = sum_hij dS_hij * (-<q~_i, k~_j> / (sqrt(D) tau^2)).
    d_out: [M, Hq, D].  Returns (ds [M], dg [Hq], dtau) in float64.

    scales=True also returns the same three sums taken over absolute values
    with |dS_ij| replaced by P_ij (|dP_ij| + |Delta_i|): a first-order bound
    on how far each result moves when every logit moves by a relative amount
    and every Delta_i by a relative amount (the condition scale a rounded
    implementation's error is measured against).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    s_kept = np.asarray(s_kept, dtype=np.float64)
    gain = np.asarray(gain, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    ck = np.asarray(cu_kept, dtype=np.int64)
    m_tot, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if not (tau > 0 and math.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    grp = hq // hkv
    scale = 1.0 / (math.sqrt(d) * float(tau))
    ds = np.zeros(m_tot)
    dg = np.zeros(hq)
    dtau = 0.0
    ds_mag = np.zeros(m_tot)
    dg_mag = np.zeros(hq)
    dtau_mag = 0.0
    for si in range(len(ck) - 1):
        a, b = int(ck[si]), int(ck[si + 1])
        if a == b:
            continue
        p = pos[a:b]
        qr = rope(q[a:b], p, rope_base)
        kr = rope(k[a:b], p, rope_base)
        vs = v[a:b]
        mask = p[None, :] > p[:, None]
        for h in range(hq):
            hk = h // grp
            qk = (qr[:, h, :] @ kr[:, hk, :].T) * scale
            logit = qk + gain[h] * s_kept[a:b][None, :]
            logit[mask] = -np.inf
            e = np.exp(logit - logit.max(axis=1, keepdims=True))
            pr = e / e.sum(axis=1, keepdims=True)
            dp = d_out[a:b, h, :] @ vs[:, hk, :].T
            delta = (pr * dp).sum(axis=1, keepdims=True)
            dsm = pr * (dp - delta)
            col = dsm.sum(axis=0)
            ds[a:b] += gain[h] * col
            dg[h] += float(s_kept[a:b] @ col)
            dtau += float((dsm * (-qk / float(tau))).sum())
            if scales:
                env = pr * (np.abs(dp) + np.abs(delta))
                ecol = env.sum(axis=0)
                ds_mag[a:b] += abs(gain[h]) * ecol
                dg_mag[h] += float(np.abs(s_kept[a:b]) @ ecol)
                dtau_mag += float((env * np.abs(qk / float(tau))).sum())
    if scales:
        return ds, dg, dtau, (ds_mag, dg_mag, dtau_mag)
    return ds, dg, dtau


def keybias_attention_gate_grads_at(q, k, v, s_kept, gain, tau, pos, cu_kept, d_out, out, lse,
                                    rope_base: float = 1e6, scales: bool = False):
    """The same three gradients as keybias_attention_gate_grads, evaluated at a
    stored forward (out, lse) instead of one recomputed exactly.

    A backward pass that receives the forward's outputs (as FlashAttention-style
    backward passes do) takes the probabilities from the stored log-sum-exp and
    Delta from the stored output:
        P_ij = exp(l_ij - lse_i)  (0 where pos_j > pos_i),
        Delta_i = <dO_i, out_i>,   dS_ij = P_ij (<dO_i, v_j> - Delta_i),
    and then, exactly as in keybias_attention_gate_grads,
        dL/ds_j = sum_h g_h sum_i dS_hij,   dL/dg_h = sum_ij s_j dS_hij,
        dL/dtau = sum_hij dS_hij * (-<q~_i, k~_j> / (sqrt(D) tau^2)).
    With (out, lse) the exact forward outputs this is the same function (softmax
    rows sum to one, and out_i = sum_j P_ij v_j gives Delta_i = sum_j P_ij dP_ij).
    out: [M, Hq, D]; lse: [Hq, M] (natural log).

    scales=True also returns two sets of condition sums over the terms
    e_ij = P_ij (|dP_ij| + |Delta_i|) times |g_h|, |s_j| or |<q~, k~>| / (sqrt(D) tau^2):
    their plain sums (as keybias_attention_gate_grads gives), and their
    quadrature sums, the scale of independent relative errors: for dL/ds_j the
    root of the sum of squared terms of its column; for dL/dg_h and dL/dtau the
    root of the sum over query rows of the squared row sums (an error shared by
    the terms of one row, such as one in Delta_i, adds up along the row and in
    quadrature across rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    s_kept = np.asarray(s_kept, dtype=np.float64)
    gain = np.asarray(gain, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    ck = np.asarray(cu_kept, dtype=np.int64)
    m_tot, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if not (tau > 0 and math.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    grp = hq // hkv
    scale = 1.0 / (math.sqrt(d) * float(tau))
    ds = np.zeros(m_tot)
    dg = np.zeros(hq)
    dtau = 0.0
    ds_mag = np.zeros(m_tot)
    dg_mag = np.zeros(hq)
    dtau_mag = 0.0
    ds_q2 = np.zeros(m_tot)
    dg_q2 = np.zeros(hq)
    dtau_q2 = 0.0
    for si in range(len(ck) - 1):
        a, b = int(ck[si]), int(ck[si + 1])
        if a == b:
            continue
        p = pos[a:b]
        qr = rope(q[a:b], p, rope_base)
        kr = rope(k[a:b], p, rope_base)
        vs = v[a:b]
        mask = p[None, :] > p[:, None]
        for h in range(hq):
            hk = h // grp
            qk = (qr[:, h, :] @ kr[:, hk, :].T) * scale
            logit = qk + gain[h] * s_kept[a:b][None, :]
            pr = np.exp(logit - lse[h, a:b][:, None])
            pr[mask] = 0.0
            dp = d_out[a:b, h, :] @ vs[:, hk, :].T
            delta = np.sum(d_out[a:b, h, :] * out[a:b, h, :], axis=1)[:, None]
            dsm = pr * (dp - delta)
            col = dsm.sum(axis=0)
            ds[a:b] += gain[h] * col
            dg[h] += float(s_kept[a:b] @ col)
            dtau += float((dsm * (-qk / float(tau))).sum())
            if scales:
                env = pr * (np.abs(dp) + np.abs(delta))
                ecol = env.sum(axis=0)
                ds_mag[a:b] += abs(gain[h]) * ecol
                dg_mag[h] += float(np.abs(s_kept[a:b]) @ ecol)
                et = env * np.abs(qk / float(tau))
                dtau_mag += float(et.sum())
                ds_q2[a:b] += gain[h] ** 2 * (env ** 2).sum(axis=0)
                dg_q2[h] += float(((env @ np.abs(s_kept[a:b])) ** 2).sum())
                dtau_q2 += float((et.sum(axis=1) ** 2).sum())
    if scales:
        return ds, dg, dtau, (ds_mag, dg_mag, dtau_mag), (np.sqrt(ds_q2), np.sqrt(dg_q2), math.sqrt(dtau_q2))
    return ds, dg, dtau


def keybias_decode(q_new, q_pos, k, v, s_kept, gain, tau, pos, cu_kept, rope_base: float = 1e6):
    """One decode step of token-gated attention over the kept-only cache.

    [ES] "¿Qué es la atención con control de acceso por tokens…?": above the
    gate layer only kept tokens have keys and values (pruned tokens never get
    KV entries), and every kept key carries its gate-score bias.  A token
    generated after the prefill therefore attends to that kept cache.

    Reading (the pages do not describe decoding): the new query of sequence s
    sits at original position q_pos[s] and uses the prefill logit
        l_j = <R(q, q_pos[s]), R(k_j, pos_j)> / (sqrt(D) * tau) + g_h * s_j
    over the kept keys j of s with pos_j <= q_pos[s].  The new token's own key
    is part of the cache only if the caller appended it.  A query that sees no
    key gets O = 0 and LSE = -inf.

    q_new: [S, Hq, D]; q_pos: [S]; k, v: [M, Hkv, D]; s_kept: [M]; gain: [Hq];
    pos: [M]; cu_kept: [S+1].  Returns (O [S, Hq, D], LSE [Hq, S]) float64.
    """
    q_new = np.asarray(q_new, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s_kept = np.asarray(s_kept, dtype=np.float64)
    gain = np.asarray(gain, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    ck = np.asarray(cu_kept, dtype=np.int64)
    n_seqs, hq, d = q_new.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if not (tau > 0 and math.isfinite(tau)):
        raise ValueError("tau must be positive and finite")
    grp = hq // hkv
    scale = 1.0 / (math.sqrt(d) * float(tau))
    out = np.zeros((n_seqs, hq, d))
    lse = np.full((hq, n_seqs), -np.inf)
    for si in range(n_seqs):
        a, b = int(ck[si]), int(ck[si + 1])
        vis = np.nonzero(pos[a:b] <= q_pos[si])[0]
        if vis.size == 0:
            continue
        qr = rope(q_new[si:si + 1], q_pos[si:si + 1], rope_base)[0]     # [Hq, D]
        kr = rope(k[a:b], pos[a:b], rope_base)[vis]                      # [n_vis, Hkv, D]
        vv = v[a:b][vis]
        for h in range(hq):
            hk = h // grp
            logit = (kr[:, hk, :] @ qr[h]) * scale + gain[h] * s_kept[a:b][vis]
            mx = logit.max()
            e = np.exp(logit - mx)
            den = e.sum()
            out[si, h] = (e @ vv[:, hk, :]) / den
            lse[h, si] = mx + math.log(den)
    return out, lse


# ----------------------------------------------------------------------------
# The whole gated layer, for end-to-end checks
# ----------------------------------------------------------------------------
def gated_layer(x, w1, b1, w2, b2, cu_seqlens, doc_begin, doc_end, k_doc):
    """Gate -> select -> gather.  Attention inputs are projections of the kept
    residuals that the host model owns; callers pass them separately.
    Returns dict with fp64 scores, their float32 rounding (what the selector
    consumes), kept_idx, cu_kept, x_kept, s_kept, pos_kept."""
    s64 = gate_score(x, w1, b1, w2, b2)
    s32 = s64.astype(np.float32)
    kept, cu_kept = topk_select(s32, cu_seqlens, doc_begin, doc_end, k_doc)
    xk, sk, pk = gather_kept(x, s32, kept, cu_seqlens, cu_kept)
    return dict(scores=s64, scores_f32=s32, kept_idx=kept, cu_kept=cu_kept,
                x_kept=xk, s_kept=sk, pos_kept=pk)
