"""Seeded synthetic workloads for the TokenGate pruned-prefill hot path.

This module only draws inputs.  It holds none of the method's arithmetic and
imports neither the oracle nor the HIP library; both of those are fed from
here.  The real workloads of the pages (NIAH at 16k-128k and four long-context
QA / summarisation / code tasks, timed on Qwen3-1.7B at batch size 1) are not
available offline, so these draws stand in for their shapes.

Every component is drawn from its own PCG64 stream, seeded with
(config seed, component id), so that any part can be regenerated without
drawing the others.  bf16 values are produced by round-to-nearest-even from
float32; both the GPU path and the oracle receive the identical bf16 values.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# component ids of the per-component random streams
(_C_OUTLIER, _C_X, _C_W1, _C_W2, _C_NEEDLE, _C_SCORES, _C_TIES, _C_GAIN, _C_TAU, _C_Q, _C_K, _C_V, _C_LENS,
 _C_DOUT) = range(14)


def _rng(seed: int, comp: int) -> np.random.Generator:
    return np.random.default_rng([seed, comp])


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """Round float32 -> bfloat16 (round to nearest even), as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    """Exact float32 values of a bfloat16 tensor."""
    return t.to(torch.float32).numpy()


@dataclass
class Workload:
    name: str
    seed: int
    seqlens: list
    q_lens: list                   # question (always kept) tokens at the end of each sequence
    k_doc: list                    # per-sequence document budget
    d_model: int
    d_hid: int
    x_dtype: str                   # "f32" or "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_base: float = 1e6
    tau: float | None = None       # fixed tau, or None = drawn U(0.8, 1.0)
    outliers: int = 0              # channels scaled x20
    needles: int = 0               # residuals shifted by +6 along a random unit direction
    tie_frac: float = 0.0          # fraction of document scores forced to one value
    peaky_scores: int = 0          # planted high scores in the selector input
    extra: dict = field(default_factory=dict)

    # ---- sequence metadata ------------------------------------------------
    @property
    def n_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def doc_begin(self) -> np.ndarray:
        return np.zeros(self.n_seqs, dtype=np.int32)

    @property
    def doc_end(self) -> np.ndarray:
        return (np.asarray(self.seqlens) - np.asarray(self.q_lens)).astype(np.int32)

    @property
    def k_doc_arr(self) -> np.ndarray:
        return np.asarray(self.k_doc, dtype=np.int32)

    @property
    def n_tokens(self) -> int:
        return int(sum(self.seqlens))

    def kept_seqlens(self) -> np.ndarray:
        n = np.asarray(self.seqlens)
        nd = self.doc_end - self.doc_begin
        return np.minimum(self.k_doc_arr, nd) + (n - nd)

    def cu_kept(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.kept_seqlens())]).astype(np.int32)

    # ---- gate inputs ---------------------------------------------------------
    def gate_inputs(self, with_bias: bool = False):
        """x [N, d_model], W1 [d_hid, d_model], b1 [d_hid] or None, w2 [d_hid], b2.

        Returns a dict with torch CPU tensors (x, w1 in x_dtype; w2/b1 float32)
        and their exact float32 values as numpy arrays (x_f, w1_f, ...).
        """
        n, d, dh = self.n_tokens, self.d_model, self.d_hid
        out_ch = None
        if self.outliers:
            out_ch = _rng(self.seed, _C_OUTLIER).choice(d, self.outliers, replace=False)
        x = _rng(self.seed, _C_X).standard_normal((n, d), dtype=np.float32)
        if out_ch is not None:
            x[:, out_ch] *= 20.0
        if self.needles:
            r = _rng(self.seed, _C_NEEDLE)
            cands = np.concatenate([np.arange(c0, c0 + de) for c0, de in
                                    zip(self.cu_seqlens[:-1], self.doc_end)])
            where = r.choice(cands, self.needles, replace=False)
            u = r.standard_normal(d)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            x[where] += 6.0 * u
            self.extra["needle_rows"] = np.sort(where)
        w1 = (_rng(self.seed, _C_W1).standard_normal((dh, d)) * 0.02).astype(np.float32)
        w2 = (_rng(self.seed, _C_W2).standard_normal(dh) * 0.02).astype(np.float32)
        b1 = b2 = None
        if with_bias:
            rb = _rng(self.seed, 100)
            b1 = (rb.standard_normal(dh) * 0.1).astype(np.float32)
            b2 = float(np.float32(rb.standard_normal() * 0.1))
        res = {}
        if self.x_dtype == "bf16":
            xt, w1t = to_bf16(x), to_bf16(w1)
            w2 = bf16_values(to_bf16(w2))
            res.update(x=xt, w1=w1t, x_f=bf16_values(xt), w1_f=bf16_values(w1t))
        else:
            res.update(x=torch.from_numpy(x), w1=torch.from_numpy(w1), x_f=x, w1_f=w1)
        res.update(w2=torch.from_numpy(w2), w2_f=w2,
                   b1=None if b1 is None else torch.from_numpy(b1), b1_f=b1,
                   b2=0.0 if b2 is None else b2)
        return res

    # ---- selector input --------------------------------------------------------
    def topk_scores(self) -> np.ndarray:
        """float32 [N] synthetic selector input with this workload's structure:
        N(0, 1) scores, plus planted peaks and exact tie groups when configured."""
        n = self.n_tokens
        s = _rng(self.seed, _C_SCORES).standard_normal(n).astype(np.float32)
        cu, de = self.cu_seqlens, self.doc_end
        if self.peaky_scores:
            r = _rng(self.seed, _C_NEEDLE + 50)
            cands = np.concatenate([np.arange(c0, c0 + e) for c0, e in zip(cu[:-1], de)])
            where = r.choice(cands, self.peaky_scores, replace=False)
            s[where] = (6.0 + 0.01 * np.arange(self.peaky_scores)).astype(np.float32)
        if self.tie_frac > 0:
            r = _rng(self.seed, _C_TIES)
            for i in range(self.n_seqs):
                a, nd = int(cu[i]), int(de[i])
                t_cnt = int(self.tie_frac * nd)
                if t_cnt == 0:
                    continue
                tie_pos = r.choice(nd, t_cnt, replace=False)
                rest = np.setdiff1d(np.arange(nd), tie_pos)
                rank = max(1, min(int(self.k_doc[i]) - t_cnt // 2, rest.shape[0]))
                # value placed so that the budget cut falls inside the tie group
                t = np.sort(s[a + rest])[::-1][rank - 1]
                s[a + tie_pos] = t
        return s

    # ---- attention inputs ------------------------------------------------------
    def attn_params(self):
        gain = _rng(self.seed, _C_GAIN).uniform(0.5, 2.0, self.n_q_heads).astype(np.float32)
        tau = self.tau
        if tau is None:
            tau = float(np.float32(_rng(self.seed, _C_TAU).uniform(0.8, 1.0)))
        return gain, float(np.float32(tau))

    def qkv(self, m_tot: int | None = None):
        """Q [M, Hq, D], K and V [M, Hkv, D] in bfloat16 (CPU tensors): stand-ins
        for the host model's projections of the kept residuals."""
        m = int(self.cu_kept()[-1]) if m_tot is None else m_tot
        hq, hkv, dd = self.n_q_heads, self.n_kv_heads, self.head_dim
        q = to_bf16(_rng(self.seed, _C_Q).standard_normal((m, hq, dd), dtype=np.float32))
        k = to_bf16(_rng(self.seed, _C_K).standard_normal((m, hkv, dd), dtype=np.float32))
        v = to_bf16(_rng(self.seed, _C_V).standard_normal((m, hkv, dd), dtype=np.float32))
        return q, k, v

    def d_out(self, m_tot: int | None = None, seed_offset: int = 0):
        """dL/dO [M, Hq, D] in bfloat16 (CPU tensor): a stand-in for the gradient
        that training hands back to the attention output."""
        m = int(self.cu_kept()[-1]) if m_tot is None else m_tot
        r = _rng(self.seed + seed_offset, _C_DOUT)
        return to_bf16(r.standard_normal((m, self.n_q_heads, self.head_dim), dtype=np.float32))


def _qwen_layer(**kw):
    base = dict(d_model=2048, d_hid=256, x_dtype="bf16", n_q_heads=16, n_kv_heads=8,
                head_dim=128, rope_base=1e6, outliers=8)
    base.update(kw)
    return Workload(**base)


def tiny() -> Workload:
    """512 tokens (448 document + 64 question), d_model 256 fp32, gate 256->64->1,
    keep 128 document tokens, 4 q / 2 kv heads, head_dim 64, tau 0.9, seed 0."""
    return Workload(name="tiny", seed=0, seqlens=[512], q_lens=[64], k_doc=[128],
                    d_model=256, d_hid=64, x_dtype="f32", n_q_heads=4, n_kv_heads=2,
                    head_dim=64, rope_base=1e6, tau=0.9)


def qwen16k() -> Workload:
    """Qwen3-1.7B-shaped gated layer at 16k: 16128 document + 256 question tokens,
    keep 1536 document tokens."""
    return _qwen_layer(name="16k", seed=1, seqlens=[16384], q_lens=[256], k_doc=[1536])


BUDGET_PCTS = (5, 10, 25, 50, 100)


def sweep32k(pct: int = 5) -> Workload:
    """32k budget sweep: 32512 document + 256 question tokens, budget = floor
    (n_doc * pct / 100), 32 needle residuals and 32 planted peak scores."""
    n_doc = 32768 - 256
    return _qwen_layer(name=f"32k@{pct}%", seed=2, seqlens=[32768], q_lens=[256],
                       k_doc=[n_doc * pct // 100], needles=32, peaky_scores=32)


def long128k() -> Workload:
    """128k: 130816 document + 256 question tokens, keep 8192 document tokens."""
    return _qwen_layer(name="128k", seed=3, seqlens=[131072], q_lens=[256], k_doc=[8192])


def varlen() -> Workload:
    """8 packed sequences, lengths U{4096..65536}, questions U{128..512}, budget
    8% of each document, 5% of document scores in one exact tie group."""
    r = _rng(4, _C_LENS)
    lens = r.integers(4096, 65537, 8).tolist()
    qls = r.integers(128, 513, 8).tolist()
    k = [(n - q) * 8 // 100 for n, q in zip(lens, qls)]
    return _qwen_layer(name="varlen", seed=4, seqlens=lens, q_lens=qls, k_doc=k, tie_frac=0.05)


def all_configs():
    return [tiny(), qwen16k()] + [sweep32k(p) for p in BUDGET_PCTS] + [long128k(), varlen()]


def by_name(name: str) -> Workload:
    for w in all_configs():
        if w.name == name:
            return w
    raise KeyError(name)


def custom(seqlens, q_lens, k_doc, d_model=256, d_hid=64, x_dtype="bf16", n_q_heads=4,
           n_kv_heads=2, head_dim=64, seed=7, **kw) -> Workload:
    """Small workload of any shape, for edge cases (ragged lengths, tiny budgets)."""
    return Workload(name="custom", seed=seed, seqlens=list(seqlens), q_lens=list(q_lens),
                    k_doc=list(k_doc), d_model=d_model, d_hid=d_hid, x_dtype=x_dtype,
                    n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim, **kw)


LONG_PAD = 65537   # far above the 16 Ki tokens up to which the one-workgroup selector runs


def pad_long_sequence(scores, cu_seqlens, doc_begin, doc_end, k_doc, n=LONG_PAD, seed=99):
    """The same selector input with one sequence of n tokens appended (its
    whole length a document, 1% budget, N(0,1) fp32 scores).  The original
    tokens keep their indices and, since kept indices are stored sequence by
    sequence, their kept list is the first part of the padded call's output.
    Used to send small inputs through the chunked selector (max_seqlen > 16 Ki).
    scores may be None (random-K mode draws its own)."""
    n0 = int(np.asarray(cu_seqlens)[-1])
    cu = np.concatenate([np.asarray(cu_seqlens, np.int64), [n0 + n]]).astype(np.int32)
    b = np.concatenate([np.asarray(doc_begin, np.int64), [0]]).astype(np.int32)
    e = np.concatenate([np.asarray(doc_end, np.int64), [n]]).astype(np.int32)
    k = np.concatenate([np.asarray(k_doc, np.int64), [n // 100]]).astype(np.int32)
    if scores is not None:
        extra = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
        scores = np.concatenate([np.asarray(scores, np.float32), extra])
    return scores, cu, b, e, k
