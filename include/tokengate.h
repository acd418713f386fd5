/*
 * tokengate.h - C ABI of libtokengate, the gfx950 (MI355X) hot path of
 * TokenGate's pruned prefill: gate score -> top-K select -> compaction ->
 * token-gated (key-bias) causal GQA attention over the kept tokens.
 *
 * Source of the method: the TokenGate news pages, chiefly the spke.com
 * article "Investigadores de Stanford y UC Berkeley Presentan TokenGate: La
 * Atencion con Compuertas por Token Hace el Prefill de Contexto Largo Hasta
 * 11.3x Mas Rapido", sections "Como funciona la poda de tokens aprendida de
 * TokenGate?" (three-phase forward pass, gate module, pruned forward, question
 * never pruned), "Que es la atencion con control de acceso por tokens?"
 * (score as attention-logit bias, per-head gain, temperature) and "Como se
 * despliega TokenGate?" (document placeholder and keep budget).
 *
 * Conventions shared by every call
 *  - Pointers marked [device] are caller-owned device memory; pointers marked
 *    [host] are ordinary host memory.  The library never allocates or frees
 *    memory; scratch space comes from the caller through a workspace
 *    argument sized by the matching *_workspace_bytes() call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every device call is asynchronous and stream-ordered; none synchronises.
 *  - Inputs are read-only.  Outputs must not alias inputs and are fully
 *    overwritten.
 *  - All scalar arguments and host-visible pointers are validated before any
 *    HIP call; a failed check returns TG_ERR_INVALID_ARG / TG_ERR_UNSUPPORTED
 *    / TG_ERR_WORKSPACE and launches nothing.  A failed launch returns
 *    TG_ERR_HIP.  Device-resident metadata (cu_seqlens, spans, budgets,
 *    cu_kept, kept indices, positions) is trusted: inconsistent values are
 *    undefined behaviour, unless TG_DEBUG=1 is set in the environment (read
 *    at every call).  Then each call that takes such metadata first copies it
 *    to the host, synchronising `stream`, and checks it: offsets start at 0,
 *    never decrease and end at the stated totals; no sequence is longer than
 *    max_seqlen / max_kept_seqlen; document spans lie inside their sequences
 *    and budgets are >= 0; cu_kept equals tg_kept_counts of the rest; kept
 *    indices lie in their sequences, ascending; positions are >= 0 and
 *    strictly increase within a sequence; and a call that reads a prepared
 *    cache (tg_attn_forward, tg_attn_decode, tg_attn_gate_grads) finds in the
 *    header tg_attn_prepare left in it the same n_seqs, n_kept_total,
 *    n_kv_heads, head_dim, rotary base and cu_kept (by a hash) as its own.
 *    A violation returns TG_ERR_INVALID_ARG and launches nothing.
 *  - Calls are reentrant and thread-safe, except that calls of
 *    tg_topk_select_noalloc on one GPU share its scratch array and must not
 *    overlap (see there).  The only global state is, per
 *    kernel, an atomic mask of the devices on which its dynamic LDS limit has
 *    been raised (once per device, at that kernel's first call there), the
 *    per-device address of tg_topk_select_noalloc's scratch array, a cache
 *    of the per-device CU count, and a mutex-guarded cache of recent forward
 *    grid plans.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARG = 1,  /* bad scalar, NULL required pointer, misaligned pointer */
    TG_ERR_UNSUPPORTED = 2,  /* a shape or dtype the library has no kernel for */
    TG_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    TG_ERR_HIP = 4           /* a HIP launch failed */
};

enum { TG_F32 = 0, TG_BF16 = 1 };   /* element type of residuals / gate weights */

/* Human-readable name of a status code (static string, never NULL). */
const char* tg_status_string(int status);

/*
 * Kept-token counts, on the host.  Only the document span of each sequence is
 * prunable and the question (every token outside the span) is always kept
 * (spke.com article, section on how the pruning works), so the kept count is
 * known before any score exists:
 *     M_s = min(k_doc[s], doc_end[s] - doc_begin[s]) + (n_s - n_doc_s).
 *   n_seqs        number of packed sequences S >= 0
 *   cu_seqlens_h  [host] S+1 int32 prefix offsets, cu[0] = 0, non-decreasing
 *   doc_begin_h,
 *   doc_end_h     [host] S int32, in-sequence document span, 0 <= b <= e <= n_s
 *   k_doc_h       [host] S int32 document budgets >= 0
 *   cu_kept_h     [host, out] S+1 int32 prefix offsets of kept tokens
 * Errors: TG_ERR_INVALID_ARG on NULL pointers, negative sizes, inconsistent
 * spans or int32 overflow.  Never touches the GPU.
 */
int tg_kept_counts(int32_t n_seqs, const int32_t* cu_seqlens_h, const int32_t* doc_begin_h,
                   const int32_t* doc_end_h, const int32_t* k_doc_h, int32_t* cu_kept_h);

/*
 * Gate MLP score of every token (spke.com article, gate-module phase: a small
 * MLP scores each token from its post-attention residual at the gate layer):
 *     scores[t] = w2 . SiLU(W1 x_t + b1) + b2,   SiLU(a) = a * sigmoid(a).
 * The hidden layer is kept in fp32 (bf16 MFMA products, fp32 accumulation).
 *   x             [device] n_tokens rows of d_model elements of x_dtype,
 *                 consecutive rows x_row_stride elements apart
 *   x_dtype       TG_BF16 (MFMA path) or TG_F32 (fp32 FMA path)
 *   w1            [device] d_hid x d_model, row-major (nn.Linear layout), x_dtype
 *   b1            [device] d_hid fp32, or NULL for no bias
 *   w2            [device] d_hid fp32
 *   b2            scalar fp32 output bias
 *   scores        [device, out] n_tokens fp32
 * Requirements: d_model % 8 == 0, x_row_stride >= d_model and % 8 == 0,
 * x and w1 16-byte aligned.  bf16: d_model % 64 == 0, x_row_stride < 2^23
 * and d_hid in {64, 128, 192, 256}; fp32: 1 <= d_hid <= 1024 and d_model <=
 * 2048 (TG_ERR_UNSUPPORTED otherwise).  n_tokens == 0 is a no-op.
 */
int tg_gate_score(const void* x, int32_t x_dtype, int64_t n_tokens, int32_t d_model,
                  int64_t x_row_stride, const void* w1, const float* b1, const float* w2,
                  float b2, int32_t d_hid, float* scores, void* stream);

/* Workspace bytes tg_topk_select needs: per-sequence counters (the
 * first-level histogram, a ticket, the candidate count) and state, per-chunk
 * counts and output offsets, and 8 bytes per token for threshold
 * candidates. */
size_t tg_topk_workspace_bytes(int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen);

/*
 * Top-K selection with the question always kept (spke.com article, gate-module
 * phase and the rule that only the document is prunable).  Per sequence s:
 * keep K_eff = min(k_doc[s], n_doc_s) document tokens in the order (score
 * descending, index ascending), plus every token outside [doc_begin,
 * doc_end).  Score comparison: -0.0 == +0.0, NaN ranks below -inf (NaNs among
 * themselves by index), +-inf order normally.  Output is exact and
 * deterministic.
 *   scores        [device] n_tokens_total fp32
 *   cu_seqlens    [device] S+1 int32
 *   doc_begin, doc_end, k_doc   [device] S int32 each
 *   cu_kept       [device] S+1 int32, as produced by tg_kept_counts
 *   kept_idx      [device, out] cu_kept[S] int32 GLOBAL token indices,
 *                 ascending within each sequence
 *   max_seqlen    host upper bound of every n_s (sizes the grid); at most 4 Mi
 *                 tokens and at most n_tokens_total.  Up to 16 Ki tokens the
 *                 call is one launch of one workgroup per sequence (the
 *                 workspace is then not touched), up to 64 Ki two launches,
 *                 beyond that four launches over token chunks; all give the
 *                 same result.
 *   workspace     [device] >= tg_topk_workspace_bytes(...) bytes, 256-byte
 *                 aligned, contents need not be initialised (the call's first
 *                 kernel zeroes the counters it needs).  Calls that share a
 *                 workspace must not overlap.
 * Errors: TG_ERR_INVALID_ARG on NULL pointers or bad sizes, TG_ERR_UNSUPPORTED
 * for max_seqlen above 4 Mi, TG_ERR_WORKSPACE for a missing or short workspace.
 * n_s > max_seqlen is undefined behaviour (outputs incomplete, never out of
 * bounds).
 */
int tg_topk_select(const float* scores, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                   const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                   const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * tg_topk_select for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as tg_topk_select, without the
 * workspace: the selector's scratch is a library-owned device array of
 * tg_topk_noalloc_max_bytes() = 6 MiB per GPU, allocated with the library's
 * code object on each device it runs on and held until the process ends.  The
 * call itself allocates nothing.
 *   Limit: tg_topk_workspace_bytes(n_seqs, n_tokens_total, max_seqlen) <= 6 MiB
 *   (for example 64 sequences of 512 Ki tokens in total); larger calls return
 *   TG_ERR_UNSUPPORTED before any GPU work.
 *   The first call on each device resolves the array's device address; make
 *   it before capturing the call into a graph.  Every call on one GPU uses the
 *   same array (each call first zeroes the counters it needs): calls that
 *   overlap on one GPU, from several streams or threads, race and give wrong
 *   results, so serialise them.
 */
size_t tg_topk_noalloc_max_bytes(void);
int tg_topk_select_noalloc(const float* scores, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                           const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                           const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx, void* stream);

/*
 * Random-budget sampling, on the host: the training schedule averages a
 * full-context loss and a loss at a random token budget, so that one gate
 * serves every budget (spke.com article, section on token-gated attention).
 * The pages name no distribution; sequence s draws its document budget
 * uniformly from {0, ..., doc_end[s] - doc_begin[s]} (0 keeps only the
 * question, the top value the whole context):
 *     k_doc[s] = floor(u_s (n_doc_s + 1) / 2^53),  u_s = top 53 bits of
 *     SplitMix64 output s for `seed` (see tg_random_k_select),
 * in exact integer arithmetic.  Use a seed other than the random-K scores'.
 *   doc_begin_h, doc_end_h  [host] S int32, 0 <= b <= e
 *   k_doc_h       [host, out] S int32, ready for tg_kept_counts
 * Errors: TG_ERR_INVALID_ARG on NULL pointers, negative S or spans.  Never
 * touches the GPU.
 */
int tg_random_budgets(uint64_t seed, int32_t n_seqs, const int32_t* doc_begin_h, const int32_t* doc_end_h,
                      int32_t* k_doc_h);

/* Workspace bytes tg_random_k_select needs: what tg_topk_select needs plus 4
 * bytes per token for the random scores. */
size_t tg_random_k_workspace_bytes(int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen);

/*
 * Random-K selector mode: the ablation the pages report, where a random
 * token choice replaces the learned gate (aikraft.ru article, section
 * "Техническая реализация").  Same budget, same always-kept question and same
 * output as tg_topk_select, but the K_eff document tokens of each sequence
 * are a seeded uniform random subset: tg_topk_select applied to the scores
 * r_t = the positive normal fp32 with bit pattern 2^23 + d_t, where d_t is the
 * top 30 bits of SplitMix64 output t for `seed` and t the global token index
 * (SplitMix64: Steele, Lea and Flood, OOPSLA 2014; output t = finalizer of
 * seed + (t+1) * 0x9E3779B97F4A7C15).  r_t orders exactly like d_t; equal draws
 * keep the lower index.  Arguments, requirements and errors as for
 * tg_topk_select, without `scores`; workspace >= tg_random_k_workspace_bytes.
 */
int tg_random_k_select(uint64_t seed, int32_t n_seqs, int64_t n_tokens_total, int32_t max_seqlen,
                       const int32_t* cu_seqlens, const int32_t* doc_begin, const int32_t* doc_end,
                       const int32_t* k_doc, const int32_t* cu_kept, int32_t* kept_idx, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Compaction of the kept set (spke.com article, pruned-forward phase: layers
 * above the gate see only the kept tokens and never create KV for the rest):
 *     x_kept[m] = x[kept_idx[m]],  scores_kept[m] = scores[kept_idx[m]],
 *     pos_kept[m] = kept_idx[m] - cu_seqlens[seq(m)]   (original position).
 *   x             [device] residual rows as in tg_gate_score
 *   scores        [device] fp32 per token (may be NULL: then scores_kept must be NULL)
 *   kept_idx      [device] n_kept_total int32 global indices
 *   cu_seqlens, cu_kept   [device] S+1 int32
 *   x_kept        [device, out] n_kept_total x d_model, dense rows, x_dtype
 *   scores_kept   [device, out] n_kept_total fp32 (or NULL)
 *   pos_kept      [device, out] n_kept_total int32 (or NULL)
 * Bit-exact copy.  Requirements as tg_gate_score for x.
 */
int tg_gather_kept(const void* x, int32_t x_dtype, int32_t d_model, int64_t x_row_stride,
                   const float* scores, const int32_t* kept_idx, int64_t n_kept_total,
                   int32_t n_seqs, const int32_t* cu_seqlens, const int32_t* cu_kept,
                   void* x_kept, float* scores_kept, int32_t* pos_kept, void* stream);

/*
 * The front half of the gated layer in one call: tg_gate_score, then
 * tg_topk_select on those scores, then tg_gather_kept (spke.com article,
 * gate-module and pruned-forward phases), after all three argument sets are
 * validated (nothing is launched if any check fails): the kernels of the
 * three calls back to back on `stream`, except that with bf16 x and the
 * four-launch selector (max_seqlen > 65536) the gate kernel also zeroes the
 * selector's counters, so the selector's clear kernel is not launched (five
 * kernels: gate; histogram, filter, write of the selection; row copy).
 * Results are bit-identical to the three calls made one by one.  The call does no host synchronisation, no
 * allocation and no memset, so a caller can capture it (and the attention
 * after it) into one HIP graph and replay the whole layer as a single launch.
 *   x, x_dtype, n_tokens_total, d_model, x_row_stride, w1, b1, w2, b2, d_hid:
 *                 as for tg_gate_score
 *   n_seqs, max_seqlen, cu_seqlens, doc_begin, doc_end, k_doc, cu_kept:
 *                 as for tg_topk_select
 *   n_kept_total  cu_kept[S] (host value, as for tg_gather_kept)
 *   scores        [device, out] n_tokens_total fp32
 *   kept_idx      [device, out] n_kept_total int32
 *   x_kept, scores_kept, pos_kept   [device, out] as for tg_gather_kept
 *   workspace     [device] >= tg_topk_workspace_bytes(...) bytes, 256-B aligned
 * Requirements and errors: those of the three calls.
 */
int tg_gated_select(const void* x, int32_t x_dtype, int64_t n_tokens_total, int32_t d_model,
                    int64_t x_row_stride, const void* w1, const float* b1, const float* w2, float b2,
                    int32_t d_hid, int32_t n_seqs, int32_t max_seqlen, const int32_t* cu_seqlens,
                    const int32_t* doc_begin, const int32_t* doc_end, const int32_t* k_doc,
                    const int32_t* cu_kept, int64_t n_kept_total, float* scores, int32_t* kept_idx,
                    void* x_kept, float* scores_kept, int32_t* pos_kept, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes tg_keybias_attn_prefill (and tg_attn_prepare / tg_attn_forward)
 * need for these sizes: the kept-only cache, plus, for 1024 or more kept
 * tokens with ceil(n_kept_total / 64) * n_kv_heads <= 512, the forward's
 * key-split scratch (512 tickets and 512 partial slots of 256 (D/2 + 2)
 * floats: 34.6 MB for D = 128, 17.8 MB for D = 64), plus a 256-B header in
 * which the pre-pass records what it prepared. */
size_t tg_attn_workspace_bytes(int32_t n_seqs, int64_t n_kept_total, int32_t n_kv_heads,
                               int32_t head_dim);

/*
 * Token-gated causal GQA attention over the kept tokens (spke.com article,
 * section on token-gated attention: every kept token's gate score is added as
 * a bias to the attention logits of the layers above the gate, scaled by a
 * learnable per-head gain, with a learnable temperature).  Formula used
 * (the pages do not print one):
 *     l_ij = <R(q_i,pos_i), R(k_j,pos_j)> / (sqrt(D) * tau) + head_gain[h] * key_score[j]
 * over keys j of the same sequence with pos_j <= pos_i; O_i = softmax_j(l_ij) V;
 * lse[h][i] = log sum_j exp(l_ij).  q head h reads kv head h / (Hq / Hkv).
 * R is rotary embedding on original positions (rotate-half pairing (m, m+D/2),
 * angle pos * rope_base^(-2m/D), angles reduced in fp64); rope_base <= 0
 * disables it.  bf16 MFMA with fp32 accumulation and fp32 online softmax.
 * Accuracy: the rotated q, scaled by log2(e) / (sqrt(D) tau), and the rotated
 * k are rounded to bf16 (2^-9 relative) before the MFMAs, so a logit is off by
 * about 2^-9 of its q.k term, which grows as 1/tau.  For q and k of unit-scale
 * entries (the synthetic workloads: N(0,1), D = 64 or 128) O and lse stay
 * within 2e-2 of the exact (fp64) result for tau >= 0.7 (about 0.01 at
 * tau = 0.9); below that the error grows as 1/tau (0.032 at tau = 0.3).
 *   q             [device] bf16, token m head h at q + m*q_row_stride + h*D
 *   k, v          [device] bf16, token m kv head g at k + m*kv_row_stride + g*D
 *   key_score     [device] n_kept_total fp32 (the kept tokens' gate scores)
 *   head_gain     [device] n_q_heads fp32
 *   tau           temperature > 0, finite
 *   pos           [device] n_kept_total int32 original positions, strictly
 *                 increasing within each sequence (tg_gather_kept output is)
 *   cu_kept       [device] S+1 int32 prefix offsets of the kept sequences
 *   max_kept_seqlen  host upper bound of max_s M_s (sizes the grid)
 *   out           [device, out] bf16 n_kept_total x n_q_heads x D, dense
 *   lse           [device, out] fp32 n_q_heads x n_kept_total, or NULL
 *   workspace     [device] >= tg_attn_workspace_bytes(...) bytes, 256-B aligned
 * Requirements: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0 and the
 * group size Hq/Hkv in {1, 2, 4, 8}; q_row_stride >= Hq*D, kv_row_stride >=
 * Hkv*D, both multiples of 8; q, k, v 16-byte aligned.
 */
int tg_keybias_attn_prefill(const void* q, const void* k, const void* v, int64_t q_row_stride,
                            int64_t kv_row_stride, const float* key_score, const float* head_gain,
                            float tau, const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs,
                            int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, double rope_base, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of tg_keybias_attn_prefill, for callers that keep the kept
 * tokens' keys and values for several query passes, or time the attention
 * kernel alone.  Calling tg_attn_prepare then tg_attn_forward on one stream
 * gives bit-identical results to tg_keybias_attn_prefill (same kernels).
 *
 * tg_attn_prepare writes the kept-only key/value cache into `workspace`
 * (spke.com article, pruned-forward phase: layers above the gate hold keys
 * and values for the kept tokens only, and the token-gated attention section:
 * the key's gate score is its bias).  Per kv head it stores the keys rotated
 * on their original positions with the gate score folded into extra columns,
 * the values transposed, and per kept token the rotary cos/sin table that the
 * forward pass applies to the queries.  Arguments and requirements as for
 * tg_keybias_attn_prefill (k, v, kv_row_stride, key_score, pos, cu_kept,
 * n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base, workspace).
 */
int tg_attn_prepare(const void* k, const void* v, int64_t kv_row_stride, const float* key_score,
                    const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs, int64_t n_kept_total,
                    int32_t n_kv_heads, int32_t head_dim, double rope_base, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * tg_attn_forward runs the token-gated attention of tg_keybias_attn_prefill
 * over a workspace filled by tg_attn_prepare (q, q_row_stride, head_gain, tau,
 * max_kept_seqlen, n_q_heads, out, lse as there).  cu_kept, n_seqs,
 * n_kept_total, n_kv_heads, head_dim and rope_base must equal those of the
 * tg_attn_prepare call that filled the workspace, and that call must precede
 * this one in stream order; otherwise the results are undefined.  The cache
 * is only read.  A grid of at most two workgroups per CU may cut its long
 * query tiles into key chunks whose partials go to the workspace's key-split
 * scratch and are merged by the last chunk to finish; the chunk tickets there
 * are zeroed by tg_attn_prepare and left at zero by every forward.  So
 * forwards that share a workspace must not overlap, and the results are
 * deterministic.
 */
int tg_attn_forward(const void* q, int64_t q_row_stride, const float* head_gain, float tau,
                    const int32_t* cu_kept, int32_t n_seqs, int64_t n_kept_total,
                    int32_t max_kept_seqlen, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    double rope_base, void* out, float* lse, const void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes tg_attn_decode needs for its per-split partials. */
size_t tg_attn_decode_workspace_bytes(int32_t n_seqs, int32_t max_kept_seqlen, int32_t n_q_heads,
                                      int32_t head_dim);

/*
 * One decode step of token-gated attention over the kept-only cache that
 * tg_attn_prepare wrote (spke.com article, pruned-forward phase: above the
 * gate only kept tokens have keys and values; token-gated attention section:
 * each kept key keeps its gate-score bias).  The pages do not describe
 * decoding; this is the prefill logit for one new query per sequence:
 *     l_j = <R(q_s, q_pos[s]), R(k_j, pos_j)> / (sqrt(D) * tau) + head_gain[h] * key_score[j]
 * over the kept keys j of sequence s with pos_j <= q_pos[s]; O = softmax_j(l) V,
 * lse[h][s] = log sum_j exp(l_j).  The new token's own key is attended only
 * if the caller placed it in the cache.  A query that sees no key gets O = 0
 * and lse = -inf.  fp32 logits, probabilities and sums (no bf16 rounding of
 * q or P); the keys and values are the cache's bf16.
 *   q             [device] bf16, sequence s head h at q + s*q_row_stride + h*D
 *   q_pos         [device] n_seqs int32 original position of each new query
 *   head_gain, tau  as for tg_keybias_attn_prefill
 *   pos           [device] n_kept_total int32: the kept positions the cache
 *                 was prepared with
 *   cu_kept, n_seqs, n_kept_total, n_kv_heads, head_dim, rope_base: those of
 *                 the tg_attn_prepare call that filled `cache` (which must
 *                 precede this call in stream order; the cache is only read)
 *   max_kept_seqlen  host upper bound of max_s M_s
 *   cache         [device] that tg_attn_prepare workspace, cache_bytes >=
 *                 tg_attn_workspace_bytes(n_seqs, n_kept_total, n_kv_heads, head_dim)
 *   out           [device, out] bf16 n_seqs x n_q_heads x D, dense
 *   lse           [device, out] fp32 n_q_heads x n_seqs, or NULL
 *   workspace     [device] >= tg_attn_decode_workspace_bytes(...) bytes, 256-B
 *                 aligned, overwritten
 * Requirements: head_dim in {64, 128}; group size Hq/Hkv in {1, 2, 4, 8};
 * q_row_stride >= Hq*D.  Errors as for the prefill; nothing is launched
 * unless every check passes.
 */
int tg_attn_decode(const void* q, int64_t q_row_stride, const int32_t* q_pos, const float* head_gain,
                   float tau, const int32_t* pos, const int32_t* cu_kept, int32_t n_seqs,
                   int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, double rope_base, const void* cache, size_t cache_bytes, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes tg_attn_gate_grads needs: the prepared queries and dL/dO
 * rows (2 Hq rows of D+16 bf16 per padded kept row) plus four fp32 per q head
 * and kept token (column sums of up to four query ranges) and a few
 * per-block partials. */
size_t tg_attn_gate_grads_workspace_bytes(int32_t n_seqs, int64_t n_kept_total, int32_t max_kept_seqlen,
                                          int32_t n_q_heads, int32_t head_dim);

/*
 * Gate-side gradients of token-gated attention (spke.com article, section on
 * token-gated attention: the per-head gain and the temperature are learned,
 * and the score bias is how the loss reaches the gate's scores in training).
 * With the logit of tg_keybias_attn_prefill, P = softmax_j(l), dO = dL/dO and
 *     dS_ij = P_ij (<dO_i, v_j> - <dO_i, O_i>)      (= dL/dl_ij),
 * this writes
 *     d_score[j] = sum_h head_gain[h] sum_i dS_hij
 *     d_gain[h]  = sum_ij key_score[j] dS_hij
 *     d_tau[0]   = -(1/tau) sum_hij dS_hij <R(q_i), R(k_j)> / (sqrt(D) tau)
 * (sums over each sequence's causal pairs).  P is recomputed from the
 * forward's lse; the q.k logits run on bf16 MFMA as in the forward, and
 * every sum is fp32.  Deterministic: no atomics.  When the kept keys give
 * fewer key blocks than the GPU has CUs, each block's query rows are cut
 * into up to four ranges (a dispatch model picks the count), and the ranges'
 * partial sums are added in a fixed order.
 *   q, q_row_stride       the forward's queries
 *   v, kv_row_stride      the values tg_attn_prepare was given (kv head hk of
 *                         token m at v + m*kv_row_stride + hk*D)
 *   key_score, head_gain, tau, cu_kept, n_seqs, n_kept_total, max_kept_seqlen,
 *   n_q_heads, n_kv_heads, head_dim, rope_base: those of the forward
 *   out           [device] bf16 n_kept_total x n_q_heads x D: the forward's O
 *   lse           [device] fp32 n_q_heads x n_kept_total: the forward's lse
 *   d_out         [device] bf16 dL/dO, token m head h at d_out + m*d_out_row_stride + h*D
 *   cache         [device] the workspace tg_attn_prepare filled for this
 *                 forward (read only), cache_bytes >= tg_attn_workspace_bytes(...)
 *   d_score       [device, out] fp32 n_kept_total
 *   d_gain        [device, out] fp32 n_q_heads
 *   d_tau         [device, out] fp32 1
 *   workspace     [device] >= tg_attn_gate_grads_workspace_bytes(...) bytes,
 *                 256-B aligned, overwritten
 * Requirements as for the prefill, and d_out_row_stride >= Hq*D, a multiple of
 * 8; out, d_out and v 16-B aligned.  With no kept token d_gain and d_tau are
 * set to zero.  Errors as for the prefill; nothing is launched unless every
 * check passes.
 */
int tg_attn_gate_grads(const void* q, int64_t q_row_stride, const void* v, int64_t kv_row_stride,
                       const float* key_score, const float* head_gain, float tau, const int32_t* cu_kept,
                       int32_t n_seqs, int64_t n_kept_total, int32_t max_kept_seqlen, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, double rope_base, const void* out,
                       const float* lse, const void* d_out, int64_t d_out_row_stride, const void* cache,
                       size_t cache_bytes, float* d_score, float* d_gain, float* d_tau, void* workspace,
                       size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
