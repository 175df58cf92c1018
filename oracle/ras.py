"""CPU oracle for KVzip reconstruction-attention scoring, selection, compaction.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Everything here is the plain definition, written out in float64 (numpy), with
no online softmax, no tiling of the key axis and no fusion.  Query rows are
processed a block at a time only to bound memory; every row is the full dense
softmax over its visible keys.

Sources (page titles and sections; no line numbers):

* [blog]      "KVzip: Query-Agnostic KV Cache Compression with Context
              Reconstruction", jjl357 blog post: section 4.1 (method overview,
              steps 1-5), 4.3.1 (reconstruction attention), 4.3.2 (importance
              score as a max over g and i), 4.5.1 (chunked scoring and the
              merge of per-chunk scores).
* [rebuttal]  paperhub.cn OpenReview rebuttals by the authors: the answer on
              positional OOD (each chunk's positions continue after the whole
              prefilled context, so every chunk attends to the full cache), the
              answer on head-level scores (S has shape L x H x n_c), the answer
              on max versus average aggregation, the computational analysis
              (2x prefill attention FLOPs).
* [atlas]     atlas.scime.ai summary, "Approach" (evict the lowest-scoring pairs
              once per context) and "Measured effects" (non-uniform head
              budgets help).

Readings taken where the pages are silent or garbled (each is listed again in
the design notes):

* softmax scale 1/sqrt(d) applied to the exact dot product (the blog's formula
  prints no scale); the caller passes ``scale``;
* key set of a chunk's query rows: all n_c context keys, then the chunk's own
  keys (repeat prompt + copied context) under one causal mask, row i seeing
  in-chunk keys 0..i;
* only context keys are scored; the in-chunk keys enter the normaliser only;
* chunk scores merge by a running max (the chunks partition the query set of
  the max in [blog] 4.3.2);
* selection keeps exactly K = round-half-up(r * N) entries, ordered by score
  descending and then by flat index (l*H + h)*n_c + j ascending;
* the packed output holds heads in flat order and rows in ascending j.

Pins of this oracle against facts other than itself live in
tests/test_oracle_pins.py.  Every function below is pinned there.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# exact input conversion
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly (a bf16 is the top half
    of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    """Storage array ('bf16' bit patterns or 'f32' floats) to float64."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# reconstruction attention of one chunk  ([blog] 4.3.1, 4.3.2, 4.5.1)
# ---------------------------------------------------------------------------

def chunk_probabilities(q_g, k_ctx_h, k_in_h, scale, rows=None):
    """Dense softmax rows of one query head over its visible keys.

    q_g: [n_in][d] float64 queries (repeat prompt rows first, then the chunk).
    k_ctx_h: [n_c][d] context keys; k_in_h: [n_in][d] in-chunk keys.
    Returns P: [len(rows)][n_c + n_in] float64 where row i's entries on
    in-chunk keys t > i are exactly 0 (causal), and every row sums to 1.
    """
    n_in = q_g.shape[0]
    n_c = k_ctx_h.shape[0]
    if rows is None:
        rows = np.arange(n_in)
    rows = np.asarray(rows)
    keys = np.concatenate([k_ctx_h, k_in_h], axis=0)          # [n_c + n_in][d]
    logits = (q_g[rows] @ keys.T) * scale                      # [r][n_c + n_in]
    t = np.arange(n_in)
    invisible = t[None, :] > rows[:, None]                    # causal in-chunk mask
    logits[:, n_c:][invisible] = -np.inf
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    return e / e.sum(axis=1, keepdims=True)


def score_chunk(q, k_ctx, k_in, scale, S, row_block=256, mode="max"):
    """Fold one reconstruction chunk into the running scores of one layer.

    q: [H][G][n_in][d], k_ctx: [H][n_c][d], k_in: [H][n_in][d], all float64.
    S: [H][n_c] float64, updated in place, for context keys j only:
      mode "max" (the method, [blog] 4.3.2):
          S[h, j] = max(S[h, j], max over g and rows i of P_{h,g}[i, j]);
      mode "sum" (the aggregation the [rebuttal] answer on average
          aggregation compares against; sum and mean rank keys alike):
          S[h, j] += sum over g and rows i of P_{h,g}[i, j];
      mode "raw" (the no-softmax ablation, [blog] 5.5.5 and [atlas] Measured
          effects): S[h, j] = max(S[h, j], max over g, i of scale * q . k_j),
          the unnormalised logit (start S at -inf).
    Returns S.
    """
    H, G, n_in, _ = q.shape
    n_c = k_ctx.shape[1]
    for h in range(H):
        for g in range(G):
            for r0 in range(0, n_in, row_block):
                rows = np.arange(r0, min(n_in, r0 + row_block))
                if mode == "raw":
                    x = (q[h, g][rows] @ k_ctx[h].T) * scale
                    np.maximum(S[h], x.max(axis=0), out=S[h])
                    continue
                P = chunk_probabilities(q[h, g], k_ctx[h], k_in[h], scale, rows)
                if mode == "max":
                    np.maximum(S[h], P[:, :n_c].max(axis=0), out=S[h])
                elif mode == "sum":
                    S[h] += P[:, :n_c].sum(axis=0)
                else:
                    raise ValueError(mode)
    return S


def chunk_attention_output(q, k_ctx, k_in, v_ctx, v_in, scale, row_block=256):
    """Output of the reconstruction attention of one chunk: every query row's
    softmax over its visible keys applied to their values.

    The scoring stage is a full forward of the model over [repeat prompt;
    chunk] ([rebuttal] computational analysis: one MLP pass and two times the
    prefill's attention work), so each layer's attention also produces
    O = P [V_c ; V_in] for the layer above; a FlashAttention kernel returns
    exactly this product and nothing else ([blog] 4.4).

    q: [H][G][n_in][d], k_ctx, v_ctx: [H][n_c][d], k_in, v_in: [H][n_in][d],
    all float64.  Returns O: [H][G][n_in][d] with
    O[h, g, i] = sum_j P_{h,g}[i, j] * [v_ctx[h]; v_in[h]][j].
    """
    H, G, n_in, _ = q.shape
    dv = v_ctx.shape[2]
    O = np.zeros((H, G, n_in, dv))
    for h in range(H):
        vals = np.concatenate([v_ctx[h], v_in[h]], axis=0)      # [n_c + n_in][dv]
        for g in range(G):
            for r0 in range(0, n_in, row_block):
                rows = np.arange(r0, min(n_in, r0 + row_block))
                P = chunk_probabilities(q[h, g], k_ctx[h], k_in[h], scale, rows)
                O[h, g, rows] = P @ vals
    return O


def score_layer(chunks, k_ctx, scale, mode="max"):
    """Scores of one layer from a list of chunks [(q, k_in), ...], S starting
    at 0 (max and sum of probabilities) or -inf (raw logits)."""
    H = k_ctx.shape[0]
    S = np.full((H, k_ctx.shape[1]), -np.inf if mode == "raw" else 0.0)
    for q, k_in in chunks:
        score_chunk(q, k_ctx, k_in, scale, S, mode=mode)
    return S


# ---------------------------------------------------------------------------
# head-level and token-level aggregates of S  ([rebuttal] answer on
# head-level scores: max over the sequence axis of S[L][H][n_c]; [blog] 4.3.3:
# one score per token as the max over layers and heads)
# ---------------------------------------------------------------------------

def head_scores(S2d):
    """[n_heads][n_c] -> [n_heads]: max over the tokens of each head."""
    return np.asarray(S2d).max(axis=1)


def token_scores(S2d):
    """[n_heads][n_c] -> [n_c]: max over all (layer, head) rows per token."""
    return np.asarray(S2d).max(axis=0)


# ---------------------------------------------------------------------------
# global selection  ([blog] 4.1 step 5; [atlas] Approach, Measured effects)
# ---------------------------------------------------------------------------

def keep_count(n_total: int, ratio: float) -> int:
    """K = r * N rounded half up, clamped to [0, N]."""
    k = math.floor(ratio * n_total + 0.5)
    return max(0, min(int(n_total), int(k)))


def select(S_flat, n_heads: int, n_c: int, K: int):
    """Exact top-K over all (l, h, j) entries of the flat score array.

    Order: score descending, then flat index ascending.  Returns
    (mask uint8 [N], head_offsets int64 [n_heads + 1], tau) where tau is the
    K-th largest score (+inf when K == 0).
    """
    S_flat = np.asarray(S_flat)
    N = S_flat.shape[0]
    assert N == n_heads * n_c
    order = np.lexsort((np.arange(N), -S_flat.astype(np.float64)))
    mask = np.zeros(N, np.uint8)
    mask[order[:K]] = 1
    tau = float(S_flat[order[K - 1]]) if K > 0 else math.inf
    budget = mask.reshape(n_heads, n_c).sum(axis=1, dtype=np.int64)
    offsets = np.zeros(n_heads + 1, np.int64)
    offsets[1:] = np.cumsum(budget)
    return mask, offsets, tau


# ---------------------------------------------------------------------------
# structured eviction variants built on the same scores
# ---------------------------------------------------------------------------

def head_evict(S2d, K_heads: int, n_sink: int, n_recent: int):
    """Context-independent head-level eviction ([rebuttal] answer on how the
    head-level scores were computed: a head's score is the max of S along the
    sequence axis; [blog] 5.4: KVzip's scores drive head-level eviction in
    place of DuoAttention's optimised head scores).

    The K_heads heads with the highest head scores keep every token; ties go
    to the lower flat head index (the order of select()).  The pages do not
    say what an evicted head keeps; here, as for DuoAttention's streaming
    heads, it keeps its first n_sink and its last n_recent tokens.
    Returns (mask uint8 [N], head_offsets int64 [n_heads + 1],
    head_keep uint8 [n_heads])."""
    S2d = np.asarray(S2d)
    n_heads, n_c = S2d.shape
    head_keep, _, _ = select(head_scores(S2d), 1, n_heads, K_heads)
    j = np.arange(n_c)
    window = (j < n_sink) | (j >= n_c - n_recent)
    mask = np.where(head_keep[:, None] == 1, True, window[None, :]).astype(np.uint8)
    budget = mask.sum(axis=1, dtype=np.int64)
    offsets = np.zeros(n_heads + 1, np.int64)
    offsets[1:] = np.cumsum(budget)
    return mask.reshape(-1), offsets, head_keep


def token_evict(S2d, K_tokens: int):
    """Token-level eviction ([blog] 4.3.3: one score per token, the max over
    every layer and head; sorting those scores decides which tokens stay).

    The K_tokens positions with the highest token scores (ties: lower
    position first) are kept in every head.  Returns (mask uint8 [N],
    head_offsets int64 [n_heads + 1], token_keep uint8 [n_c])."""
    S2d = np.asarray(S2d)
    n_heads, n_c = S2d.shape
    token_keep, _, _ = select(token_scores(S2d), 1, n_c, K_tokens)
    mask = np.tile(token_keep, n_heads)
    offsets = np.arange(n_heads + 1, dtype=np.int64) * int(token_keep.sum())
    return mask, offsets, token_keep


# ---------------------------------------------------------------------------
# decode attention over a packed per-head cache  ([abstract] and [atlas] Key
# results: the compressed cache cuts FlashAttention decode latency about 2x;
# [rebuttal] computational analysis: decode attention latency against the
# kept ratio)
# ---------------------------------------------------------------------------

def decode_attention(q, k_out, v_out, head_offsets, scale):
    """One decode token per query head over each KV head's kept rows.

    q: [n_heads][G][d]; k_out, v_out: [K][d] packed rows, head h owning rows
    head_offsets[h]..head_offsets[h+1]; all float64.  Returns
    out[h, g] = softmax(scale * q[h, g] . K_h^T) @ V_h (zeros for an empty head).
    """
    n_heads, G, d = q.shape
    out = np.zeros((n_heads, G, d))
    for h in range(n_heads):
        a, b = int(head_offsets[h]), int(head_offsets[h + 1])
        if b == a:
            continue
        K = k_out[a:b]
        V = v_out[a:b]
        x = (q[h] @ K.T) * scale                       # [G][len]
        x -= x.max(axis=1, keepdims=True)
        p = np.exp(x)
        p /= p.sum(axis=1, keepdims=True)
        out[h] = p @ V
    return out


# ---------------------------------------------------------------------------
# compaction into a packed per-head cache  ([blog] 4.1 step 5;
# [rebuttal] reusable compressed cache for offline compression)
# ---------------------------------------------------------------------------

def compact(k_ctx, v_ctx, mask, head_offsets):
    """Gather the kept rows, heads in flat order, rows in ascending position.

    k_ctx, v_ctx: [n_heads][n_c][d] in their storage type (copied bit-exactly).
    mask: [n_heads * n_c] uint8.  Returns (k_out, v_out, idx) with
    k_out[head_offsets[h] + r] = k_ctx[h, j_r] for the r-th kept j of head h.
    """
    n_heads, n_c = k_ctx.shape[0], k_ctx.shape[1]
    m = np.asarray(mask).reshape(n_heads, n_c).astype(bool)
    total = int(head_offsets[-1])
    k_out = np.empty((total,) + k_ctx.shape[2:], k_ctx.dtype)
    v_out = np.empty((total,) + v_ctx.shape[2:], v_ctx.dtype)
    idx = np.empty(total, np.int32)
    for h in range(n_heads):
        js = np.nonzero(m[h])[0]
        o = int(head_offsets[h])
        assert o + len(js) == int(head_offsets[h + 1])
        k_out[o:o + len(js)] = k_ctx[h, js]
        v_out[o:o + len(js)] = v_ctx[h, js]
        idx[o:o + len(js)] = js
    return k_out, v_out, idx
