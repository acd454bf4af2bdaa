"""The block predictor's arithmetic, written from its definition (test infrastructure only).

Sources: the ``predictor.rs`` page -- its module doc (Q @ P, K @ P for every
token of a block, and a block score that is the max over query heads and tokens
of the projected dot product, used only to rank eviction victims), the layout
comments on ``a_g_bytes`` and the ``Predictor`` fields, ``project_q``,
``project_kv_block`` and ``score_blocks``; and the ``qsa_select.rs`` page's
host top-k for the rule "lower index on ties".

Notation: L layers, Hq query heads, Hk kv heads, g = Hq / Hk, D head_dim, R rank,
B block_size, N max_blocks; S sequences, n blocks per sequence, M query rows.
All arrays are row-major.  bf16 tensors are uint16 bit patterns.

Readings where the pages leave a step open:

* accumulation: products and sums in float64, one RNE rounding to bf16;
* GQA: query head h reads kv head floor(h / g);
* several query rows: the score is also maximised over rows, with no causal mask;
* scores carry no 1/sqrt(D) scale (the score kernel takes no scale argument);
* scores and ranks are indexed by a block's *logical* position in its sequence's
  block table (an absent table is the identity, which is the pages' contiguous
  ``k_lr_seq`` case); ties rank the lower logical index first;
* every one of a block's B tokens is scored (the pages pass no fill length);
  the masked variant scores only the first ``last_fill[s]`` tokens of a
  sequence's last block (fill 0: -inf);
* ranking key: -0 is +0, every NaN ranks first;
* per-row keep sets (the qsa_select.rs page's prefill selection, rebuilt on the
  predictor's score): a row at position p sees blocks ``b < (p + 1) // B`` (the
  block size is the page's ratio), scores the rest -inf, keeps the top-k by
  descending score with the lower index first on ties; NaN goes last, and a row
  with fewer than k complete blocks pads its list with -1.
"""

import numpy as np

from . import bf16


# ---------------------------------------------------------------- projections

def project(x_bits, p_bits):
    """``bf16(x @ P)`` for bf16 ``x [..., D]`` and ``P [D, R]``: float64 sums, one rounding.

    ``project_q`` (Q @ P) and ``project_kv_block`` (K @ P per token) are both
    this map; only their layouts differ.
    """
    x = bf16.decode(x_bits)
    p = bf16.decode(p_bits)
    lead = x.shape[:-1]
    y = x.reshape(-1, x.shape[-1]) @ p
    return bf16.encode(y).reshape(*lead, p.shape[1])


def project_q(q_bits, p_bits):
    """``q [..., Hq, D]`` -> ``q_proj [..., Hq, R]`` (``project_q``)."""
    return project(q_bits, p_bits)


def project_kv_slots(k_bits, p_bits):
    """Low-rank keys of whole blocks in A_g slot layout.

    ``k [n, B, Hk, D]`` (the page's ``k_block`` layout, one block per leading
    index) -> ``[n, Hk, B, R]``, the ``[num_kv_heads, block_size, r]`` order an
    A_g slot holds.
    """
    a = project(k_bits, p_bits)            # [n, B, Hk, R]
    return np.ascontiguousarray(a.transpose(0, 2, 1, 3))


def project_kv_block(a_g, layer, k_bits, table, p_bits):
    """Write ``K @ P`` of ``n`` blocks into ``a_g [L, N, Hk, B, R]`` at ``a_g[layer, table[i]]``.

    Out-of-range ``layer`` or table entries raise, as the page's
    ``project_kv_block`` rejects an out-of-range layer or block.
    """
    L, N = a_g.shape[0], a_g.shape[1]
    if not 0 <= layer < L:
        raise IndexError(f"layer {layer} out of range")
    slots = project_kv_slots(k_bits, p_bits)
    for i, phys in enumerate(np.asarray(table).tolist()):
        if not 0 <= phys < N:
            raise IndexError(f"block {phys} out of range")
        a_g[layer, phys] = slots[i]
    return a_g


# ---------------------------------------------------------------------- scores

def score_one(q_rows, slots, last_fill=None):
    """Scores of one (layer, sequence) in float64.

    ``q_rows [M, Hq, R]`` bf16 projected queries; ``slots [n, Hk, B, R]`` bf16
    low-rank keys of the sequence's blocks in logical order.  Returns ``[n]``:
    ``max over i < M, h < Hq, t < B of sum_j q[i, h, j] * A[b, h // g, t, j]``.
    With ``last_fill`` the last block (b = n - 1) holds only its first
    ``last_fill`` tokens and the max runs over those (-inf when there are none).
    """
    if last_fill is not None and len(slots):
        out = score_one(q_rows, slots)
        f = max(0, min(int(last_fill), slots.shape[2]))
        out[-1] = score_one(q_rows, slots[-1:, :, :f])[0] if f else -np.inf
        return out
    q = bf16.decode(q_rows)
    M, Hq, R = q.shape
    n, Hk, B, _ = slots.shape
    g = Hq // Hk
    out = np.full(n, -np.inf)
    # bound the size of each logits matrix (M*g rows x chunk*B columns)
    chunk = max(1, min(n, (1 << 24) // max(1, M * g * B)))
    for b0 in range(0, n, chunk):
        a = bf16.decode(slots[b0:b0 + chunk])          # [c, Hk, B, R]
        c = a.shape[0]
        for k in range(Hk):
            qk = q[:, k * g:(k + 1) * g, :].reshape(M * g, R)
            ak = a[:, k].reshape(c * B, R)
            logits = qk @ ak.T                          # [M*g, c*B]
            best = logits.max(axis=0).reshape(c, B).max(axis=1)
            out[b0:b0 + c] = np.maximum(out[b0:b0 + c], best)
    return out


def score_blocks(q_proj, a_g, layer0, tables, n_blocks, last_fill=None):
    """``score_blocks`` for ``n_layers`` layers and ``S`` sequences, float64.

    ``q_proj [n_layers, S, M, Hq, R]`` bf16; ``a_g [L, N, Hk, B, R]`` bf16;
    ``tables [S, n_blocks]`` int physical ids, or None for the identity (the
    pages' contiguous slots ``0..n-1``); ``last_fill [S]`` tokens held by each
    sequence's last block, or None for full blocks.  Returns ``[n_layers, S, n_blocks]``.
    """
    n_layers, S = q_proj.shape[0], q_proj.shape[1]
    out = np.empty((n_layers, S, n_blocks))
    for l in range(n_layers):
        for s in range(S):
            ids = np.arange(n_blocks) if tables is None else np.asarray(tables[s])[:n_blocks]
            fill = None if last_fill is None else last_fill[s]
            out[l, s] = score_one(q_proj[l, s], a_g[layer0 + l][ids], fill)
    return out


# ---------------------------------------------------------------------- ranking

def order_key(scores_f32):
    """Totally ordered uint32 key of float32 scores (ascending key = ascending score).

    -0 counts as +0; any NaN gets key 0 so it ranks first.
    """
    s = np.asarray(scores_f32, dtype=np.float32)
    u = s.view(np.uint32).astype(np.uint64)
    u = np.where(u == 0x80000000, 0, u)                  # -0 -> +0
    neg = (u >> 31) == 1
    key = np.where(neg, u ^ 0xFFFFFFFF, u ^ 0x80000000)
    key = np.where(np.isnan(s), 0, key)
    return key.astype(np.uint32)


def rank_victims(scores_f32):
    """Eviction order of each row of ``scores [G, n]``: ascending score, lower index first on ties.

    Returns int32 logical block indices ``[G, n]``; element 0 of a row is the
    first victim.
    """
    s = np.atleast_2d(np.asarray(scores_f32, dtype=np.float32))
    keys = order_key(s)
    return np.argsort(keys, axis=1, kind="stable").astype(np.int32)


def select_victims(scores, k):
    """The k lowest-scored blocks of every row in eviction order: by definition the
    first k entries of ``rank_victims`` (the predictor page's module doc: scores only
    rank eviction victims; a cache evicts a few blocks at a time)."""
    return rank_victims(scores)[:, :k]


# ------------------------------------------------- per-row causal keep sets

def complete_blocks(first_pos, row, ratio, limit):
    """Blocks complete at position ``first_pos + row``: ``(first_pos + row + 1) // ratio``,
    at most ``limit`` (the qsa_select.rs page's per-row count in its prefill selection)."""
    return min(limit, (first_pos + row + 1) // ratio)


def score_rows(q_rows, slots, first_pos, stride):
    """Per-row causal block scores of one layer and sequence, float64.

    ``q_rows [rows, Hq, R]`` bf16, row i at position ``first_pos + i``; ``slots
    [n, Hk, B, R]`` bf16 low-rank keys of the sequence's blocks in logical order.
    Returns ``[rows, stride]``: for ``b < complete(i) = min(n, (first_pos + i + 1) // B)``
    the predictor's score of block b for row i alone (max over query heads h and
    tokens t of ``q[i, h] . A[b, h // g, t]``), and -inf for the other columns
    (qsa_select.rs page: each row sees only the blocks complete at its position;
    the block size plays the page's ratio).
    """
    q = bf16.decode(q_rows)
    rows, Hq, R = q.shape
    n, Hk, B, _ = slots.shape
    g = Hq // Hk
    best = np.full((rows, n), -np.inf)
    chunk = max(1, min(n, (1 << 24) // max(1, rows * B)))   # logits of at most 2^24 entries
    for b0 in range(0, n, chunk):
        a = bf16.decode(slots[b0:b0 + chunk])                # [c, Hk, B, R]
        c = a.shape[0]
        for h in range(Hq):
            ak = a[:, h // g].reshape(c * B, R)
            logits = q[:, h, :] @ ak.T                       # [rows, c*B]
            per_block = logits.reshape(rows, c, B).max(axis=2)
            best[:, b0:b0 + c] = np.maximum(best[:, b0:b0 + c], per_block)
    out = np.full((rows, stride), -np.inf)
    for i in range(rows):
        c = complete_blocks(first_pos, i, B, min(n, stride))
        out[i, :c] = best[i, :c]
    return out


def keep_sets(scores_f32, first_pos, ratio, topk):
    """Per-row keep lists (qsa_select.rs page, prefill selection's host top-k).

    For row i of ``scores [rows, stride]`` (float32) the first
    ``complete(i) = min(stride, (first_pos + i + 1) // ratio)`` scores are ordered
    larger first, equal scores by lower index; the first ``topk`` indices are the
    row's keep list, and slots past ``complete(i)`` hold -1.  -0 equals +0; NaN
    (which the page's comparator leaves unordered) goes after every number.
    Returns int32 ``[rows, topk]``.
    """
    s = np.atleast_2d(np.asarray(scores_f32, dtype=np.float32))
    rows, stride = s.shape
    out = np.full((rows, topk), -1, np.int32)
    for i in range(rows):
        c = complete_blocks(first_pos, i, ratio, stride)
        v = s[i, :c].astype(np.float64)
        nan = np.isnan(v)
        neg = np.where(nan, 0.0, -v) + 0.0                   # descending; -0 and +0 become one key
        order = np.lexsort((np.arange(c), neg, nan))         # last key is the primary one
        m = min(topk, c)
        out[i, :m] = order[:m]
    return out
