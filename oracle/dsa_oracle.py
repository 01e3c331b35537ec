"""Plain fp64 CPU oracle for content-aware dynamic block-sparse causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or calls this module.  Only the tests, the
``smoke()`` check and the ``cpu_baseline`` leg of ``bench.py`` may use it.  It
shares no code, table or helper with the HIP path; it takes plain numpy arrays
(the same bf16 values the GPU receives, upcast exactly to float64).

What it computes, step by step, in the order the method runs:

  O1 ``block_means``   mean of each b-row tile of Q (and of K).
  O2 ``block_scores``  score of every causal KV block per query block: the dot
                        product of the two tile means times 1/sqrt(d); for
                        grouped-query attention the max over the group's heads.
  O3 ``select_row`` /  keep the k best-scoring blocks per query block, with the
     ``select_topk``   sink block 0 and the diagonal block always kept.
  O4 ``attend``        softmax(s * q k^T) v over exactly the keys of the kept
                        blocks that are causally visible to each row.
  ``prefill`` / ``decode`` chain O1-O4.
  O5 ``attend_backward`` dQ, dK, dV of O4 with the selection held fixed (the
                        chain rule through O4's own definition, row by row).

Sources (the pages; cited by title and section):
  [ZB]  dynamic sparse attention explainer, zblog.xzdbk.com/559.html --
        sections "基于Top-k选择的局部-全局混合" (per query keep the k
        highest-scoring keys, zero the rest; global tokens + local window),
        "硬件友好的稀疏计算实现" / "工程实践建议" (decide per 64x64 or 128x128
        block), "动态开销与计算收益的权衡" (precompute the sparse index at
        cache time), "前沿方向" (GQA/MQA share the KV cache and its index).
  [SvF] "稀疏注意力 vs Flash Attention v2：3 种长序列场景下的推理延迟与精度对比",
        section 1 (content-aware sparsity picks the top-k keys by query-key
        similarity; the ``sparse_attention`` pseudo-code: logits q k^T, apply
        the pattern, softmax of logits / sqrt(d_k), weights times values).
  [NSA] DeepSeek NSA article, pnsm.cn/news/1939904.html -- section 2.2
        (routing scores in fp32, weighted sum in bf16).

Readings where the pages leave a point open (all listed in the design doc):
  * block statistic = mean(Q tile) . mean(K tile) / sqrt(d) (the workload
    definition); a ragged last tile is averaged over its real rows;
  * k counts the forced blocks; a row with fewer visible blocks than k keeps
    them all; exact score ties go to the lower block index;
  * fractional budget k_r = ceil(num * n_r / den) in integer arithmetic;
  * decode: the new token is the last cache position, so every cached key is
    visible; the forced "diagonal" block is the last block;
  * query head h reads KV head floor(h / G);
  * backward: the selection is a discrete choice and is held constant; dK and
    dV of a KV head sum the contributions of its G query heads.

Parity status: every function here is pinned by tests in ``tests/`` that do
not re-use this module's formulas (dense special case against a library
attention routine, brute-force subset enumeration, scalar loops, closed forms,
invariants).  No function is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

FORCE_SINK = 1  # keep block 0 in every row
FORCE_DIAG = 2  # keep the row's own (diagonal / last visible) block

# near-tie rule for flagging rows (see ``near``)
TIE_REL = 1e-3
TIE_ABS = 1e-6


def n_blocks(n: int, block: int) -> int:
    """Number of blocks covering n positions (the last one may be ragged)."""
    return -(-n // block)


# --------------------------------------------------------------------------
# O1 -- block mean pooling
# --------------------------------------------------------------------------
def block_means(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over each run of ``block`` consecutive rows.

    x: [..., N, d].  Returns float64 [..., ceil(N / block), d].  A ragged last
    block is averaged over the rows it really has.

    [ZB] "硬件友好的稀疏计算实现": the decision is made per fixed-size block;
    the block summary is the tile mean named by the workload definition.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-2]
    nb = n_blocks(n, block)
    out = np.empty(x.shape[:-2] + (nb, x.shape[-1]), dtype=np.float64)
    for j in range(nb):
        rows = x[..., j * block : min(n, (j + 1) * block), :]
        out[..., j, :] = rows.sum(axis=-2) / rows.shape[-2]
    return out


# --------------------------------------------------------------------------
# O2 -- block scores
# --------------------------------------------------------------------------
def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """Causal block-score matrix per KV head.

    qbar: [B, Hq, nB, d]; kbar: [B, Hkv, nB, d].  Query head h reads KV head
    h // G with G = Hq / Hkv.  Returns [B, Hkv, nB, nB] float64 with

        S[b, g, i, j] = max over h in group g of  scale * <qbar[b,h,i], kbar[b,g,j]>

    for j <= i and -inf for j > i (a block after the query block is never
    visible under the causal rule).

    [SvF] section 1: content-aware sparsity ranks keys by query-key
    similarity.  [ZB] "前沿方向": a GQA group shares one KV cache, so one
    selection per group; the group's heads are merged with max.
    """
    B, Hq, nB, d = qbar.shape
    Hkv = kbar.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((B, Hkv, nB, nB), -np.inf, dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            per_head = []
            for h in range(g * G, (g + 1) * G):
                per_head.append(scale * (qbar[b, h] @ kbar[b, g].T))  # [nB, nB]
            s = np.max(np.stack(per_head), axis=0)
            for i in range(nB):
                out[b, g, i, : i + 1] = s[i, : i + 1]
    return out


# --------------------------------------------------------------------------
# O3 -- top-k selection with forced blocks
# --------------------------------------------------------------------------
def row_budget(n_visible: int, topk: int, num: int, den: int, n_forced: int) -> int:
    """Number of blocks a row keeps, forced blocks included.

    Fixed k (topk > 0) or the fraction k = ceil(num * n_visible / den) computed
    in integers; raised to the number of forced blocks and capped at the number
    of visible blocks (a row cannot keep more blocks than it can see).
    """
    if topk > 0:
        k = topk
    else:
        k = (num * n_visible + den - 1) // den
    return min(max(k, n_forced), n_visible)


def forced_set(n_visible: int, flags: int) -> list[int]:
    """Blocks kept regardless of score: the sink (block 0) and the row's own
    block (the last visible one).

    [ZB] "基于Top-k选择的局部-全局混合": global tokens plus a local window;
    [SvF] section 1 hybrid mode: local window plus periodic global anchors.
    """
    f = set()
    if flags & FORCE_SINK:
        f.add(0)
    if flags & FORCE_DIAG:
        f.add(n_visible - 1)
    return sorted(f)


def near(a: float, b: float) -> bool:
    """Near-tie test between two scores: relative gap below 1e-3 (the
    acceptance rule), or an absolute gap below 1e-6, which bounds the fp32
    rounding of a block score for the synthetic workloads."""
    if a == b:
        return True
    if not (math.isfinite(a) and math.isfinite(b)):
        return False
    gap = abs(a - b)
    return gap < TIE_REL * max(abs(a), abs(b)) or gap < TIE_ABS


@dataclass
class RowSelection:
    """Selection of one row and what another correct selection may differ in.

    ``idx``: the kept blocks, ascending.  ``forced``: blocks kept regardless.
    ``must``: candidates any accepted set contains.  ``band``: near-tie
    candidates of which exactly ``need`` are kept.  Unflagged rows have an
    empty band (the selection is unique)."""

    idx: list
    forced: list
    must: set
    band: set = field(default_factory=set)
    need: int = 0
    flagged: bool = False


def select_row(scores: np.ndarray, n_visible: int, k_budget: int, forced: list) -> RowSelection:
    """Keep ``k_budget`` of the ``n_visible`` blocks of one row.

    The forced blocks are kept; the remaining m = k_budget - |forced| are the
    highest-scoring candidates, ordered by (score descending, index
    ascending).  [ZB] "基于Top-k选择的局部-全局混合": per query keep the
    k highest-scoring keys and drop the rest.

    A row is flagged when the m-th and (m+1)-th candidates are near-ties
    (``near``); its band holds the ranks from the first to the last candidate
    near either of those two scores.
    """
    fs = set(forced)
    cand = np.array([j for j in range(n_visible) if j not in fs], dtype=np.int64)
    m = k_budget - len(forced)
    if cand.size == 0 or m <= 0:
        return RowSelection(idx=sorted(fs), forced=sorted(fs), must=set())
    sc = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -sc))  # primary: score descending; ties: lower index
    ranked = cand[order]
    rsc = sc[order]
    chosen = set(int(j) for j in ranked[:m])
    sel = sorted(fs | chosen)
    if m >= ranked.size or not near(float(rsc[m - 1]), float(rsc[m])):
        return RowSelection(idx=sel, forced=sorted(fs), must=chosen)
    a, b = float(rsc[m - 1]), float(rsc[m])
    in_band = [r for r in range(ranked.size) if near(float(rsc[r]), a) or near(float(rsc[r]), b)]
    lo, hi = min(in_band), max(in_band)
    must = set(int(j) for j in ranked[:lo])
    band = set(int(j) for j in ranked[lo : hi + 1])
    return RowSelection(idx=sel, forced=sorted(fs), must=must, band=band, need=m - lo, flagged=True)


def kmax(n_rows: int, topk: int, num: int, den: int, flags: int, causal: bool, n_cols: int) -> int:
    """Largest per-row budget: the width of the index array."""
    best = 0
    for i in range(n_rows):
        nv = i + 1 if causal else n_cols
        best = max(best, row_budget(nv, topk, num, den, len(forced_set(nv, flags))))
    return best


def select_topk(scores: np.ndarray, topk: int, num: int = 0, den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG,
                causal: bool = True):
    """Row-wise selection over a score array [..., R, C].

    causal=True (prefill): row i sees blocks 0..i.  causal=False (decode):
    every row sees all C blocks.  Returns (idx, cnt, rows) where idx is int32
    [..., R, kmax] ascending and -1 padded, cnt is int32 [..., R] and rows is a
    flat list of ``RowSelection`` in C order.
    """
    lead = scores.shape[:-2]
    R, C = scores.shape[-2:]
    km = kmax(R, topk, num, den, flags, causal, C)
    flat = scores.reshape((-1, R, C))
    idx = np.full((flat.shape[0], R, km), -1, dtype=np.int32)
    cnt = np.zeros((flat.shape[0], R), dtype=np.int32)
    rows = []
    for u in range(flat.shape[0]):
        for i in range(R):
            nv = i + 1 if causal else C
            f = forced_set(nv, flags)
            kb = row_budget(nv, topk, num, den, len(f))
            rs = select_row(flat[u, i, :nv], nv, kb, f)
            idx[u, i, : len(rs.idx)] = rs.idx
            cnt[u, i] = len(rs.idx)
            rows.append(rs)
    return idx.reshape(lead + (R, km)), cnt.reshape(lead + (R,)), rows


# --------------------------------------------------------------------------
# O4 -- attention over the selected blocks
# --------------------------------------------------------------------------
def _softmax_row(logits: np.ndarray):
    mx = logits.max()
    w = np.exp(logits - mx)
    ssum = w.sum()
    return w / ssum, mx + math.log(ssum)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, cnt: np.ndarray, block: int,
           units=None):
    """Causal attention restricted to the selected key blocks.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; idx: [B, Hkv, nB, kmax] (ascending
    block ids, -1 padded); cnt: [B, Hkv, nB].  For row p of query block i the
    visible keys are the positions c <= p inside the blocks idx[..., i, :cnt].
    The logits are s * q_p . k_c with s = 1/sqrt(d); returns O float64
    [B, Hq, N, d] and the natural-log LSE [B, Hq, N].  ``units`` optionally
    restricts the work to a list of (b, h, i) query blocks; the other rows of
    O and LSE are left at zero.

    [SvF] section 1 pseudo-code: logits, apply the sparsity pattern, softmax of
    the scaled logits, times the values.  The pattern is applied by gathering
    the visible keys -- a dropped key never enters the sum, so its value
    cannot leak into the output ([ZB]: the others are set to zero).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    nB = n_blocks(N, block)
    if units is None:
        units = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nB)]
    o = np.zeros((B, Hq, N, d), dtype=np.float64)
    lse = np.zeros((B, Hq, N), dtype=np.float64)
    for (b, h, i) in units:
        g = h // G
        blocks = [int(j) for j in idx[b, g, i, : cnt[b, g, i]]]
        keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block)) for j in blocks])
        keys.sort()
        ks, vs = k[b, g, keys], v[b, g, keys]
        for p in range(i * block, min(N, (i + 1) * block)):
            n_vis = int(np.searchsorted(keys, p, side="right"))  # the keys c <= p
            logits = scale * (ks[:n_vis] @ q[b, h, p])
            w, lse[b, h, p] = _softmax_row(logits)
            o[b, h, p] = w @ vs[:n_vis]
    return o, lse


def attend_backward(q, k, v, do, idx, cnt, block: int, units=None, o=None):
    """Gradients of ``attend`` with the selection held fixed.

    Returns (dq [B, Hq, N, d], dk, dv [B, Hkv, N, d]) in float64 for the loss
    whose gradient with respect to O is ``do``.  The selection is a discrete
    choice and is not differentiated; the keys a row does not see get no
    gradient from it.

    Per row p, with w the softmax weights over its visible keys c (exactly as
    in ``attend``): the chain rule through o_p = sum_c w_c v_c and
    w = softmax(s q_p . k_c) gives dv_c += w_c do_p, dw_c = do_p . v_c,
    dlogit_c = w_c (dw_c - sum_c' w_c' dw_c'), dq_p = s sum_c dlogit_c k_c and
    dk_c += s dlogit_c q_p (summed over the G query heads that share a KV
    head).  ``units`` restricts the rows as in ``attend`` (a unit (b, h, i)
    adds its rows' contributions to dk and dv).

    The term sum_c' w_c' dw_c' equals do_p . o_p.  By default it is taken from
    the exact weights; with ``o`` ([B, Hq, N, d], e.g. a rounded forward
    output) it is do_p . o[p] instead -- the quantity a backward that is handed
    the forward's output computes.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    nB = n_blocks(N, block)
    if units is None:
        units = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nB)]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for (b, h, i) in units:
        g = h // G
        blocks = [int(j) for j in idx[b, g, i, : cnt[b, g, i]]]
        keys = np.concatenate([np.arange(j * block, min(N, (j + 1) * block)) for j in blocks])
        keys.sort()
        ks, vs = k[b, g, keys], v[b, g, keys]
        for p in range(i * block, min(N, (i + 1) * block)):
            n_vis = int(np.searchsorted(keys, p, side="right"))
            kv = keys[:n_vis]
            logits = scale * (ks[:n_vis] @ q[b, h, p])
            w, _ = _softmax_row(logits)
            dw = vs[:n_vis] @ do[b, h, p]
            dsum = w @ dw if o is None else float(np.asarray(o[b, h, p], dtype=np.float64) @ do[b, h, p])
            dlogit = w * (dw - dsum)
            dq[b, h, p] = scale * (dlogit @ ks[:n_vis])
            dk[b, g, kv] += scale * np.outer(dlogit, q[b, h, p])
            dv[b, g, kv] += np.outer(w, do[b, h, p])
    return dq, dk, dv


# --------------------------------------------------------------------------
# Whole paths
# --------------------------------------------------------------------------
def prefill(q, k, v, block: int, topk: int, num: int = 0, den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG,
            attend_blocks=None):
    """Pool -> score -> select -> attend (O1-O4) for a causal prefill.

    ``attend_blocks`` optionally restricts O4 to a list of (b, h, i) query
    blocks (the rest of O and LSE is left at zero) so that large shapes can
    be checked on a sample.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    qbar, kbar = block_means(q, block), block_means(k, block)
    scores = block_scores(qbar, kbar, scale)
    idx, cnt, rows = select_topk(scores, topk, num, den, flags, causal=True)
    o, lse = attend(q, k, v, idx, cnt, block, units=attend_blocks)
    return dict(qbar=qbar, kbar=kbar, scores=scores, idx=idx, cnt=cnt, rows=rows, o=o, lse=lse)


def decode(q, kc, vc, block: int, topk: int, num: int = 0, den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG,
           units=None):
    """One decode step for S sequences (O1-O4 with a single query row).

    q: [S, Hq, d] -- the new token of each sequence, which sits at the last
    cache position L-1; kc, vc: [S, Hkv, L, d].  Scores use the block means of
    the cached keys ([ZB] "动态开销与计算收益的权衡": summaries computed at
    cache time, not reselected from raw keys), max over the group's heads; the
    sink and the last block are forced; all keys of the kept blocks are
    visible.  ``units`` optionally restricts O4 to a list of (s, g).
    Returns dict(kbar, scores [S,Hkv,nB], idx [S,Hkv,kmax], cnt [S,Hkv], rows,
    o [S,Hq,d], lse [S,Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(kc, dtype=np.float64)
    vc = np.asarray(vc, dtype=np.float64)
    S, Hq, d = q.shape
    Hkv, L = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    kbar = block_means(kc, block)  # [S, Hkv, nB, d]
    nB = kbar.shape[2]
    scores = np.empty((S, Hkv, 1, nB))
    for s in range(S):
        for g in range(Hkv):
            per_head = [scale * (kbar[s, g] @ q[s, h]) for h in range(g * G, (g + 1) * G)]
            scores[s, g, 0] = np.max(np.stack(per_head), axis=0)
    idx, cnt, rows = select_topk(scores, topk, num, den, flags, causal=False)
    idx, cnt = idx[:, :, 0], cnt[:, :, 0]
    o = np.zeros((S, Hq, d))
    lse = np.zeros((S, Hq))
    todo = units if units is not None else [(s, g) for s in range(S) for g in range(Hkv)]
    for (s, g) in todo:
        keys = np.concatenate([np.arange(j * block, min(L, (j + 1) * block)) for j in idx[s, g, : cnt[s, g]]])
        keys.sort()
        for h in range(g * G, (g + 1) * G):
            logits = scale * (kc[s, g, keys] @ q[s, h])
            w, lse[s, h] = _softmax_row(logits)
            o[s, h] = w @ vc[s, g, keys]
    return dict(kbar=kbar, scores=scores[:, :, 0], idx=idx, cnt=cnt, rows=rows, o=o, lse=lse)


def accepts(rs: RowSelection, got: list) -> tuple[bool, str]:
    """Whether a selection ``got`` (ascending block ids, no padding) is a
    correct answer for the row described by ``rs``: it holds every forced
    block and every ``must`` candidate, its other candidates all lie in the
    near-tie band, it takes exactly ``need`` of them, and it is ascending."""
    if list(got) != sorted(set(got)):
        return False, f"not ascending/unique: {got}"
    gs = set(got)
    if not set(rs.forced) <= gs:
        return False, f"forced {rs.forced} missing from {got}"
    t = gs - set(rs.forced)
    if not rs.must <= t:
        return False, f"missing {sorted(rs.must - t)}"
    extra = t - rs.must
    if not extra <= rs.band:
        return False, f"outside selection/band: {sorted(extra - rs.band)}"
    if len(extra) != rs.need:
        return False, f"takes {len(extra)} from the tie band, needs {rs.need}"
    return True, ""
