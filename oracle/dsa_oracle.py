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
     variants (``SelectSpec``): global anchors + a local window as the forced
     set; threshold selection on the row's block softmax; a budget from the
     entropy of that softmax; ``bitmap`` packs a selection into bit words.
  O4 ``attend``        softmax(s * q k^T) v over exactly the keys of the kept
                        blocks that are causally visible to each row.
  ``prefill`` / ``decode`` chain O1-O4.
  I1 ``index_scores``  token-level lightning-indexer scores: for query token t
                        and earlier token s, the sum over the index heads of
                        head weight times ReLU(index query . index key).
  I2 ``select_tokens`` per query token, the top-k earlier tokens by I1 (the
                        same selection rule as O3, rows = tokens).
  I3 ``token_attend``  attention of every head over its token's selected
                        tokens.  ``index_prefill`` chains I1-I3.
  P1 ``paged_gather`` /  a paged KV cache (pages of one block, a block table
     ``paged_decode``    per sequence, a length per sequence): the decode of
                        each sequence over its own gathered cache.
  P2 ``kv_append``     append one token per sequence: write it into its page
                        and recompute that page's key block mean.
  P3 ``quantize_fp8`` / FP8 (E4M3) cache rows with one fp32 scale per
     ``dequantize_fp8``  (token, KV head) row; the fp8 paged decode is the
                        paged decode of the dequantized pools.
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
  [LC]  "低成本高性能大模型实现路径：从架构创新到工程优化"
        (yunthe.com/news/806485.html), section 2.1 "轻量化索引器设计" (the
        indexer: ReLU features, 16 index heads, each query token mapped to
        its high-value key/value tokens with a top-k of 64) and section 2.2
        (the indexer keeps its intermediates in FP8).

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
    dV of a KV head sum the contributions of its G query heads;
  * selection variants: the forced set is the first ``anchors`` blocks and
    the last ``window`` visible blocks (the window ends at the row's own
    block); a row's block distribution is the softmax of its visible block
    scores; threshold mode keeps the candidates whose share is >= tau;
    entropy mode keeps ceil(exp(H)) blocks (H the Shannon entropy of that
    distribution, nats), clamped to [k_min, k_max], then runs the top-k;
  * token indexer: the page's listing is garbled; from its text (ReLU
    features, 16 index heads, top-64 per query token) the score of earlier
    token s for query token t is sum_h w[t,h] * ReLU(qi[t,h] . ki[s]) with one
    index key per token shared by the heads; one top-k per query token (sink
    and self forced as in O3) is shared by every attention head;
  * production decode: a page holds one block of one sequence for every KV
    head; sequence s sees its first lengths[s] tokens; the block means are
    kept per page and recomputed from the page's rows when a token lands in
    it (the index data is built when the cache is written);
  * FP8 cache ([ZB] "工程实践建议": combine the sparsity with an FP8/INT4 KV
    cache): a row's scale is amax / 448 in fp32 (448 is E4M3's largest
    finite value; 1 for an all-zero row), its codes are the E4M3 values
    nearest to fp32(x / scale), ties to even; the block means and the
    attention use the dequantized values, code * scale.

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

# near-tie rule for flagging rows (see ``near``): the acceptance rule's 1e-3
# relative gap.  Token-indexer rows add an absolute floor (``TOKEN_TIE_ABS``).
TIE_REL = 1e-3
TOKEN_TIE_ABS = 1e-6

# selection modes (``SelectSpec.mode``)
SELECT_TOPK = 0
SELECT_THRESHOLD = 1
SELECT_ENTROPY = 2
# a candidate whose block share is within THR_REL (relative) of the threshold
# may be kept or dropped; an exp(entropy) within ENT_REL (relative) of an
# integer may round either way
THR_REL = 1e-3
ENT_REL = 1e-4


@dataclass(frozen=True)
class SelectSpec:
    """How a row's kept set is chosen beyond the plain top-k.

    ``anchors``: with FORCE_SINK, blocks 0 .. anchors-1 are forced (global
    anchors; 1 = the sink alone).  ``window``: with FORCE_DIAG, the last
    ``window`` visible blocks are forced (a local window ending at the row's
    own block; 1 = the diagonal alone).  ``mode``: SELECT_TOPK (budget from
    topk or the fraction), SELECT_THRESHOLD (keep candidates whose share of
    the row's block softmax is >= ``threshold``) or SELECT_ENTROPY (budget
    ceil(exp(H)) clamped to [k_min, k_max]).

    [ZB] "基于Top-k选择的局部-全局混合" (local window + global tokens);
    [NSA] section 2.2 (block-sparsify the fp32 scores with a threshold);
    [ZB] "模型精度与稀疏度的动态平衡" and "工程实践建议" (set k or the threshold
    from the attention entropy; keep more when the entropy is high)."""

    mode: int = SELECT_TOPK
    anchors: int = 1
    window: int = 1
    threshold: float = 0.0
    k_min: int = 0
    k_max: int = 0


DEFAULT_SPEC = SelectSpec()


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


def forced_set(n_visible: int, flags: int, anchors: int = 1, window: int = 1) -> list[int]:
    """Blocks kept regardless of score: the global anchors (blocks 0 ..
    anchors-1; anchors = 1 is the sink) and the local window (the last
    ``window`` visible blocks; window = 1 is the row's own block).

    [ZB] "基于Top-k选择的局部-全局混合": global tokens plus a local window;
    [SvF] section 1 hybrid mode: local window plus periodic global anchors.
    """
    f = set()
    if flags & FORCE_SINK:
        f.update(range(min(anchors, n_visible)))
    if flags & FORCE_DIAG:
        f.update(range(max(n_visible - window, 0), n_visible))
    return sorted(f)


def block_shares(scores: np.ndarray) -> np.ndarray:
    """The row's block distribution: softmax of its visible block scores,
    p_j = exp(S_j) / sum_c exp(S_c) (the largest score is subtracted first,
    which leaves the quotient unchanged)."""
    sc = np.asarray(scores, dtype=np.float64)
    e = np.exp(sc - sc.max())
    return e / e.sum()


def block_entropy(scores: np.ndarray) -> float:
    """Shannon entropy (nats) of the row's block distribution, -sum p log p
    (terms with p = 0 contribute 0)."""
    p = block_shares(scores)
    nz = p[p > 0]
    return float(-(nz * np.log(nz)).sum())


def entropy_budgets(scores: np.ndarray, n_visible: int, k_min: int, k_max: int, n_forced: int) -> list[int]:
    """Budget of an entropy-mode row: ceil(exp(H)) -- the effective number of
    blocks the row attends to -- clamped to [k_min, k_max], raised to the
    forced count and capped at the visible count.  When exp(H) is within
    ENT_REL of an integer n, fp32 can land on either side of it: both budgets
    (from n and from n + 1) are returned."""
    e = math.exp(block_entropy(np.asarray(scores)[:n_visible]))

    def fit(k):
        return min(max(min(max(k, k_min), k_max), n_forced), n_visible)

    n = round(e)
    if abs(e - n) <= ENT_REL * e:
        return sorted({fit(n), fit(n + 1)})
    return [fit(math.ceil(e))]


def threshold_row(scores: np.ndarray, n_visible: int, tau: float, forced: list) -> "RowSelection":
    """Threshold selection of one row: the forced blocks plus every candidate
    whose share of the row's block distribution is >= tau.  [NSA] section 2.2
    block-sparsifies the fp32 scores with a threshold.  Candidates whose share
    is within THR_REL of tau form a band: an accepted set may keep or drop
    each of them."""
    p = block_shares(np.asarray(scores, dtype=np.float64)[:n_visible])
    fs = set(forced)
    cand = [j for j in range(n_visible) if j not in fs]
    keep = {j for j in cand if p[j] >= tau}
    band = {j for j in cand if abs(p[j] - tau) <= THR_REL * tau}
    return RowSelection(idx=sorted(fs | keep), forced=sorted(fs), must=keep - band, band=band, need=-1,
                        flagged=bool(band))


def near(a: float, b: float, abs_floor: float = 0.0) -> bool:
    """Near-tie test between two scores: a relative gap below 1e-3, the
    acceptance rule for block indices (rel(a, b) = |a - b| / max(|a|, |b|),
    0 when a == b).  ``abs_floor`` > 0 also counts gaps below it (the token
    indexer, see ``select_tokens``)."""
    if a == b:
        return True
    if not (math.isfinite(a) and math.isfinite(b)):
        return False
    gap = abs(a - b)
    return gap < TIE_REL * max(abs(a), abs(b)) or gap < abs_floor


@dataclass
class RowSelection:
    """Selection of one row and what another correct selection may differ in.

    ``idx``: the kept blocks, ascending.  ``forced``: blocks kept regardless.
    ``must``: candidates any accepted set contains.  ``band``: near-tie
    candidates of which exactly ``need`` are kept (need = -1: any number).
    ``alts``: other selections that are equally correct (an entropy budget
    that fp32 may round either way).  Unflagged rows have an empty band and
    no alternatives (the selection is unique)."""

    idx: list
    forced: list
    must: set
    band: set = field(default_factory=set)
    need: int = 0
    flagged: bool = False
    alts: list = field(default_factory=list)


def select_row(scores: np.ndarray, n_visible: int, k_budget: int, forced: list,
               abs_floor: float = 0.0) -> RowSelection:
    """Keep ``k_budget`` of the ``n_visible`` blocks of one row.

    The forced blocks are kept; the remaining m = k_budget - |forced| are the
    highest-scoring candidates, ordered by (score descending, index
    ascending).  [ZB] "基于Top-k选择的局部-全局混合": per query keep the
    k highest-scoring keys and drop the rest.

    A row is flagged when the m-th and (m+1)-th candidates are near-ties
    (``near`` with ``abs_floor``); its band holds the ranks from the first to
    the last candidate near either of those two scores.
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
    if m >= ranked.size or not near(float(rsc[m - 1]), float(rsc[m]), abs_floor):
        return RowSelection(idx=sel, forced=sorted(fs), must=chosen)
    a, b = float(rsc[m - 1]), float(rsc[m])
    in_band = [r for r in range(ranked.size)
               if near(float(rsc[r]), a, abs_floor) or near(float(rsc[r]), b, abs_floor)]
    lo, hi = min(in_band), max(in_band)
    must = set(int(j) for j in ranked[:lo])
    band = set(int(j) for j in ranked[lo : hi + 1])
    return RowSelection(idx=sel, forced=sorted(fs), must=must, band=band, need=m - lo, flagged=True)


def spec_tau(spec: SelectSpec) -> float:
    """The threshold as the fp32 value a caller's float carries."""
    return float(np.float32(spec.threshold))


def kmax(n_rows: int, topk: int, num: int, den: int, flags: int, causal: bool, n_cols: int,
         spec: SelectSpec = DEFAULT_SPEC) -> int:
    """Largest per-row count of kept blocks: the width of the index array.
    Threshold mode: the forced blocks plus floor(1 / tau), the most candidates
    whose shares can each reach tau (the shares sum to 1)."""
    best = 0
    for i in range(n_rows):
        nv = i + 1 if causal else n_cols
        nf = len(forced_set(nv, flags, spec.anchors, spec.window))
        if spec.mode == SELECT_THRESHOLD:
            k = min(nv, nf + math.floor(1.0 / spec_tau(spec)))
        elif spec.mode == SELECT_ENTROPY:
            k = min(max(spec.k_max, nf), nv)
        else:
            k = row_budget(nv, topk, num, den, nf)
        best = max(best, k)
    return best


def select_topk(scores: np.ndarray, topk: int, num: int = 0, den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG,
                causal: bool = True, spec: SelectSpec = DEFAULT_SPEC, abs_floor: float = 0.0):
    """Row-wise selection over a score array [..., R, C].

    causal=True (prefill): row i sees blocks 0..i.  causal=False (decode):
    every row sees all C blocks.  ``spec`` picks the forced set and the mode
    (plain top-k by default).  Returns (idx, cnt, rows) where idx is int32
    [..., R, kmax] ascending and -1 padded, cnt is int32 [..., R] and rows is
    a flat list of ``RowSelection`` in C order.  ``abs_floor``: see ``near``.
    """
    lead = scores.shape[:-2]
    R, C = scores.shape[-2:]
    km = kmax(R, topk, num, den, flags, causal, C, spec)
    flat = scores.reshape((-1, R, C))
    idx = np.full((flat.shape[0], R, km), -1, dtype=np.int32)
    cnt = np.zeros((flat.shape[0], R), dtype=np.int32)
    rows = []
    for u in range(flat.shape[0]):
        for i in range(R):
            nv = i + 1 if causal else C
            f = forced_set(nv, flags, spec.anchors, spec.window)
            row = flat[u, i, :nv]
            if spec.mode == SELECT_THRESHOLD:
                rs = threshold_row(row, nv, spec_tau(spec), f)
            elif spec.mode == SELECT_ENTROPY:
                ks = entropy_budgets(row, nv, spec.k_min, spec.k_max, len(f))
                rs = select_row(row, nv, ks[0], f, abs_floor)
                if len(ks) > 1:
                    rs.alts = [select_row(row, nv, kb, f, abs_floor) for kb in ks[1:]]
                    rs.flagged = True
            else:
                rs = select_row(row, nv, row_budget(nv, topk, num, den, len(f)), f, abs_floor)
            idx[u, i, : len(rs.idx)] = rs.idx
            cnt[u, i] = len(rs.idx)
            rows.append(rs)
    return idx.reshape(lead + (R, km)), cnt.reshape(lead + (R,)), rows


def bitmap(idx: np.ndarray, cnt: np.ndarray, n_cols: int) -> np.ndarray:
    """A selection as bit words: [..., ceil(n_cols / 32)] uint32 with bit
    j % 32 of word j // 32 set when block j is kept.  [ZB] "工程实践建议":
    store the sparse index as a compressed bitmap rather than a full index
    array."""
    words = (n_cols + 31) // 32
    lead = cnt.shape
    out = np.zeros(lead + (words,), dtype=np.uint32)
    fi = idx.reshape((-1, idx.shape[-1]))
    fc = cnt.reshape(-1)
    fo = out.reshape((-1, words))
    for r in range(fc.size):
        for j in fi[r, : fc[r]]:
            fo[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return out


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
            attend_blocks=None, spec: SelectSpec = DEFAULT_SPEC):
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
    idx, cnt, rows = select_topk(scores, topk, num, den, flags, causal=True, spec=spec)
    o, lse = attend(q, k, v, idx, cnt, block, units=attend_blocks)
    return dict(qbar=qbar, kbar=kbar, scores=scores, idx=idx, cnt=cnt, rows=rows, o=o, lse=lse)


def decode(q, kc, vc, block: int, topk: int, num: int = 0, den: int = 1, flags: int = FORCE_SINK | FORCE_DIAG,
           units=None, spec: SelectSpec = DEFAULT_SPEC):
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
    idx, cnt, rows = select_topk(scores, topk, num, den, flags, causal=False, spec=spec)
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
    correct answer for the row described by ``rs`` or one of its
    alternatives: it holds every forced block and every ``must`` candidate,
    its other candidates all lie in the near-tie band, it takes exactly
    ``need`` of them (any number when need = -1), and it is ascending."""
    ok, why = _accepts_one(rs, got)
    if ok:
        return ok, why
    for alt in rs.alts:
        if _accepts_one(alt, got)[0]:
            return True, ""
    return False, why


def _accepts_one(rs: RowSelection, got: list) -> tuple[bool, str]:
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
    if rs.need >= 0 and len(extra) != rs.need:
        return False, f"takes {len(extra)} from the tie band, needs {rs.need}"
    return True, ""


# --------------------------------------------------------------------------
# I1-I3 -- token-level lightning indexer and token-gather attention
# --------------------------------------------------------------------------
def index_score_row(qi_t: np.ndarray, ki: np.ndarray, wi_t: np.ndarray, t: int) -> np.ndarray:
    """Scores of tokens 0..t for query token t: I[s] = sum_h wi_t[h] *
    max(0, qi_t[h] . ki[s]).  qi_t [HI, dI], ki [N, dI], wi_t [HI].

    [LC] section 2.1: ReLU feature heads (HI = 16) score where the query
    token should look."""
    dots = np.asarray(ki, dtype=np.float64)[: t + 1] @ np.asarray(qi_t, dtype=np.float64).T  # [t+1, HI]
    return np.maximum(dots, 0.0) @ np.asarray(wi_t, dtype=np.float64)


def index_scores(qi: np.ndarray, ki: np.ndarray, wi: np.ndarray) -> np.ndarray:
    """I [B, N, N]: row t holds index_score_row for s <= t and -inf above.
    qi [B, N, HI, dI], ki [B, N, dI], wi [B, N, HI]."""
    B, N = qi.shape[:2]
    out = np.full((B, N, N), -np.inf)
    for b in range(B):
        for t in range(N):
            out[b, t, : t + 1] = index_score_row(qi[b, t], ki[b], wi[b, t], t)
    return out


def select_tokens(scores: np.ndarray, topk: int, flags: int = FORCE_SINK | FORCE_DIAG,
                  spec: SelectSpec = DEFAULT_SPEC):
    """Per query token t the forced tokens (the sink token 0 and t itself, per
    ``flags``) and the best other tokens up to ``topk`` by index score (ties
    to the lower position), ascending: the O3 rule with rows and columns
    being tokens.  scores [B, N, N]; returns idx [B, N, kmax], cnt [B, N],
    rows.

    Near ties: besides the 1e-3 relative gap, two token scores within
    ``TOKEN_TIE_ABS`` (1e-6) of each other flag the row.  A token score is a
    sum of ReLU(index query . index key) terms; a dot product that lies
    within fp32 rounding of zero is clipped to zero in one evaluation and
    kept as a tiny positive value in another, so scores that close to each
    other near zero cannot be ordered in fp32.  Block scores pass through no
    such clip and use the relative rule alone."""
    idx, cnt, rows = select_topk(np.asarray(scores)[:, None], topk, 0, 1, flags, causal=True, spec=spec,
                                 abs_floor=TOKEN_TIE_ABS)
    return idx[:, 0], cnt[:, 0], rows


def token_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, cnt: np.ndarray, units=None):
    """Attention of query token t, head h over the tokens idx[b, t, :cnt]
    (all <= t): softmax of s * q . k over them, times their values, s =
    1/sqrt(d); query head h reads KV head h // G.  q [B, Hq, N, d]; k, v
    [B, Hkv, N, d]; returns O [B, Hq, N, d] and LSE [B, Hq, N] (float64).
    ``units`` restricts the rows to a list of (b, h, t)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(d)
    if units is None:
        units = [(b, h, t) for b in range(B) for h in range(Hq) for t in range(N)]
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for (b, h, t) in units:
        keys = [int(s) for s in idx[b, t, : cnt[b, t]]]
        logits = scale * (k[b, h // G, keys] @ q[b, h, t])
        w, lse[b, h, t] = _softmax_row(logits)
        o[b, h, t] = w @ v[b, h // G, keys]
    return o, lse


def index_prefill(qi, ki, wi, q, k, v, topk: int, flags: int = FORCE_SINK | FORCE_DIAG, attend_units=None):
    """I1 -> I2 -> I3 for a causal prefill."""
    sc = index_scores(qi, ki, wi)
    idx, cnt, rows = select_tokens(sc, topk, flags)
    o, lse = token_attend(q, k, v, idx, cnt, units=attend_units)
    return dict(scores=sc, idx=idx, cnt=cnt, rows=rows, o=o, lse=lse)


# --------------------------------------------------------------------------
# P1-P2 -- paged KV cache, per-sequence lengths, appends
# --------------------------------------------------------------------------
def paged_gather(pool: np.ndarray, table: np.ndarray, s: int, length: int, block: int) -> np.ndarray:
    """The first ``length`` rows of sequence s from a paged pool [n_pages,
    Hkv, block, d]: logical block j lives in page table[s, j].  Returns
    [Hkv, length, d]."""
    nb = n_blocks(length, block)
    if nb == 0:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    rows = [np.asarray(pool[int(table[s, j])], dtype=np.float64) for j in range(nb)]
    return np.concatenate(rows, axis=1)[:, :length]


def paged_decode(q, k_pool, v_pool, table, lengths, block: int, topk: int, num: int = 0, den: int = 1,
                 flags: int = FORCE_SINK | FORCE_DIAG, spec: SelectSpec = DEFAULT_SPEC, units=None):
    """One decode step over a paged cache with a length per sequence: for
    every sequence the O1-O4 decode of its own gathered cache (its new token
    is at position lengths[s] - 1; its last block may be partial).  [ZB]
    "动态开销与计算收益的权衡" ties the index data to the KV cache.

    q [S, Hq, d]; pools [n_pages, Hkv, block, d]; table [S, max_blocks];
    lengths [S].  Returns o [S, Hq, d], lse [S, Hq], idx [S, Hkv, kmax] (-1
    padded, kmax from the longest possible sequence, max_blocks * block),
    cnt [S, Hkv] and rows (a list per (s, g), None for empty sequences).
    ``units`` restricts the attention to a list of (s, g)."""
    q = np.asarray(q, dtype=np.float64)
    S, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    max_blocks = table.shape[1]
    km = kmax(1, topk, num, den, flags, False, max_blocks, spec)
    o = np.zeros((S, Hq, d))
    lse = np.full((S, Hq), -np.inf)
    idx = np.full((S, Hkv, km), -1, dtype=np.int32)
    cnt = np.zeros((S, Hkv), dtype=np.int32)
    rows = [None] * (S * Hkv)
    for s in range(S):
        L = int(lengths[s])
        if L == 0:
            continue
        kc = paged_gather(k_pool, table, s, L, block)[None]
        vc = paged_gather(v_pool, table, s, L, block)[None]
        todo = [(0, g) for g in range(Hkv) if units is None or (s, g) in units]
        r = decode(q[s : s + 1], kc, vc, block, topk, num, den, flags, units=todo, spec=spec)
        for g in range(Hkv):
            c = int(r["cnt"][0, g])
            idx[s, g, :c] = r["idx"][0, g, :c]
            cnt[s, g] = c
            rows[s * Hkv + g] = r["rows"][g]
            if units is None or (s, g) in units:
                o[s, g * G : (g + 1) * G] = r["o"][0, g * G : (g + 1) * G]
                lse[s, g * G : (g + 1) * G] = r["lse"][0, g * G : (g + 1) * G]
    return dict(o=o, lse=lse, idx=idx, cnt=cnt, rows=rows)


def kv_append(k_pool, v_pool, kbar_pool, table, lengths, k_new, v_new, block: int):
    """Append one token per sequence, in place: sequence s writes k_new[s],
    v_new[s] ([Hkv, d]) at position lengths[s] (page table[s, pos // block],
    slot pos % block), recomputes that page's key mean over its rows 0 ..
    pos % block, and advances lengths[s]."""
    for s in range(len(lengths)):
        pos = int(lengths[s])
        page = int(table[s, pos // block])
        slot = pos % block
        k_pool[page, :, slot] = k_new[s]
        v_pool[page, :, slot] = v_new[s]
        kbar_pool[page] = np.asarray(k_pool[page, :, : slot + 1], dtype=np.float64).mean(axis=1)
        lengths[s] = pos + 1


def paged_block_means(k_pool, table, lengths, block: int, n_pages: int) -> np.ndarray:
    """Key block means per page for the pages the sequences use: the mean of
    the page's rows that lie below the sequence's length.  Unused pages stay
    zero.  Returns [n_pages, Hkv, d]."""
    out = np.zeros((n_pages, k_pool.shape[1], k_pool.shape[3]))
    for s in range(len(lengths)):
        L = int(lengths[s])
        for j in range(n_blocks(L, block)):
            rows = min(block, L - j * block)
            out[int(table[s, j])] = np.asarray(k_pool[int(table[s, j]), :, :rows], dtype=np.float64).mean(axis=1)
    return out


# --------------------------------------------------------------------------
# P3 -- FP8 (E4M3) cache rows
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def quantize_fp8(x: np.ndarray):
    """Rows of x (last axis) -> (codes uint8 [..., d], scales float32 [...]).

    scale = fp32(amax(|row|) / 448) (1 for an all-zero row); code = E4M3
    (OCP, no infinities) value nearest to fp32(x / scale), ties to even --
    the division is taken in fp32, the precision the decision is made in.
    The rounding itself is torch's float8_e4m3fn cast (a library step)."""
    import torch

    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[..., None]).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def fp8_values(codes: np.ndarray) -> np.ndarray:
    """The E4M3 value of each code (float64)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def dequantize_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """code value * row scale (float64, exact)."""
    return fp8_values(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def kv_append_fp8(k8, v8, k_scale, v_scale, kbar_pool, table, lengths, k_new, v_new, block: int):
    """``kv_append`` for an FP8 cache: the new rows are quantized (their own
    scales) and written; the page mean is recomputed from the dequantized
    rows 0 .. slot."""
    for s in range(len(lengths)):
        pos = int(lengths[s])
        page = int(table[s, pos // block])
        slot = pos % block
        kc, ks = quantize_fp8(k_new[s])
        vc, vs = quantize_fp8(v_new[s])
        k8[page, :, slot], k_scale[page, :, slot] = kc, ks
        v8[page, :, slot], v_scale[page, :, slot] = vc, vs
        kbar_pool[page] = dequantize_fp8(k8[page, :, : slot + 1], k_scale[page, :, : slot + 1]).mean(axis=1)
        lengths[s] = pos + 1

