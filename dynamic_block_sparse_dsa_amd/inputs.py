"""Seeded synthetic inputs for block-sparse attention workloads.

This module only draws random numbers and plants structure into them; it holds
none of the attention method's arithmetic, so both the HIP path and the CPU
oracle can take their inputs from it.

Recipe (one torch generator per (batch or sequence, KV head) unit, so any unit
can be regenerated alone):
  * values: float32 N(0, 1), drawn in the order Q (the G query heads of the
    group), K, V, then the structure; cast to bf16 with round-to-nearest-even;
  * ``planted`` (amplitude a): every KV block j gets a random unit direction
    u_j added to all of its key rows (times a); every query block i >= 2 picks
    min(4, i - 1) target blocks among 1..i-1 and adds a times the unit vector
    along the sum of their directions to its query rows (all heads of the
    group share the targets; the noise is per head).  Decode plants the same
    way with the single query token aiming at targets among 1..nB-2;
  * ``heavy`` (amplitude a, fraction f): per unit, round(f * nB) blocks among
    1..nB-1 get a times one shared unit direction u added to their key rows,
    and every query row gets a times u;
  * ``plain``: no structure.
Target picks are drawn on the CPU with a generator of their own so that the
values drawn on the device do not depend on them.

Token-indexer workloads (``IndexWorkload``, ``make_index``; one generator per
batch entry): index queries qi [B, N, HI, dI] and keys ki [B, N, dI] are
N(0, 1); with ``clusters`` C > 0 every token s belongs to a cluster c(s)
(uniform over C) whose random unit direction times the amplitude is added to
ki[s], and every query token t aims all its index heads at one cluster drawn
uniformly (the same direction times the amplitude added to qi[t, h]); head
weights wi [B, N, HI] are U(0, 1) fp32; the attention Q, K, V are N(0, 1).
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" or "decode"
    batch: int  # B (prefill) or number of sequences S (decode)
    n_q_heads: int
    n_kv_heads: int
    seq_len: int  # N (prefill) or cache length L (decode)
    head_dim: int
    block: int
    topk: int  # > 0: fixed number of kept blocks (forced ones included)
    topk_num: int = 0  # topk == 0: keep ceil(num * visible / den) blocks
    topk_den: int = 1
    structure: str = "plain"
    amplitude: float = 0.0
    heavy_frac: float = 0.0
    seed: int = 0

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    w.name: w
    for w in [
        Workload("prefill_tiny_n1024", "prefill", 1, 2, 2, 1024, 64, 64, 4, seed=0),
        Workload("prefill_n8192_h32", "prefill", 1, 32, 32, 8192, 128, 64, 16, structure="planted", amplitude=2.0,
                 seed=1),
        Workload("prefill_gqa_n32768", "prefill", 1, 32, 8, 32768, 128, 64, 0, 15, 100, structure="planted",
                 amplitude=2.0, seed=2),
        Workload("prefill_n131072_b128", "prefill", 1, 16, 16, 131072, 128, 128, 64, structure="heavy", amplitude=3.0,
                 heavy_frac=0.05, seed=3),
        Workload("decode_s32_l65536", "decode", 32, 32, 8, 65536, 128, 64, 32, structure="planted", amplitude=2.0,
                 seed=4),
    ]
}


def _gen(device, seed: int, unit: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed << 40) ^ (unit << 8) ^ stream)
    return g


def _unit_rows(n: int, d: int, gen, device) -> torch.Tensor:
    return torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)


def _directions(n: int, d: int, gen, device) -> torch.Tensor:
    u = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    return u / u.norm(dim=-1, keepdim=True)


def _target_matrix(nb_rows: int, first_target: int, last_target_of, count: int, cpu_gen, n_cols: int) -> torch.Tensor:
    """0/1 matrix M[i, j] = 1 when row i targets column j."""
    m = torch.zeros((nb_rows, n_cols), dtype=torch.float32)
    for i in range(nb_rows):
        hi = last_target_of(i)  # targets drawn from first_target..hi inclusive
        span = hi - first_target + 1
        if span <= 0:
            continue
        pick = torch.randperm(span, generator=cpu_gen)[: min(count, span)] + first_target
        m[i, pick] = 1.0
    return m


def _aim(m: torch.Tensor, u: torch.Tensor) -> torch.Tensor:
    """Unit vector along the sum of each row's target directions (zero rows stay zero)."""
    w = m.to(u.device) @ u
    nrm = w.norm(dim=-1, keepdim=True)
    return torch.where(nrm > 0, w / nrm.clamp_min(1e-30), torch.zeros_like(w))


def _expand_blocks(per_block: torch.Tensor, n: int, block: int) -> torch.Tensor:
    """[nB, d] -> [n, d]: row r takes the entry of block r // block."""
    return per_block.repeat_interleave(block, dim=0)[:n]


def make_prefill(w: Workload, device="cpu", seed: int | None = None):
    """Q [B, Hq, N, d], K and V [B, Hkv, N, d] as contiguous bf16 tensors."""
    assert w.kind == "prefill"
    seed = w.seed if seed is None else seed
    B, Hq, Hkv, N, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    G, nb = w.group, w.n_blocks
    q = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=device)
    for bi in range(B):
        for g in range(Hkv):
            unit = bi * Hkv + g
            gen = _gen(device, seed, unit, 1)
            qs = torch.randn((G, N, d), generator=gen, device=device, dtype=torch.float32)
            ks = _unit_rows(N, d, gen, device)
            vs = _unit_rows(N, d, gen, device)
            if w.structure == "planted":
                u = _directions(nb, d, gen, device)
                ks += w.amplitude * _expand_blocks(u, N, b)
                m = _target_matrix(nb, 1, lambda i: i - 1, 4, _gen("cpu", seed, unit, 2), nb)
                qs += w.amplitude * _expand_blocks(_aim(m, u), N, b)[None]
            elif w.structure == "heavy":
                u = _directions(1, d, gen, device)[0]
                n_heavy = int(round(w.heavy_frac * nb))
                heavy = torch.randperm(nb - 1, generator=_gen("cpu", seed, unit, 2))[:n_heavy] + 1
                mask = torch.zeros(nb, dtype=torch.float32)
                mask[heavy] = 1.0
                ks += w.amplitude * _expand_blocks(mask.to(device)[:, None] * u[None], N, b)
                qs += w.amplitude * u
            elif w.structure != "plain":
                raise ValueError(w.structure)
            q[bi, g * G : (g + 1) * G] = qs.to(torch.bfloat16)
            k[bi, g] = ks.to(torch.bfloat16)
            v[bi, g] = vs.to(torch.bfloat16)
    return q, k, v


def make_decode(w: Workload, device="cpu", seed: int | None = None, units=None):
    """q [S, Hq, d]; K and V caches [S, Hkv, L, d]; all contiguous bf16.

    ``units`` (a list of (s, g)) draws only those units and returns them
    stacked as [len(units), G, d] / [len(units), L, d] tensors instead, so a
    sample of a large cache can be regenerated on the host."""
    assert w.kind == "decode"
    seed = w.seed if seed is None else seed
    S, Hq, Hkv, L, d, b = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len, w.head_dim, w.block
    G, nb = w.group, w.n_blocks
    todo = units if units is not None else [(s, g) for s in range(S) for g in range(Hkv)]
    if units is None:
        q = torch.empty((S, Hq, d), dtype=torch.bfloat16, device=device)
        kc = torch.empty((S, Hkv, L, d), dtype=torch.bfloat16, device=device)
        vc = torch.empty((S, Hkv, L, d), dtype=torch.bfloat16, device=device)
    else:
        q = torch.empty((len(todo), G, d), dtype=torch.bfloat16, device=device)
        kc = torch.empty((len(todo), L, d), dtype=torch.bfloat16, device=device)
        vc = torch.empty((len(todo), L, d), dtype=torch.bfloat16, device=device)
    for n, (s, g) in enumerate(todo):
        unit = s * Hkv + g
        gen = _gen(device, seed, unit, 1)
        qs = torch.randn((G, d), generator=gen, device=device, dtype=torch.float32)
        ks = _unit_rows(L, d, gen, device)
        vs = _unit_rows(L, d, gen, device)
        if w.structure == "planted":
            u = _directions(nb, d, gen, device)
            ks += w.amplitude * _expand_blocks(u, L, b)
            m = _target_matrix(1, 1, lambda i: nb - 2, 4, _gen("cpu", seed, unit, 2), nb)
            qs += w.amplitude * _aim(m, u)
        elif w.structure != "plain":
            raise ValueError(w.structure)
        if units is None:
            q[s, g * G : (g + 1) * G] = qs.to(torch.bfloat16)
            kc[s, g] = ks.to(torch.bfloat16)
            vc[s, g] = vs.to(torch.bfloat16)
        else:
            q[n] = qs.to(torch.bfloat16)
            kc[n] = ks.to(torch.bfloat16)
            vc[n] = vs.to(torch.bfloat16)
    return q, kc, vc


@dataclass(frozen=True)
class IndexWorkload:
    """Token-level indexer + token-gather attention workload."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    head_dim: int
    n_index_heads: int
    index_dim: int
    topk: int
    clusters: int = 0
    amplitude: float = 0.0
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


INDEX_WORKLOADS = {
    w.name: w
    for w in [
        IndexWorkload("index_tiny_n512", 1, 4, 2, 512, 64, 16, 64, 64, clusters=16, amplitude=4.0, seed=10),
        IndexWorkload("index_n8192", 1, 32, 8, 8192, 128, 16, 128, 64, clusters=128, amplitude=4.0, seed=11),
        IndexWorkload("index_n32768", 1, 32, 8, 32768, 128, 16, 128, 64, clusters=512, amplitude=4.0, seed=12),
    ]
}


def make_index(w: IndexWorkload, device="cpu", seed: int | None = None):
    """qi [B, N, HI, dI] bf16, ki [B, N, dI] bf16, wi [B, N, HI] fp32, and
    Q [B, Hq, N, d], K, V [B, Hkv, N, d] bf16, all contiguous."""
    seed = w.seed if seed is None else seed
    B, N, HI, dI = w.batch, w.seq_len, w.n_index_heads, w.index_dim
    Hq, Hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    qi = torch.empty((B, N, HI, dI), dtype=torch.bfloat16, device=device)
    ki = torch.empty((B, N, dI), dtype=torch.bfloat16, device=device)
    wi = torch.empty((B, N, HI), dtype=torch.float32, device=device)
    q = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        gen = _gen(device, seed, b, 3)
        qs = torch.randn((N, HI, dI), generator=gen, device=device, dtype=torch.float32)
        ks = torch.randn((N, dI), generator=gen, device=device, dtype=torch.float32)
        ws = torch.rand((N, HI), generator=gen, device=device, dtype=torch.float32)
        if w.clusters > 0:
            u = _directions(w.clusters, dI, gen, device)
            cg = _gen("cpu", seed, b, 4)
            member = torch.randint(0, w.clusters, (N,), generator=cg)
            aim = torch.randint(0, w.clusters, (N,), generator=cg)
            ks += w.amplitude * u[member.to(device)]
            qs += w.amplitude * u[aim.to(device)][:, None, :]
        qi[b] = qs.to(torch.bfloat16)
        ki[b] = ks.to(torch.bfloat16)
        wi[b] = ws
        q[b] = torch.randn((Hq, N, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
        k[b] = torch.randn((Hkv, N, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
        v[b] = torch.randn((Hkv, N, d), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
    return qi, ki, wi, q, k, v

