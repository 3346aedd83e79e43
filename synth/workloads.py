"""Seeded synthetic inputs for the five workloads of the verify/build hot path.

Every array is drawn from numpy PCG64 streams keyed by ``SeedSequence(seed,
spawn_key=...)``.  Sequence b of a verify workload uses key (0, b) and its
hidden rows in a build workload use key (3, b), so any subset of sequences
regenerates to the same values without drawing the rest.  Batch-wide
quantities come from key (1,) (vocabulary ranks) and key (2,) (prompt
lengths, block tables, h_shared, the MASK id).

Workloads (the shapes and distributions of the speculative-decoding settings on
the pages: K=7 drafts and up to 1024 concurrent sequences as in the vLLM serve
command of the P-EAGLE blog summary, vocabularies of GPT-OSS / Qwen3 size):

  1 tiny verify        B=1,  K=3, V=32,     fp32 logits 2*N(0,1), T=1.0
  2 verify mid         B=8,  K=5, V=32000,  fp32 logits 3*N(0,1) with one +6
                       boosted token per row, T=1.0
  3 P-EAGLE build      B=64, K=7, H=2880 bf16, prompt lengths U{32..2048},
                       accepted counts U{0..7}
  4 verify large vocab B=64, K=7, V=201088, bf16 logits 3*N(0,1) + 6/rank(v),
                       T=0.7
  5 fused step         B=1024, K=7, V=151936 as workload 4, then the build with
                       H=2048 bf16, prompt lengths U{64..8192}

The draft distribution q of row k is the drafter's own distribution: the
stored target row plus Gaussian noise, divided by the drafter's temperature,
exponentiated and normalised in fp64, then stored as fp32.  Draft tokens are
drawn from it with ``Generator.choice``.  The test uniforms are fp32 in [0, 1).
"""
from __future__ import annotations

import dataclasses
import multiprocessing as mp
import os
from typing import Optional, Sequence

import numpy as np

CONFIG_NAMES = {
    1: "tiny-verify",
    2: "verify-mid",
    3: "peagle-build",
    4: "verify-large-vocab",
    5: "fused-high-concurrency",
}


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- specs
@dataclasses.dataclass(frozen=True)
class VerifySpec:
    config: int
    B: int
    K: int
    V: int
    dtype: str            # "f32" or "bf16" target logits
    sigma: float          # logits = sigma * N(0,1) + boost
    boost: str            # "none" | "one-token" | "zipf-head"
    temperature: float    # target sampling temperature
    draft_noise: float    # sigma of the drafter's perturbation
    draft_temperature: float
    seed: int


@dataclasses.dataclass(frozen=True)
class BuildSpec:
    config: int
    B: int
    K: int
    H: int
    V: int                # target vocabulary (MASK id lies outside it)
    L_min: int
    L_max: int
    block_size: int
    seed: int
    synth_accept: bool    # True: draw accepted counts / tokens here (workload 3)


def verify_config(n: int) -> VerifySpec:
    if n == 1:
        return VerifySpec(1, 1, 3, 32, "f32", 2.0, "none", 1.0, 0.5, 1.0, 1)
    if n == 2:
        return VerifySpec(2, 8, 5, 32000, "f32", 3.0, "one-token", 1.0, 1.0, 1.0, 2)
    if n == 4:
        return VerifySpec(4, 64, 7, 201088, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7, 4)
    if n == 5:
        return VerifySpec(5, 1024, 7, 151936, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7, 5)
    raise ValueError(f"workload {n} has no verify part")


def build_config(n: int) -> BuildSpec:
    if n == 3:
        return BuildSpec(3, 64, 7, 2880, 201088, 32, 2048, 16, 3, True)
    if n == 5:
        return BuildSpec(5, 1024, 7, 2048, 151936, 64, 8192, 16, 5, False)
    raise ValueError(f"workload {n} has no build part")


# ---------------------------------------------------------------- streams
def _seq_rng(seed: int, b: int, tag: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, b))))


def _global_rng(seed: int, tag: int = 1) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag,))))


def _zipf_head(spec) -> np.ndarray:
    """6 / rank(v) with rank from one seeded permutation of the vocabulary."""
    g = _global_rng(spec.seed)
    perm = g.permutation(spec.V)                 # perm[r] = token of rank r+1
    head = np.empty(spec.V, dtype=np.float32)
    head[perm] = (6.0 / np.arange(1, spec.V + 1, dtype=np.float64)).astype(np.float32)
    return head


# ---------------------------------------------------------------- verify inputs
@dataclasses.dataclass
class VerifyInputs:
    spec: VerifySpec
    seqs: np.ndarray              # which sequences of the workload these rows are
    logits: np.ndarray            # [n, K+1, V] float32, or uint16 bf16 bits
    draft_probs: np.ndarray       # [n, K, V] float32
    draft_tokens: np.ndarray      # [n, K] int32
    uniforms: np.ndarray          # [n, K+1] float32

    @property
    def temperature(self) -> float:
        return self.spec.temperature

    def logits_f64(self, i: int) -> np.ndarray:
        """Stored logits of sequence i widened exactly to fp64 (for checks)."""
        z = self.logits[i]
        if self.spec.dtype == "bf16":
            z = bf16_bits_to_f32(z)
        return z.astype(np.float64)


def _draw_verify_seq(spec: VerifySpec, b: int, head: Optional[np.ndarray]):
    K, V = spec.K, spec.V
    rng = _seq_rng(spec.seed, b)
    z = rng.standard_normal((K + 1, V), dtype=np.float32)
    z *= np.float32(spec.sigma)
    if spec.boost == "one-token":
        idx = rng.integers(0, V, size=K + 1)
        z[np.arange(K + 1), idx] += np.float32(6.0)
    elif spec.boost == "zipf-head":
        z += head[None, :]
    if spec.dtype == "bf16":
        stored = f32_to_bf16_bits(z)
        seen = bf16_bits_to_f32(stored).astype(np.float64)
    else:
        stored = z
        seen = z.astype(np.float64)
    # the drafter's distribution: perturbed target row at the drafter's temperature
    noise = rng.standard_normal((K, V), dtype=np.float32).astype(np.float64)
    x = (seen[:K] + spec.draft_noise * noise) / spec.draft_temperature
    x -= x.max(axis=1, keepdims=True)
    np.exp(x, out=x)
    x /= x.sum(axis=1, keepdims=True)
    q = x.astype(np.float32)
    d = np.array([rng.choice(V, p=x[k]) for k in range(K)], dtype=np.int32)
    u = rng.random(K + 1, dtype=np.float32)
    return stored, q, d, u


def _verify_worker(args):
    spec, seqs = args
    head = _zipf_head(spec) if spec.boost == "zipf-head" else None
    return [(b,) + _draw_verify_seq(spec, b, head) for b in seqs]


def _workers(n_items: int, workers: Optional[int]) -> int:
    if workers is not None:
        return max(1, workers)
    if n_items < 64:
        return 1
    return max(1, min(16, os.cpu_count() or 1))


def make_verify_inputs(spec: VerifySpec, seqs: Optional[Sequence[int]] = None,
                       workers: Optional[int] = None) -> VerifyInputs:
    """Draw the verify inputs of ``spec`` (all sequences, or the subset ``seqs``).

    Large draws run in a pool of freshly spawned worker processes (none of them
    touches a GPU); the result does not depend on the number of workers.
    """
    seqs = np.arange(spec.B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    n, K, V = len(seqs), spec.K, spec.V
    ldt = np.uint16 if spec.dtype == "bf16" else np.float32
    logits = np.empty((n, K + 1, V), dtype=ldt)
    q = np.empty((n, K, V), dtype=np.float32)
    d = np.empty((n, K), dtype=np.int32)
    u = np.empty((n, K + 1), dtype=np.float32)
    pos = {int(b): i for i, b in enumerate(seqs)}
    nw = _workers(n, workers)
    if nw == 1:
        results = [_verify_worker((spec, [int(b) for b in seqs]))]
    else:
        chunks = [[int(b) for b in seqs[i::nw]] for i in range(nw)]
        ctx = mp.get_context("spawn")
        with ctx.Pool(nw) as pool:
            results = pool.map(_verify_worker, [(spec, c) for c in chunks])
    for res in results:
        for b, zs, qs, ds, us in res:
            i = pos[b]
            logits[i], q[i], d[i], u[i] = zs, qs, ds, us
    return VerifyInputs(spec, seqs, logits, q, d, u)


# ---------------------------------------------------------------- build inputs
@dataclasses.dataclass
class BuildInputs:
    spec: BuildSpec
    start_pos: np.ndarray         # [B] int64, L_b = position of verify slot 0
    block_table: np.ndarray       # [B, max_blocks] int32, -1 past the sequence's blocks
    target_hidden: np.ndarray     # [B*(K+1), H] uint16 bf16 bits
    h_shared: np.ndarray          # [H] uint16 bf16 bits
    mask_token_id: int
    # workload 3 draws the verify outcome here; workload 5 takes it from verify
    draft_tokens: Optional[np.ndarray] = None      # [B, K] int32
    out_tokens: Optional[np.ndarray] = None        # [B, K+1] int32
    num_accepted: Optional[np.ndarray] = None      # [B] int32

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def make_build_inputs(spec: BuildSpec) -> BuildInputs:
    B, K, H, bs = spec.B, spec.K, spec.H, spec.block_size
    g = _global_rng(spec.seed, tag=2)
    L = g.integers(spec.L_min, spec.L_max + 1, size=B).astype(np.int64)
    nblk = (L + 2 * K + bs - 1) // bs
    pool = g.permutation(int(nblk.sum())).astype(np.int32)
    maxb = int(nblk.max())
    bt = np.full((B, maxb), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, : nblk[b]] = pool[off: off + nblk[b]]
        off += int(nblk[b])
    h_shared = f32_to_bf16_bits(g.standard_normal(H, dtype=np.float32))
    mask_id = int(spec.V + g.integers(1, 1024))
    hid = np.empty((B * (K + 1), H), dtype=np.uint16)
    d = out = a = None
    if spec.synth_accept:
        d = np.empty((B, K), dtype=np.int32)
        out = np.full((B, K + 1), -1, dtype=np.int32)
        a = np.empty(B, dtype=np.int32)
    for b in range(B):
        rng = _seq_rng(spec.seed, b, tag=3)
        hid[b * (K + 1):(b + 1) * (K + 1)] = f32_to_bf16_bits(
            rng.standard_normal((K + 1, H), dtype=np.float32))
        if spec.synth_accept:
            ab = int(rng.integers(0, K + 1))
            d[b] = rng.integers(0, spec.V, size=K)
            cb = int(rng.integers(0, spec.V))
            a[b] = ab
            out[b, :ab] = d[b, :ab]
            out[b, ab] = cb
    return BuildInputs(spec, L, bt, hid, h_shared, mask_id, d, out, a)


def make_fused_inputs(workers: Optional[int] = None):
    """Workload 5: verify inputs, and build inputs whose accept outcome and
    draft tokens come from the verify step on the same device."""
    vi = make_verify_inputs(verify_config(5), workers=workers)
    bi = make_build_inputs(build_config(5))
    bi.draft_tokens = vi.draft_tokens
    return vi, bi



# ---------------------------------------------------------------- drafter outputs
@dataclasses.dataclass(frozen=True)
class DraftSpec:
    """Drafter prediction rows to be sampled into the next verify's drafts.

    rows_per_seq = K: the logits hold exactly the K prediction rows of each
    sequence (row b*K + k).  rows_per_seq > K: the logits hold every row of
    the drafter batch and ``row_index`` picks K distinct rows per sequence.
    mixed: per-sequence temperatures from {0 (greedy), 0.5, 0.7, 1.0, 1.3}.
    """
    name: str
    B: int
    K: int
    V: int
    dtype: str
    sigma: float
    boost: str
    temperature: float
    rows_per_seq: int
    mixed: bool
    seed: int


DRAFT_CONFIGS = {
    "draft-tiny": DraftSpec("draft-tiny", 2, 3, 32, "f32", 2.0, "none", 1.0, 3, False, 11),
    "draft-ragged": DraftSpec("draft-ragged", 5, 4, 30011, "bf16", 3.0, "zipf-head", 0.7, 8,
                              True, 12),
    "draft-mid": DraftSpec("draft-mid", 48, 7, 151936, "bf16", 3.0, "zipf-head", 0.7, 7, False, 13),
}


@dataclasses.dataclass
class DraftInputs:
    spec: DraftSpec
    logits: np.ndarray                  # [B*rows_per_seq, V] float32 or uint16 bf16 bits
    uniforms: np.ndarray                # [B, K] float32
    row_index: Optional[np.ndarray]     # [B, K] int32, or None (row b*K + k)
    temperatures: Optional[np.ndarray]  # [B] float32, or None (the scalar temperature)

    @property
    def temperature(self) -> float:
        return self.spec.temperature


def make_draft_inputs(spec: DraftSpec) -> DraftInputs:
    B, K, V, R = spec.B, spec.K, spec.V, spec.rows_per_seq
    head = _zipf_head(spec) if spec.boost == "zipf-head" else None
    ldt = np.uint16 if spec.dtype == "bf16" else np.float32
    logits = np.empty((B * R, V), dtype=ldt)
    u = np.empty((B, K), dtype=np.float32)
    rows = np.empty((B, K), dtype=np.int32) if R > K else None
    temps = np.empty(B, dtype=np.float32) if spec.mixed else None
    for b in range(B):
        rng = _seq_rng(spec.seed, b, tag=4)
        z = rng.standard_normal((R, V), dtype=np.float32)
        z *= np.float32(spec.sigma)
        if head is not None:
            z += head[None, :]
        logits[b * R:(b + 1) * R] = f32_to_bf16_bits(z) if spec.dtype == "bf16" else z
        u[b] = rng.random(K, dtype=np.float32)
        if rows is not None:
            rows[b] = b * R + rng.choice(R, size=K, replace=False)
        if temps is not None:
            temps[b] = np.float32(rng.choice([0.0, 0.5, 0.7, 1.0, 1.3]))
    return DraftInputs(spec, logits, u, rows, temps)


# ---------------------------------------------------------------- mixed batches
MIXED_TEMPERATURES = (0.0, 0.5, 0.7, 1.0, 1.3)


def make_temperatures(B: int, seed: int,
                      choices: Sequence[float] = MIXED_TEMPERATURES) -> np.ndarray:
    """Per-sequence temperatures [B] fp32 for a mixed serving batch: each
    sequence draws one of ``choices`` (0 = a greedy request) from its own
    stream, key (5, b)."""
    out = np.empty(B, dtype=np.float32)
    for b in range(B):
        out[b] = np.float32(_seq_rng(seed, b, tag=5).choice(np.asarray(choices, np.float64)))
    return out


# ---------------------------------------------------------------- draft trees
@dataclasses.dataclass(frozen=True)
class TreeSpec:
    """Draft trees of N nodes per sequence (node 0 = the root).

    shape "chain": node i's parent is i-1; "static": one branching shape for
    every sequence, widths per depth; "random": per sequence, node i picks
    its parent uniformly among the last few nodes.  Children are drawn
    independently from their parent's draft row.
    """
    name: str
    B: int
    N: int
    V: int
    dtype: str
    sigma: float
    boost: str
    temperature: float
    draft_noise: float
    draft_temperature: float
    shape: str
    widths: tuple
    seed: int


TREE_CONFIGS = {
    "tree-tiny": TreeSpec("tree-tiny", 3, 6, 32, "f32", 2.0, "none", 1.0, 0.5, 1.0, "random", (),
                          21),
    "tree-mid": TreeSpec("tree-mid", 16, 15, 32000, "f32", 3.0, "one-token", 1.0, 1.0, 1.0,
                         "static", (3, 2, 1), 22),
    "tree-large": TreeSpec("tree-large", 64, 15, 151936, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7,
                           "static", (3, 2, 1), 23),
    "tree-bench": TreeSpec("tree-bench", 256, 15, 151936, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7,
                           "static", (3, 2, 1), 24),
}


def static_tree_parents(widths: Sequence[int]) -> np.ndarray:
    """Parents of a tree in which every node at depth d has widths[d] children
    (breadth-first numbering; node 0 is the root)."""
    parents, level = [], [0]
    for w in widths:
        nxt = []
        for p in level:
            for _ in range(w):
                parents.append(p)
                nxt.append(len(parents))
        level = nxt
    return np.asarray(parents, dtype=np.int32)


@dataclasses.dataclass
class TreeInputs:
    spec: TreeSpec
    logits: np.ndarray        # [B, N+1, V] float32 or uint16 bf16 bits
    draft_probs: np.ndarray   # [B, N+1, V] float32: row n drafted node n's children
    parents: np.ndarray       # [B, N] int32
    tokens: np.ndarray        # [B, N] int32
    uniforms: np.ndarray      # [B, N+1] float32: [:, i] tests node i, [:, 0] the final draw

    @property
    def temperature(self) -> float:
        return self.spec.temperature


def _tree_seq(spec: TreeSpec, b: int, head: Optional[np.ndarray], static: Optional[np.ndarray]):
    N, V = spec.N, spec.V
    rng = _seq_rng(spec.seed, b, tag=6)
    z = rng.standard_normal((N + 1, V), dtype=np.float32)
    z *= np.float32(spec.sigma)
    if spec.boost == "one-token":
        z[np.arange(N + 1), rng.integers(0, V, size=N + 1)] += np.float32(6.0)
    elif head is not None:
        z += head[None, :]
    if spec.dtype == "bf16":
        stored = f32_to_bf16_bits(z)
        seen = bf16_bits_to_f32(stored).astype(np.float64)
    else:
        stored = z
        seen = z.astype(np.float64)
    noise = rng.standard_normal((N + 1, V), dtype=np.float32).astype(np.float64)
    x = (seen + spec.draft_noise * noise) / spec.draft_temperature
    x -= x.max(axis=1, keepdims=True)
    np.exp(x, out=x)
    x /= x.sum(axis=1, keepdims=True)
    if spec.shape == "chain":
        par = np.arange(N, dtype=np.int32)
    elif static is not None:
        par = static
    else:
        par = np.array([int(rng.integers(max(0, i - 3), i)) for i in range(1, N + 1)],
                       dtype=np.int32)
    tok = np.array([rng.choice(V, p=x[par[i]]) for i in range(N)], dtype=np.int32)
    u = rng.random(N + 1, dtype=np.float32)
    return b, stored, x.astype(np.float32), par, tok, u


def _tree_worker(args):
    spec, seqs = args
    head = _zipf_head(spec) if spec.boost == "zipf-head" else None
    static = static_tree_parents(spec.widths) if spec.shape == "static" else None
    return [_tree_seq(spec, b, head, static) for b in seqs]


def make_tree_inputs(spec: TreeSpec, workers: Optional[int] = None) -> TreeInputs:
    """Draw the tree inputs of ``spec``; large draws use a pool of freshly
    spawned processes (the values do not depend on the number of workers)."""
    B, N, V = spec.B, spec.N, spec.V
    if spec.shape == "static":
        assert static_tree_parents(spec.widths).size == N
    ldt = np.uint16 if spec.dtype == "bf16" else np.float32
    logits = np.empty((B, N + 1, V), dtype=ldt)
    q = np.empty((B, N + 1, V), dtype=np.float32)
    parents = np.empty((B, N), dtype=np.int32)
    tokens = np.empty((B, N), dtype=np.int32)
    u = np.empty((B, N + 1), dtype=np.float32)
    nw = _workers(B, workers)
    if nw == 1:
        results = [_tree_worker((spec, list(range(B))))]
    else:
        ctx = mp.get_context("spawn")
        with ctx.Pool(nw) as pool:
            results = pool.map(_tree_worker, [(spec, list(range(i, B, nw))) for i in range(nw)])
    for res in results:
        for b, zs, qs, ps, ts, us in res:
            logits[b], q[b], parents[b], tokens[b], u[b] = zs, qs, ps, ts, us
    return TreeInputs(spec, logits, q, parents, tokens, u)
