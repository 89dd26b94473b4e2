"""Seeded synthetic workloads for budgeted KV compaction.

This module draws inputs only: random tensors, span placements, tag chains
and tables. It contains none of the method's arithmetic (no attention,
selection, rotation, bonus or quantisation) and is shared by the tests, the
benchmark and the oracle side of parity checks, which all consume the same
drawn tensors.

Draws: K, V and the window queries are i.i.d. N(0,1) rounded to bf16. The
workloads describe keys and queries as RoPE-rotated at their positions; an
isotropic Gaussian is invariant under rotation, so rotated N(0,1) vectors
are again N(0,1) and are drawn directly. Spans are non-overlapping, placed
uniformly at random between the sink tokens and the recent window.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    n_tokens: int
    window: int
    n_sink: int
    n_recent: int
    budget: int
    rope_base: float
    renumber_base: int            # first renumbered position, or -1 to keep positions
    n_spans: int
    span_len: tuple               # (lo, hi) inclusive, or (L, L) for a fixed length
    n_referenced: int             # spans with a future reader; the rest have none
    flat_bonus: bool = False      # every referenced span is needed now (steps_ahead 0)
    definition_back: Optional[int] = None  # place the rank-0 span this many tokens before T
    seed: int = 20261200
    note: str = ""

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def rows(self):
        return self.n_seq * self.n_layers * self.n_kv_heads

    def kv_bytes(self):
        return 2 * self.rows * self.n_tokens * self.head_dim * 2


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, 1, 2, 8, 64, 4096, 16, 4, 64, 512, 1e4, 0, 4, (32, 32), 4, flat_bonus=True,
        seed=20261201,
        note="1 layer, 2 KV heads, GQA 4, d=64, T=4096, W=16, 4 spans of 32 (+1e3), "
             "4 sink + 64 recent, B=512, renumber to 0..511"),
    "qwen3_8b_100k": Workload(
        "qwen3_8b_100k", 1, 36, 8, 32, 128, 100_000, 32, 4, 128, 2048, 1e6, 0, 64, (16, 512), 8,
        seed=20261202,
        note="Qwen3-8B shape (36 layers, 8 KV heads, 32 Q heads, d=128), T=100,000, W=32, "
             "B=2048 with 4 sinks + 128 recent, 64 spans U[16,512], 8 referenced ranked soonest-first, "
             "renumber to 0..2047"),
    "qwen3_8b_1m": Workload(
        "qwen3_8b_1m", 1, 36, 8, 32, 128, 1_048_576, 32, 4, 128, 2048, 1e6, 0, 128, (16, 512), 128,
        definition_back=900_000, seed=20261203,
        note="Qwen3-8B shape, T=1,048,576 (154.6 GB of K+V), processed layer by layer, "
             "128 spans ranked, the rank-0 definition span 900,000 tokens before the query"),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, seed, device="cpu"):
    """i.i.d. N(0,1) rounded to bf16, drawn on `device` from a seeded generator."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    return torch.randn(shape, generator=g, device=dev, dtype=torch.float32 if dev.type == "cpu" else torch.bfloat16).to(torch.bfloat16)


def place_spans(rng, n, lengths, lo, hi, fixed=None):
    """Non-overlapping [start, start+len) spans inside [lo, hi); `fixed` spans
    (start, len) are placed first. Returns a list of (start, length)."""
    spans = list(fixed or [])
    taken = np.zeros(hi, dtype=bool)
    for s, ln in spans:
        taken[s:s + ln] = True
    for ln in lengths:
        for _ in range(10000):
            s = int(rng.integers(lo, hi - ln))
            if not taken[s:s + ln].any():
                taken[s:s + ln] = True
                spans.append((s, int(ln)))
                break
        else:
            raise RuntimeError("could not place span")
    return spans


@dataclass
class SpanTable:
    spans: list                    # [(start, length)] per span k (tag k+1)
    steps_ahead: list              # per span: planned steps until its next reader, or None
    tags: np.ndarray = field(repr=False, default=None)   # uint8 [T] (span k -> tag k+1, 0 = none)

    @property
    def n_tags(self):
        return len(self.spans) + 1


def make_spans(w: Workload) -> SpanTable:
    rng = np.random.default_rng(w.seed + 17)
    lo, hi = w.n_sink, w.n_tokens - w.n_recent
    lens = rng.integers(w.span_len[0], w.span_len[1] + 1, size=w.n_spans)
    fixed = []
    if w.definition_back is not None:
        start = w.n_tokens - w.definition_back
        fixed = [(start, int(lens[0]))]
        lens = lens[1:]
    spans = place_spans(rng, len(lens), lens, lo, hi, fixed)
    n = len(spans)
    if w.flat_bonus:
        steps = [0] * w.n_referenced + [None] * (n - w.n_referenced)
    else:
        # referenced spans get distinct soonest-first ranks 0..n_referenced-1; with a
        # definition span it keeps rank 0 and the rest are shuffled
        ranks = list(range(w.n_referenced))
        order = list(range(n))
        if w.definition_back is None:
            rng.shuffle(order)
            steps = [None] * n
            for k, si in enumerate(order[: w.n_referenced]):
                steps[si] = ranks[k]
        else:
            steps = [None] * n
            steps[0] = 0
            rest = list(range(1, n))
            rng.shuffle(rest)
            for k, si in enumerate(rest[: w.n_referenced - 1]):
                steps[si] = ranks[k + 1]
    tags = np.zeros(w.n_tokens, dtype=np.uint8)
    for k, (s, ln) in enumerate(spans):
        tags[s:s + ln] = k + 1
    assert len(spans) + 1 <= 256
    return SpanTable(spans, steps, tags)


@dataclass
class CompactionInputs:
    w: Workload
    K: torch.Tensor      # bf16 [N][L][Hkv][T][d]
    V: torch.Tensor      # bf16 [N][L][Hkv][T][d]
    Q_obs: torch.Tensor  # bf16 [N][L][Hq][W][d]
    q_dec: torch.Tensor  # bf16 [N][L][Hq][d] one decode query per layer
    spans: SpanTable
    tags: torch.Tensor   # uint8 [N][T]


def make_compaction_inputs(w: Workload, device="cpu", layers=None) -> CompactionInputs:
    """Draw one session's inputs. `layers` restricts the drawn layers (the
    per-layer processing of very long sessions)."""
    L = w.n_layers if layers is None else layers
    N, Hkv, Hq, T, d, W = w.n_seq, w.n_kv_heads, w.n_q_heads, w.n_tokens, w.head_dim, w.window
    K = normal_bf16((N, L, Hkv, T, d), w.seed * 16 + 1, device)
    V = normal_bf16((N, L, Hkv, T, d), w.seed * 16 + 2, device)
    Q = normal_bf16((N, L, Hq, W, d), w.seed * 16 + 3, device)
    qd = normal_bf16((N, L, Hq, d), w.seed * 16 + 4, device)
    sp = make_spans(w)
    tags = torch.from_numpy(np.tile(sp.tags, (N, 1))).to(device)
    return CompactionInputs(w, K, V, Q, qd, sp, tags)


def small_case(T, Hkv=2, Hq=8, d=64, W=16, L=1, N=1, seed=7, device="cpu"):
    """Free-shaped random tensors for parity sweeps (ragged T, other GQA groups)."""
    K = normal_bf16((N, L, Hkv, T, d), seed * 16 + 1, device)
    V = normal_bf16((N, L, Hkv, T, d), seed * 16 + 2, device)
    Q = normal_bf16((N, L, Hq, W, d), seed * 16 + 3, device)
    return K, V, Q


def decode_pools(N, L, Hkv, Hq, d, stride_h, stride_l=0, seed=11, device="cpu"):
    """Random decode inputs: queries, a bf16 pool with per-row token counts in
    [0, stride_h] (the first rows pinned to 0, 1 and stride_h), and optionally an
    int8 pool (codes uniform in [-127, 127], fp16 scales uniform in [1e-3, 3e-2])
    with counts in [0, stride_l]."""
    rows = N * L * Hkv
    rng = np.random.default_rng(seed)
    q = normal_bf16((N, L, Hq, d), seed * 16 + 5, device)
    K = normal_bf16((rows, stride_h, d), seed * 16 + 6, device)
    V = normal_bf16((rows, stride_h, d), seed * 16 + 7, device)
    n_h = rng.integers(0, stride_h + 1, rows)
    n_h[: min(3, rows)] = [0, 1, stride_h][: min(3, rows)]
    out = dict(q=q, K=K, V=V, n_h=torch.from_numpy(n_h.astype(np.int32)).to(device))
    if stride_l:
        n_l = rng.integers(0, stride_l + 1, rows)
        if rows > 3:
            n_l[0] = stride_l          # a row with only int8 tokens
            n_l[3] = 0
        codes = rng.integers(-127, 128, (2, rows, stride_l, d)).astype(np.int8)
        scales = rng.uniform(1e-3, 3e-2, (2, rows, stride_l)).astype(np.float16).view(np.int16)
        out.update(Kq=torch.from_numpy(codes[0]).to(device), Vq=torch.from_numpy(codes[1]).to(device),
                   Ks=torch.from_numpy(scales[0].copy()).to(device),
                   Vs=torch.from_numpy(scales[1].copy()).to(device),
                   n_l=torch.from_numpy(n_l.astype(np.int32)).to(device))
    return out


def page_table(N, n_pages_storage, blocks_per_seq, seed=13):
    """Per sequence, `blocks_per_seq` distinct page ids drawn from the row
    storage's pages, in random order (a paged view of a cache)."""
    rng = np.random.default_rng(seed)
    tbl = np.stack([rng.permutation(n_pages_storage)[:blocks_per_seq] for _ in range(N)])
    return torch.from_numpy(tbl.astype(np.int32))


def kept_and_actions(rows, T, n_keep, seed=17, with_actions=True):
    """Ascending random kept-index lists (n_keep per row, the last row keeping
    fewer) and per-entry actions uniform over {0: release, 1: int8, 2: bf16}."""
    rng = np.random.default_rng(seed)
    kept = np.full((rows, n_keep), -1, np.int32)
    n = np.full(rows, n_keep, np.int32)
    n[-1] = n_keep // 2
    for r in range(rows):
        kept[r, : n[r]] = np.sort(rng.choice(T, n[r], replace=False))
    act = rng.integers(0, 3, (rows, n_keep)).astype(np.uint8) if with_actions else None
    return kept, n, act
