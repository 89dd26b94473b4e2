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


# ---------------------------------------------------------------- PASK-style mixed precision

@dataclass(frozen=True)
class PaskWorkload:
    """Batch of structured-generation requests: a prompt compacted by window
    scoring, then generated tokens whose structural tags drive per-layer-group
    release / int8 / bf16 actions."""
    name: str = "pask_llama3_8b"
    n_seq: int = 64
    n_layers: int = 32
    n_groups: int = 4
    n_kv_heads: int = 8
    n_q_heads: int = 32
    head_dim: int = 128
    n_prompt: int = 4096
    n_gen: int = 1024
    window: int = 32
    n_sink: int = 4
    n_recent: int = 128          # prompt tokens protected at the end of the prompt
    budget: int = 1365           # prompt tokens kept per row
    gen_recent: int = 128        # last generated tokens held in bf16 whatever their action
    n_tags: int = 8
    stay: float = 5.0 / 6.0      # Markov chain: P(next tag = current tag); mean run 6
    n_critical: int = 2
    budget_fraction: float = 1.0 / 3.0
    rope_base: float = 5e5
    seed: int = 20261204
    low_bits: int = 8            # low tier: 8 = int8, 4 = INT4 (two nibbles per byte)

    @property
    def rows(self):
        return self.n_seq * self.n_layers * self.n_kv_heads


PASK_WORKLOADS = {
    "pask_llama3_8b": PaskWorkload(),
    # same structure at a size the float64 oracle checks row by row in seconds
    "pask_small": PaskWorkload("pask_small", n_seq=3, n_layers=4, n_groups=4, n_kv_heads=2, n_q_heads=8,
                               head_dim=128, n_prompt=640, n_gen=300, window=16, n_recent=32,
                               budget=213, gen_recent=32, seed=20261214),
    # the pages' own low tier: INT4
    "pask_llama3_8b_int4": PaskWorkload("pask_llama3_8b_int4", low_bits=4),
    "pask_small_int4": PaskWorkload("pask_small_int4", n_seq=3, n_layers=4, n_groups=4, n_kv_heads=2,
                                    n_q_heads=8, head_dim=128, n_prompt=640, n_gen=300, window=16,
                                    n_recent=32, budget=213, gen_recent=32, seed=20261224, low_bits=4),
}


def tag_chain(rng, n_seq, n_tok, n_tags, stay):
    """Per sequence an n_tags-state Markov chain: the first tag uniform, then the
    same tag with probability `stay`, else uniform over the other tags."""
    tags = np.zeros((n_seq, n_tok), np.uint8)
    for n in range(n_seq):
        z = int(rng.integers(0, n_tags))
        moves = rng.random(n_tok) >= stay
        jumps = rng.integers(1, n_tags, n_tok)
        for t in range(n_tok):
            if t and moves[t]:
                z = (z + int(jumps[t])) % n_tags
            tags[n, t] = z
    return tags


def pask_table(rng, n_tags, n_groups, n_critical):
    """Frozen [tag x layer group] table: base action a0 uniform over {R, L, H},
    floor amin <= a0, upgrade priorities U(0,1) for R->L and L->H, and
    `n_critical` critical tags."""
    a0 = rng.integers(0, 3, (n_tags, n_groups)).astype(np.uint8)
    amin = np.minimum(a0, rng.integers(0, 3, (n_tags, n_groups))).astype(np.uint8)
    prio = rng.random((n_tags, n_groups, 2)).astype(np.float32)
    crit = np.zeros(n_tags, np.uint8)
    crit[rng.choice(n_tags, n_critical, replace=False)] = 1
    return a0, amin, prio, crit


@dataclass
class PaskInputs:
    w: PaskWorkload
    K: torch.Tensor       # bf16 [N][L][Hkv][n_prompt][d] prompt keys
    V: torch.Tensor
    Q_obs: torch.Tensor   # bf16 [N][L][Hq][W][d] last W prompt queries
    K_gen: torch.Tensor   # bf16 [N][L][Hkv][n_gen][d] generated tokens' keys
    V_gen: torch.Tensor
    q_dec: torch.Tensor   # bf16 [N][L][Hq][d] query at position n_prompt + n_gen
    tags: np.ndarray      # uint8 [N][n_gen]
    a0: np.ndarray
    amin: np.ndarray
    prio: np.ndarray
    critical: np.ndarray


def make_pask_inputs(w: PaskWorkload, device="cpu") -> PaskInputs:
    N, L, Hkv, Hq, d = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim
    s = w.seed * 16
    K = normal_bf16((N, L, Hkv, w.n_prompt, d), s + 1, device)
    V = normal_bf16((N, L, Hkv, w.n_prompt, d), s + 2, device)
    Q = normal_bf16((N, L, Hq, w.window, d), s + 3, device)
    Kg = normal_bf16((N, L, Hkv, w.n_gen, d), s + 4, device)
    Vg = normal_bf16((N, L, Hkv, w.n_gen, d), s + 5, device)
    qd = normal_bf16((N, L, Hq, d), s + 6, device)
    rng = np.random.default_rng(w.seed + 29)
    tags = tag_chain(rng, N, w.n_gen, w.n_tags, w.stay)
    a0, amin, prio, crit = pask_table(rng, w.n_tags, w.n_groups, w.n_critical)
    return PaskInputs(w, K, V, Q, Kg, Vg, qd, tags, a0, amin, prio, crit)


# ---------------------------------------------------------------- CommitKV-style page lifecycle

@dataclass(frozen=True)
class CommitWorkload:
    """Agent trajectories at a tool-call commit: T_pre cached tokens in pages,
    a pre-commit query window at the end of the tool call, an appended
    observation, and a post-commit window. Planted "completion" pages have
    keys aligned with the pre-commit queries and opposed to the post-commit
    ones (logit shift +-plant_logit)."""
    name: str = "commitkv_28l"
    n_seq: int = 16
    n_layers: int = 28
    n_kv_heads: int = 4
    n_q_heads: int = 28
    head_dim: int = 128
    n_pre: int = 32_768          # tokens before the commit (tool call ends at n_pre - 1)
    n_obs: int = 512             # appended observation
    window: int = 32             # W of both windows; the post-commit window is cached too
    page_size: int = 16
    n_planted: int = 64
    plant_logit: float = 9.0     # c^2 / sqrt(d): c = sqrt(plant_logit * sqrt(d))
    budget: int = 4096           # tokens retained at the checkpoint
    layer: int = 27              # the attention layer whose effects decide
    tau_use: float = 0.05
    tau_dead: float = 1e-3
    rho_use: float = 0.75
    rho_dead: float = 0.25
    tau_joint: float = 1e-2
    max_scan: int = 64
    seed: int = 20261205
    event_max: int = 0           # > 0: the history is a run of events of 1..event_max tokens (event pages)

    @property
    def n_tokens(self):
        return self.n_pre + self.n_obs + self.window

    @property
    def q_first_pre(self):
        return self.n_pre - self.window

    @property
    def q_first_post(self):
        return self.n_pre + self.n_obs

    @property
    def n_eligible(self):
        """Complete pages lying wholly before the pre-commit window (uniform pages)."""
        return self.q_first_pre // self.page_size

    @property
    def n_pages_all(self):
        """Pages of the whole cache (uniform pages)."""
        return self.n_tokens // self.page_size

    @property
    def rows(self):
        return self.n_seq * self.n_layers * self.n_kv_heads


COMMIT_WORKLOADS = {
    "commitkv_28l": CommitWorkload(),
    "commitkv_small": CommitWorkload("commitkv_small", n_seq=2, n_layers=3, n_kv_heads=2, n_q_heads=6,
                                     n_pre=1024, n_obs=96, window=16, n_planted=6, budget=320, layer=2,
                                     max_scan=8, seed=20261215),
    # the same commits on event pages: history events of 1..40 tokens, pages of at most 16
    "commitkv_events": CommitWorkload("commitkv_events", event_max=40, seed=20261235),
    "commitkv_events_small": CommitWorkload("commitkv_events_small", n_seq=2, n_layers=3, n_kv_heads=2,
                                            n_q_heads=6, n_pre=1024, n_obs=96, window=16, n_planted=6,
                                            budget=320, layer=2, max_scan=8, seed=20261247, event_max=40),
}


@dataclass
class CommitInputs:
    w: CommitWorkload
    K: torch.Tensor        # bf16 [N][L][Hkv][T][d], T = n_pre + n_obs + W
    V: torch.Tensor
    Q_pre: torch.Tensor    # bf16 [N][L][Hq][W][d] at positions n_pre-W .. n_pre-1
    Q_post: torch.Tensor   # bf16 [N][L][Hq][W][d] at positions n_pre+n_obs .. T-1
    q_dec: torch.Tensor    # bf16 [N][L][Hq][d] at position T
    planted: np.ndarray    # uniform pages: int64 [N][n_planted] ascending page indices;
                           # events: int64 [N][n_planted][2] (first token, length) of the planted events
    events: Optional[np.ndarray] = None   # events: int32 [N][n_events] event lengths from token 0 to T


def _history_events(w: CommitWorkload):
    """Event lengths of every trajectory's history (tokens 0 .. q_first_pre):
    one draw of lengths U[1, event_max] (the last one cut to end at the
    pre-commit window), shuffled per trajectory, so that every trajectory
    has the same events in its own order (and the same page count). Then
    the pre-commit window (the end of the tool call), the observation and
    the post-commit window as one event each."""
    rng = np.random.default_rng(w.seed + 41)
    base, total = [], 0
    while total < w.q_first_pre:
        base.append(int(rng.integers(1, w.event_max + 1)))
        total += base[-1]
    base[-1] -= total - w.q_first_pre
    hist = [np.asarray(base)] + [rng.permutation(base) for _ in range(w.n_seq - 1)]
    tail = [w.window, w.n_obs, w.window]
    return np.stack([np.concatenate([h, tail]) for h in hist]).astype(np.int32), len(base)


def make_commit_inputs(w: CommitWorkload, device="cpu") -> CommitInputs:
    """Uniform pages: n_planted of the eligible pages are completion pages.
    Event pages (w.event_max > 0): n_planted history events of page_size/2 ..
    page_size tokens (one page each) are completion events."""
    N, L, Hkv, Hq, d, T, W = (w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim,
                              w.n_tokens, w.window)
    G = Hq // Hkv
    s = w.seed * 16
    K = normal_bf16((N, L, Hkv, T, d), s + 1, device)
    V = normal_bf16((N, L, Hkv, T, d), s + 2, device)
    Qm = normal_bf16((N, L, Hq, W, d), s + 3, device)
    Qp = normal_bf16((N, L, Hq, W, d), s + 4, device)
    qd = normal_bf16((N, L, Hq, d), s + 5, device)
    rng = np.random.default_rng(w.seed + 31)
    ps = w.page_size
    events = None
    if w.event_max:
        events, n_hist = _history_events(w)
        spans = []
        for n in range(N):
            start = np.concatenate([[0], np.cumsum(events[n][:n_hist])[:-1]])
            ok = np.flatnonzero((events[n][:n_hist] >= (ps + 1) // 2) & (events[n][:n_hist] <= ps))
            if ok.size < w.n_planted:
                raise ValueError(f"{w.name}: {ok.size} events of {(ps + 1) // 2}..{ps} tokens, "
                                 f"{w.n_planted} to plant")
            pick = np.sort(rng.choice(ok, w.n_planted, replace=False))
            spans.append(np.stack([start[pick], events[n][pick]], axis=1))
        planted = np.stack(spans).astype(np.int64)
    else:
        planted = np.stack([np.sort(rng.choice(w.n_eligible, w.n_planted, replace=False)) for _ in range(N)])
    u = rng.standard_normal((N, L, Hkv, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    c = float(np.sqrt(w.plant_logit * np.sqrt(d)))
    cu = torch.from_numpy(c * u).to(device=device, dtype=torch.float32)        # [N][L][Hkv][d]
    for n in range(N):
        if w.event_max:
            tok = np.concatenate([np.arange(f, f + ln) for f, ln in planted[n]])
            idx = torch.from_numpy(tok).to(device)
            sel = K[n].index_select(2, idx).float() + cu[n][:, :, None, :]
            K[n].index_copy_(2, idx, sel.to(torch.bfloat16))
        else:
            Kn = K[n].view(L, Hkv, T // ps, ps, d)
            idx = torch.from_numpy(planted[n]).to(device)
            sel = Kn.index_select(2, idx).float() + cu[n][:, :, None, None, :]
            Kn.index_copy_(2, idx, sel.to(torch.bfloat16))
    cq = cu.repeat_interleave(G, dim=2)[:, :, :, None, :]                        # [N][L][Hq][1][d]
    Qm = (Qm.float() + cq).to(torch.bfloat16)
    Qp = (Qp.float() - cq).to(torch.bfloat16)
    return CommitInputs(w, K, V, Qm, Qp, qd, planted, events)


# ---------------------------------------------------------------- PACE-style H2O decode with eviction

@dataclass(frozen=True)
class H2OWorkload:
    """A resident cache of B + E slots per (layer, KV head) in decode: every
    cycle decodes E tokens (each step's query attends to the resident slots
    and the new tokens so far, adding its attention to the slots' cumulative
    scores), then evicts back to B slots by cumulative score plus the
    foresight bonus of the slot's span tag."""
    name: str = "pace_h2o_decode"
    n_seq: int = 1
    n_layers: int = 36
    n_kv_heads: int = 8
    n_q_heads: int = 32
    head_dim: int = 128
    budget: int = 2048
    interval: int = 32           # E: decoded tokens between evictions
    n_sink: int = 4
    n_recent: int = 128
    n_spans: int = 8             # tagged span groups among the resident slots
    span_slots: int = 24         # slots per tagged group per row
    key_sigma: float = 0.5       # per-slot key scale ~ lognormal(0, key_sigma): uneven attention
    rope_base: float = 1e6
    seed: int = 20261206
    limit: int = 0               # bounded positions: physical positions stay below L (0: positions kept)

    @property
    def rows(self):
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def slots(self):
        return self.budget + self.interval


H2O_WORKLOADS = {
    "pace_h2o_decode": H2OWorkload(),
    "h2o_small": H2OWorkload("h2o_small", n_layers=2, n_kv_heads=2, n_q_heads=8, head_dim=64, budget=96,
                             interval=8, n_recent=8, n_spans=3, span_slots=6, seed=20261216),
    # PACE's bounded positions on top: L = 8,192, renumbered with the reference store
    "pace_h2o_bounded": H2OWorkload("pace_h2o_bounded", limit=8192),
    "h2o_small_bounded": H2OWorkload("h2o_small_bounded", n_layers=2, n_kv_heads=2, n_q_heads=8, head_dim=64,
                                     budget=96, interval=8, n_recent=8, n_spans=3, span_slots=6, seed=20261226,
                                     limit=128),
}


@dataclass
class H2OInputs:
    w: H2OWorkload
    K: torch.Tensor        # bf16 [rows][B + E][d] resident keys (slots >= B: this cycle's new tokens)
    V: torch.Tensor
    pos: torch.Tensor      # int32 [rows][B + E] physical positions
    acc: torch.Tensor      # fp32 [rows][B + E] cumulative scores of the resident slots (new: 0)
    tags: torch.Tensor     # uint8 [rows][B + E] span tag per slot (0: none)
    q: torch.Tensor        # bf16 [cycles][E][N][L][Hq][d] decode queries
    K_new: torch.Tensor    # bf16 [cycles][rows][E][d] keys of the tokens decoded in each cycle
    V_new: torch.Tensor
    steps_ahead: tuple     # per tag 1..n_spans: steps until its next planned reader


def make_h2o_inputs(w: H2OWorkload, cycles, device="cpu") -> H2OInputs:
    rows, S, d, B, E = w.rows, w.slots, w.head_dim, w.budget, w.interval
    s = w.seed * 16
    g = _gen(s + 7, torch.device(device))
    scale = torch.exp(w.key_sigma * torch.randn((rows, S, 1), generator=g, device=device))
    K = (normal_bf16((rows, S, d), s + 1, device).float() * scale).to(torch.bfloat16)
    V = normal_bf16((rows, S, d), s + 2, device)
    q = normal_bf16((cycles, E, w.n_seq, w.n_layers, w.n_q_heads, d), s + 3, device)
    gn = _gen(s + 8, torch.device(device))
    sn = torch.exp(w.key_sigma * torch.randn((cycles, rows, E, 1), generator=gn, device=device))
    K_new = (normal_bf16((cycles, rows, E, d), s + 4, device).float() * sn).to(torch.bfloat16)
    V_new = normal_bf16((cycles, rows, E, d), s + 5, device)
    rng = np.random.default_rng(w.seed + 37)
    span = w.limit - 2 * E - 16 if w.limit else 8 * S     # history positions below the limit when bounded
    pos = np.stack([np.sort(rng.choice(span, B, replace=False)) for _ in range(rows)]) + 16
    pos = np.concatenate([pos, np.tile(np.arange(span + 16, span + 16 + E), (rows, 1))], axis=1)
    acc = rng.gamma(0.5, 4.0, (rows, S))
    acc[:, B:] = 0.0
    tags = np.zeros((rows, S), np.uint8)
    lo, hi = w.n_sink, B - w.n_recent
    for r in range(rows):
        slots = rng.choice(np.arange(lo, hi), w.n_spans * w.span_slots, replace=False)
        for k in range(w.n_spans):
            tags[r, slots[k * w.span_slots:(k + 1) * w.span_slots]] = k + 1
    steps = tuple(int(x) for x in rng.integers(0, 12, w.n_spans))
    return H2OInputs(w, K, V, torch.from_numpy(pos.astype(np.int32)).to(device),
                     torch.from_numpy(acc.astype(np.float32)).to(device), torch.from_numpy(tags).to(device),
                     q, K_new, V_new, steps)


# ---------------------------------------------------------------- CommitKV-style successive commits

@dataclass(frozen=True)
class CommitMultiWorkload:
    """Successive tool-call commits of agent trajectories. Before commit c the
    resident cache (B retained tokens, the previous observation and its
    window) grows by a new turn of n_call tokens whose last W tokens end the
    tool call (the pre-commit window). The turn's pages are the newly
    completed event pages: pending until their post-commit measurement. A
    checkpoint keeps B tokens; then the observation (n_obs tokens) and the
    post-commit window (W) are appended. In every turn n_plant pages have keys
    aligned with that turn's pre-commit queries and opposed to its post-commit
    ones (completion pages)."""
    name: str = "commitkv_multi"
    n_seq: int = 16
    n_layers: int = 28
    n_kv_heads: int = 4
    n_q_heads: int = 28
    head_dim: int = 128
    page_size: int = 16
    budget: int = 4096
    n_call: int = 1024
    n_obs: int = 512
    window: int = 32
    commits: int = 4
    n_plant: int = 8
    plant_logit: float = 9.0
    eta: float = 0.125
    max_protect: int = 16
    layer: int = 27
    tau_use: float = 0.05
    tau_dead: float = 1e-3
    rho_use: float = 0.75
    rho_dead: float = 0.25
    tau_joint: float = 1e-2
    max_scan: int = 64
    seed: int = 20261207

    @property
    def rows(self):
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def t_post(self):
        """Tokens after a checkpoint and its observation: B + n_obs + W."""
        return self.budget + self.n_obs + self.window

    @property
    def t_pre(self):
        """Tokens at a commit's pre-commit measurement: t_post + n_call."""
        return self.t_post + self.n_call


COMMIT_MULTI_WORKLOADS = {
    "commitkv_multi": CommitMultiWorkload(),
    "commitkv_multi_small": CommitMultiWorkload("commitkv_multi_small", n_seq=2, n_layers=3, n_kv_heads=2,
                                                n_q_heads=6, budget=256, n_call=128, n_obs=64, window=16,
                                                commits=3, n_plant=3, layer=2, max_scan=8, seed=20261217),
}


@dataclass
class CommitMultiInputs:
    w: CommitMultiWorkload
    K0: torch.Tensor       # bf16 [N][L][Hkv][t_post][d] history before the first turn
    V0: torch.Tensor
    K_call: torch.Tensor   # bf16 [C][N][L][Hkv][n_call][d] each turn's tokens
    V_call: torch.Tensor
    K_obs: torch.Tensor    # bf16 [C][N][L][Hkv][n_obs + W][d] each observation and its window
    V_obs: torch.Tensor
    Q_pre: torch.Tensor    # bf16 [C][N][L][Hq][W][d] the last W tokens of each turn
    Q_post: torch.Tensor   # bf16 [C][N][L][Hq][W][d] the last W tokens after each observation
    planted: np.ndarray    # int64 [C][N][n_plant] page indices within each turn


def make_commit_multi_inputs(w: CommitMultiWorkload, device="cpu") -> CommitMultiInputs:
    N, L, Hkv, Hq, d, C, W = w.n_seq, w.n_layers, w.n_kv_heads, w.n_q_heads, w.head_dim, w.commits, w.window
    G = Hq // Hkv
    s = w.seed * 16
    K0 = normal_bf16((N, L, Hkv, w.t_post, d), s + 1, device)
    V0 = normal_bf16((N, L, Hkv, w.t_post, d), s + 2, device)
    Kc = normal_bf16((C, N, L, Hkv, w.n_call, d), s + 3, device)
    Vc = normal_bf16((C, N, L, Hkv, w.n_call, d), s + 4, device)
    Ko = normal_bf16((C, N, L, Hkv, w.n_obs + W, d), s + 5, device)
    Vo = normal_bf16((C, N, L, Hkv, w.n_obs + W, d), s + 6, device)
    Qm = normal_bf16((C, N, L, Hq, W, d), s + 7, device)
    Qp = normal_bf16((C, N, L, Hq, W, d), s + 8, device)
    rng = np.random.default_rng(w.seed + 41)
    ps = w.page_size
    n_turn_pages = (w.n_call - W) // ps          # turn pages wholly before the pre-commit window
    planted = np.stack([np.stack([np.sort(rng.choice(n_turn_pages, w.n_plant, replace=False)) for _ in range(N)])
                        for _ in range(C)])
    c_len = float(np.sqrt(w.plant_logit * np.sqrt(d)))
    for c in range(C):
        u = rng.standard_normal((N, L, Hkv, d))
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        cu = torch.from_numpy(c_len * u).to(device=device, dtype=torch.float32)
        for n in range(N):
            Kn = Kc[c, n].view(L, Hkv, w.n_call // ps, ps, d)
            idx = torch.from_numpy(planted[c, n]).to(device)
            sel = Kn.index_select(2, idx).float() + cu[n][:, :, None, None, :]
            Kn.index_copy_(2, idx, sel.to(torch.bfloat16))
        cq = cu.repeat_interleave(G, dim=2)[:, :, :, None, :]
        Qm[c] = (Qm[c].float() + cq).to(torch.bfloat16)
        Qp[c] = (Qp[c].float() - cq).to(torch.bfloat16)
    return CommitMultiInputs(w, K0, V0, Kc, Vc, Ko, Vo, Qm, Qp, planted)
