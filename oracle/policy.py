"""Bonus, floor and protection rules applied before selection (test infrastructure).

* Layer groups -- PASK Appendix A.2 splits L layers into lower/middle/upper
  groups at b1 = floor((L+2)/3) = ceil(L/3) and b2 = floor((2L+2)/3) =
  ceil(2L/3). For n groups the same rule reads: boundary c sits at
  ceil(c*L/n), and layer l belongs to group #{c >= 1 : l >= ceil(c*L/n)}.
* Foresight bonus -- PACE §3.1, Eq. 2: a token in a span whose next planned
  reader is s* steps away gets beta = sigma * (1/2 + 1/2 * exp(-lambda*(s*-t))),
  tokens without a future reference get 0. Its floor is sigma/2 and the
  soonest-needed span ranks highest. The printed equation is garbled on the
  page; this reading is the one the surrounding text (floor sigma/2,
  soonest-first) fixes.
* Protection -- sink and recent-window masks (PASK Appendix A.3/B.2; PACE
  Table 1 counts 4 sinks and 128 recent tokens inside the budget) and
  per-(tag, group) floors from the frozen table (PASK §3.5, Eq. 11) force a
  token to be kept whatever its score.
"""
import math

import numpy as np


def layer_group(layer, n_layers, n_groups):
    """Group index of ``layer`` (0-based) among ``n_groups`` groups."""
    return sum(1 for c in range(1, n_groups)
               if layer >= math.ceil(c * n_layers / n_groups))


def group_ranges(n_layers, n_groups):
    """[(first, last_inclusive)] per group, for reading against PASK A.2."""
    out = []
    for g in range(n_groups):
        ls = [l for l in range(n_layers) if layer_group(l, n_layers, n_groups) == g]
        out.append((ls[0], ls[-1]))
    return out


def foresight_bonus(sigma, lam, steps_ahead):
    """PACE Eq. 2 for a span whose next reader is ``steps_ahead`` = s* - t >= 0
    steps away; ``None`` (no future reader) gives 0."""
    if steps_ahead is None:
        return 0.0
    return sigma * (0.5 + 0.5 * math.exp(-lam * float(steps_ahead)))


def totals_and_protection(score, tags, bonus_tbl, floor_tbl, group, n_sink, n_recent):
    """total[j] = score[j] + bonus[tag_j][group];
    protected[j] = j < n_sink  or  j >= T - n_recent  or  floor[tag_j][group].

    score: [T] float64; tags: [T] ints or None (all tag 0);
    bonus_tbl: [n_tags][n_groups] floats; floor_tbl: [n_tags][n_groups] 0/1.
    """
    score = np.asarray(score, np.float64)
    T = score.shape[0]
    if tags is None:
        tags = np.zeros(T, dtype=np.int64)
    tags = np.asarray(tags, dtype=np.int64)
    bonus = np.asarray(bonus_tbl, np.float64)[tags, group]
    floor = np.asarray(floor_tbl)[tags, group] != 0
    j = np.arange(T)
    protected = (j < n_sink) | (j >= T - n_recent) | floor
    return score + bonus, protected
