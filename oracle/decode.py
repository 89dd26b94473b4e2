"""Decode attention over a compacted cache (test infrastructure).

PASK §3.1, Eq. 1: o = V softmax(K^T q / sqrt(d_k)). PASK Appendix B.5 runs it
over disjoint partitions of the cache (BF16 rows, low-precision rows
dequantised as code*scale, the current KV) with FP32 statistics and BF16
output, merging per-partition (max, exp-sum, unnormalised value sum) by
Eq. 15. Eq. 15 is an implementation freedom: mathematically it equals one
softmax over the union, which is what this oracle computes, in float64.
Query head h reads KV head floor(h / G), G = Hq / Hkv (grouped-query
attention, PASK Appendix B.5). Every cached key is visible to the decoded
query.
"""
import numpy as np

from . import numfmt


def decode_head(q, K, V):
    """q: [d]; K, V: [n, d] float64 (n >= 1). Returns (o [d] float64, lse float64)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = K @ q / np.sqrt(q.shape[0])
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ V) / l, m + np.log(l)


def decode_partitions(q, parts):
    """One softmax over the union of partitions; parts = [(K, V), ...] with
    possibly empty partitions (n = 0), which contribute nothing."""
    Ks = [np.asarray(k, np.float64) for k, _ in parts if len(k)]
    Vs = [np.asarray(v, np.float64) for k, v in parts if len(k)]
    return decode_head(q, np.concatenate(Ks), np.concatenate(Vs))


def merge_partitions(stats):
    """PASK Eq. 15: stats = [(v_j max, l_j exp-sum, u_j unnormalised sum)] of
    non-empty partitions -> o. Used only to pin the union formulation."""
    v = max(s[0] for s in stats)
    num = sum(np.exp(vj - v) * np.asarray(uj) for vj, _, uj in stats)
    den = sum(np.exp(vj - v) * lj for vj, lj, _ in stats)
    return num / den


def decode_bf16(q, parts):
    """As decode_partitions, with the output rounded once to bf16 (bits)."""
    o, lse = decode_partitions(q, parts)
    return numfmt.f64_to_bf16_bits(o), lse
