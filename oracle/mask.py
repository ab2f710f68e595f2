"""Selection-mask oracle (integer, compared bit-exactly). Test infrastructure
only: imported by tests/, smoke() and bench.py's cpu_baseline leg.

"DeepSeek-V3.2-Exp · Sparse attention" page, "Code" section and the input
shapes (M^sel [B, T queries, T keys]): the indexer's top-k picks are 0 in an
otherwise -inf [B, T, T] mask, the causal mask is added, and the result is
shared by every head. Packed here as bits: bit (t % 32) of word t // 32 in row
(b, s) is 1 exactly when key t is live for query s (picked, and t <= s).
"""
import numpy as np


def topk_bitmask(topk_idx, T):
    """topk_idx: [B, Tq, k] int (-1 = padding), query s = row index.
    Returns uint32 [B, Tq, ceil(T/32)]."""
    t = np.asarray(topk_idx).astype(np.int64)
    B, Tq, k = t.shape
    W = -(-T // 32)
    out = np.zeros((B, Tq, W), dtype=np.uint32)
    b_i = np.broadcast_to(np.arange(B)[:, None, None], t.shape)
    s_i = np.broadcast_to(np.arange(Tq)[None, :, None], t.shape)
    live = (t >= 0) & (t <= s_i) & (t < T)
    tt = t[live]
    np.bitwise_or.at(out, (b_i[live], s_i[live], tt // 32),
                     (np.uint32(1) << (tt % 32).astype(np.uint32)))
    return out
