"""Top-k page selection over block scores: plain CPU definition.

TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and the
benchmark's CPU-baseline leg; the product path never imports it.

The selection step that follows the scorer (ATOM #2770, "How it works": the
selection and the emit after the scores are unchanged; the squashed
sparse-attention commit: the tail page is always selected) is only named on
the pages; k, the tie rule and the order of the result are not. Reading taken:
for every (row, head),
  * the live pages are those with a finite block score (a page holding no
    token the row sees scores -inf);
  * the tail page, the page holding the row's last visible token
    (limit - 1), is always selected when the row sees any token;
  * the other k - 1 places go to the live pages with the largest scores,
    ties to the lower page index;
  * the result lists the selected pages in ascending order, then -1 for the
    places left when fewer than k pages are live.
Row limits follow the scorer's masking: prefill row i of a request sees
min(seq_len, prefix_len + i + 1) tokens, a decode row seq_len.
"""
from __future__ import annotations

import numpy as np


def row_limits(mode: str, seq_lens, max_seq_len: int, cu_seqlens_q=None, prefix_lens=None) -> np.ndarray:
    """Visible tokens per query row, clipped to the output window."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    if mode == "decode":
        return np.clip(seq, 0, max_seq_len)
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    pre = np.asarray(prefix_lens, dtype=np.int64)
    out = []
    for b in range(len(seq)):
        for i in range(int(cu[b + 1] - cu[b])):
            out.append(min(int(seq[b]), int(pre[b]) + i + 1))
    return np.clip(np.asarray(out, dtype=np.int64), 0, max_seq_len)


def select_pages(block_scores: np.ndarray, limits: np.ndarray, page_size: int, k: int) -> np.ndarray:
    """block_scores [R, H, NB] float32, limits [R] -> int32 [R, H, k]."""
    bs = np.asarray(block_scores, dtype=np.float32)
    R, H, NB = bs.shape
    out = np.full((R, H, k), -1, dtype=np.int32)
    for r in range(R):
        lim = int(limits[r])
        tail = (lim - 1) // page_size if lim > 0 else -1
        for h in range(H):
            s = bs[r, h]
            live = np.nonzero(np.isfinite(s))[0]
            if k == 0 or len(live) == 0:
                continue
            others = [j for j in live if j != tail]
            # largest score first, ties to the lower page index
            others.sort(key=lambda j: (-float(s[j]), int(j)))
            chosen = ([tail] if tail in set(live.tolist()) else []) + others
            chosen = sorted(int(j) for j in chosen[:k])
            out[r, h, :len(chosen)] = chosen
    return out
