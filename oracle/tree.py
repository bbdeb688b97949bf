"""Plain CPU oracle of greedy (T = 0) tree verification.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may call this; the product library never does.  It shares
no code with the HIP library.

Method: a speculative-decoding survey (zhifeiding.github.io), sec. 2.3
(chains and trees: a tree draft expands several branches per node and the
target checks the whole tree in one pass), and the DART reading note
(zhongzhuzhou.org), sec. 2.3: at temperature zero the verifier checks the
target's argmax along a candidate path; the pages give no rule for T > 0,
so only T = 0 is implemented.

Readings where the pages leave a step open (listed in the design notes):
  * a tree of n nodes is given in topological order: node 0 is the root (the
    last committed token), every other node v has a parent p(v) < v and a
    draft token x_v; target row v holds the target's next-token logits after
    the path root .. v;
  * node v is accepted when its parent is accepted (the root always is) and
    x_v equals the target argmax of row p(v) (lowest id on ties); the walk
    goes from the root to the accepted child, the lowest-index one if two
    siblings carry the same token, and stops at a node with no accepted
    child;
  * the committed tokens are the accepted path's draft tokens followed by
    the argmax of the last accepted node's row (the bonus or correction
    token); a row the walk reads holding a NaN or +-inf logit, a parent
    outside [0, v), a draft token outside [0, V) or n outside [1, M] makes the
    request invalid (rows the walk never reads are not inspected).
"""
from __future__ import annotations

import numpy as np


def _row_argmax(row: np.ndarray) -> int:
    """Lowest index of the maximum; -1 if the row holds NaN or +-inf."""
    r = np.asarray(row, dtype=np.float64)
    if not np.all(np.isfinite(r)):
        return -1
    return int(np.argmax(r))


def tree_verify(logits, parent, tokens, n_nodes) -> dict:
    """logits [R][M][V] (fp32, or bf16 bit patterns as uint16), parent and
    tokens [R][M] int32, n_nodes [R].  Returns accepted [R] (accepted draft
    nodes, -1 for an invalid request), path [R][M] (accepted node indices,
    -1 padded) and committed [R][M] (path tokens then the bonus, -1 padded)."""
    L = np.asarray(logits)
    if L.dtype == np.uint16:
        L = (L.astype(np.uint32) << 16).view(np.float32)
    R, M, V = L.shape
    P = np.asarray(parent)
    X = np.asarray(tokens)
    n_nodes = np.asarray(n_nodes)
    accepted = np.full(R, -1, np.int32)
    path = np.full((R, M), -1, np.int32)
    committed = np.full((R, M), -1, np.int32)
    for r in range(R):
        n = int(n_nodes[r])
        ok = 1 <= n <= M
        for v in range(1, n if ok else 0):
            ok = ok and 0 <= P[r, v] < v and 0 <= X[r, v] < V
        if not ok:
            continue
        cur, seq, toks = 0, [], []
        while True:
            g = _row_argmax(L[r, cur])
            if g < 0:
                ok = False
                break
            nxt = -1
            for v in range(cur + 1, n):
                if P[r, v] == cur and X[r, v] == g:
                    nxt = v
                    break
            if nxt < 0:
                toks.append(g)
                break
            seq.append(nxt)
            toks.append(int(X[r, nxt]))
            cur = nxt
        if not ok:
            continue
        accepted[r] = len(seq)
        path[r, :len(seq)] = seq
        committed[r, :len(toks)] = toks
    return dict(accepted=accepted, path=path, committed=committed)
