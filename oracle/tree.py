"""Tree verification in fp64 -- TEST INFRASTRUCTURE ONLY.

What is computed.  "Unlocking Lossless Speedups in LLMs via Discrete
Diffusion -- explained simply" (aifromscratch.in), section "The Ψ-Spec
Sampler": besides the linear sampler (one candidate per position) the pages
name a tree sampler that takes several candidates per position (the top K)
and verifies them in a prefix tree, best at low batch sizes; like the linear
one it preserves the AR model's output distribution exactly.

The pages give no acceptance rule for the tree.  Reading taken: the
candidates are fixed (chosen, not sampled), so speculative rejection over a
node's children -- accept child c with the residual probability of its token
and, on rejection, remove that token from the residual -- is, in law, one
draw y ~ p_v from the node's AR distribution followed by a look-up of y
among the children.  The single-draw form is used:

1. start at the root (node 0, the committed context);
2. at node v, draw y from p_v = softmax(z_v / T) by inverse CDF with the
   uniform of v's depth (``inverse_cdf`` of ``oracle.verify``);
3. if a child of v carries token y, move to it (the lowest-numbered such
   child if several do) and repeat; otherwise stop: y is the last token.

Every emitted token is a draw from the AR distribution given its prefix, so
the emitted sequence has the AR law whatever the tree.  A leaf's draw is the
bonus token.  Trees arrive as parent indices (node 0 the root with parent
-1, every other node's parent numbered below it) and one token per node.
"""

import numpy as np

from .verify import inverse_cdf, log_softmax


def tree_depths(parents):
    """Depth of every node (root 0) of one tree; raises on a malformed tree."""
    par = np.asarray(parents, dtype=np.int64)
    N = par.shape[0]
    if N < 1 or par[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    d = np.zeros(N, dtype=np.int64)
    for n in range(1, N):
        if not 0 <= par[n] < n:
            raise ValueError("every parent must be numbered below its child")
        d[n] = d[par[n]] + 1
    return d


def tree_verify(node_logits, parents, tokens, uniforms, temperature=1.0):
    """Verify B candidate trees of N nodes each.

    node_logits : [B, N, V]  AR logits after each node's prefix
    parents     : [B, N] int (parents[s, 0] = -1)
    tokens      : [B, N] int token of each node (the root's is unused)
    uniforms    : [B, N]     the draw at depth d uses uniforms[s, d]
    Returns a dict: n_accepted [B] (tree tokens kept; -1 for a malformed tree
    or a token outside [0, V)), out_tokens [B, N] (kept tokens, then the
    drawn token, -1 padded), n_emitted [B], last_node [B] (-1 if malformed).
    """
    z = np.asarray(node_logits)
    par = np.asarray(parents, dtype=np.int64)
    tok = np.asarray(tokens, dtype=np.int64)
    u = np.asarray(uniforms, dtype=np.float64)
    B, N, V = z.shape
    n_acc = np.full(B, -1, dtype=np.int32)
    out = np.full((B, N), -1, dtype=np.int32)
    n_emit = np.zeros(B, dtype=np.int32)
    last = np.full(B, -1, dtype=np.int32)
    for s in range(B):
        try:
            tree_depths(par[s])
        except ValueError:
            continue
        if np.any((tok[s, 1:] < 0) | (tok[s, 1:] >= V)):
            continue
        v, depth = 0, 0
        while True:
            p = np.exp(log_softmax(z[s, v], temperature))
            y = int(inverse_cdf(p, u[s, depth]))
            out[s, depth] = y
            kids = [c for c in range(v + 1, N) if par[s, c] == v and tok[s, c] == y]
            if not kids:
                break
            v, depth = kids[0], depth + 1
        n_acc[s], n_emit[s], last[s] = depth, depth + 1, v
    return {"n_accepted": n_acc, "out_tokens": out, "n_emitted": n_emit, "last_node": last}
