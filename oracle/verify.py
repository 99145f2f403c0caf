"""Lossless block verification in fp64 -- TEST INFRASTRUCTURE ONLY.

What is computed.  "Unlocking Lossless Speedups in LLMs via Discrete
Diffusion -- explained simply" (aifromscratch.in), section "The Ψ-Spec
Sampler": the diffusion pathway proposes a block of tokens in parallel; the
sampler rejection-samples that block against the AR model in the manner of
speculative decoding and keeps the longest valid prefix; the linear variant
proposes one candidate per position; the AR output distribution is preserved
exactly.  "Uno Uses Discrete Diffusion to Accelerate LLMs Without Loss"
(cctest.ai), section "What 'lossless' means here": the AR model is the
authority and verification either rejects a candidate or adjusts it.

The pages print no formula, so the standard speculative rejection sampler is
taken as the reading of "speculative-decoding-style rejection sampling":

1. p_i = softmax(z_i / T) is the AR (target) distribution at position i and
   q_i = softmax(d_i / T) the draft distribution the token x_i was drawn from.
2. Position i is accepted when u_i < min(1, p_i(x_i) / q_i(x_i)), with u_i
   uniform on [0, 1).  The ratio is formed in log space,
   a_i = exp(min(0, log p_i(x_i) - log q_i(x_i))); log p = -inf gives a = 0,
   and log q = -inf with log p finite gives a = 1.
3. n_acc is the index of the first rejected position (L if none): the
   longest accepted prefix.
4. If n_acc < L the token at position j = n_acc is redrawn from the residual
   normalize(max(0, p_j - q_j)); if that residual has zero total mass it is
   redrawn from p_j (a zero-probability event in exact arithmetic).
   If every position is accepted and a bonus target row L is supplied, one
   extra token is drawn from p_L.
5. Tokens are drawn by inverse CDF: with C the running sum of the weights and
   R its last value, the token is the smallest k with C_k > u * R (zero-mass
   tokens are never chosen); u is the per-sequence slot L of the uniforms.
6. Emitted tokens are x_0 .. x_{n_acc-1} followed by the redrawn or bonus
   token, padded with -1; n_emitted = n_acc + 1 when a token was redrawn or
   added, else L.

Arrays may carry a leading sequence dimension of 1, which then broadcasts
over all sequences (the same logits for every trial).  Vectorising over
independent sequences changes no arithmetic.
"""

import numpy as np


def log_softmax(logits, temperature=1.0):
    """log softmax(logits / T) over the last axis, in fp64.

    Uses log-sum-exp with the row maximum factored out; the value is the
    plain definition log p_k = z_k/T - log sum_j exp(z_j/T).
    """
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    v = np.asarray(logits, dtype=np.float64) / float(temperature)
    m = np.max(v, axis=-1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("every row needs at least one finite logit")
    lse = m + np.log(np.sum(np.exp(v - m), axis=-1, keepdims=True))
    return v - lse


def acceptance_probability(logp_x, logq_x):
    """a = min(1, p(x)/q(x)) evaluated as exp(min(0, log p(x) - log q(x)))."""
    lp = np.asarray(logp_x, dtype=np.float64)
    lq = np.asarray(logq_x, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        a = np.exp(np.minimum(0.0, lp - lq))
    a = np.where(np.isneginf(lq), 1.0, a)      # q(x) = 0, p(x) > 0: ratio is +inf
    a = np.where(np.isneginf(lp), 0.0, a)      # p(x) = 0: never accept
    return a


def inverse_cdf(weights, u):
    """Smallest k with C_k > u * R, where C = cumsum(weights), R = C[-1].

    weights: [..., V] non-negative, u: [...] in [0, 1).  Returns int64 [...].
    If rounding leaves no qualifying k, the last positive-weight token is
    returned.
    """
    w = np.asarray(weights, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    c = np.cumsum(w, axis=-1)
    t = u * c[..., -1]
    hit = c > t[..., None]
    k = np.argmax(hit, axis=-1)
    none = ~np.any(hit, axis=-1)
    if np.any(none):
        pos = w > 0
        last = w.shape[-1] - 1 - np.argmax(pos[..., ::-1], axis=-1)
        k = np.where(none, last, k)
    return k.astype(np.int64)


def residual_weights(logp_row, logq_row, with_fallback=False):
    """max(0, p - q) over the vocabulary, or p itself if that has zero mass.

    The redraw law after a rejection (step 4 above).  logp_row, logq_row:
    [..., V] log-probabilities.  With with_fallback, also returns a bool
    array [...] that is True where the residual had zero mass and p was
    taken instead.
    """
    p = np.exp(np.asarray(logp_row, dtype=np.float64))
    q = np.exp(np.asarray(logq_row, dtype=np.float64))
    r = np.maximum(0.0, p - q)
    zero = np.sum(r, axis=-1, keepdims=True) == 0.0
    w = np.where(zero, p, r)
    return (w, zero[..., 0]) if with_fallback else w


def _broadcast_lead(arr, B):
    arr = np.asarray(arr)
    if arr.shape[0] not in (1, B):
        raise ValueError("leading dimension must be 1 or the number of sequences")
    return arr


def block_verify(target_logits, draft_logits, draft_tokens, uniforms,
                 temperature=1.0, has_bonus=False):
    """Verify one drafted block per sequence.

    target_logits : [B or 1, L + has_bonus, V]  AR logits z
    draft_logits  : [B or 1, L, V]              draft logits d
    draft_tokens  : [B, L] int                  drafted tokens x
    uniforms      : [B, L + 1]                  slots 0..L-1 accept, slot L redraw
    Returns a dict of NumPy arrays:
      n_accepted [B] int32 (-1 if a draft token is outside [0, V)),
      out_tokens [B, L+1] int32 (-1 padded), n_emitted [B] int32,
      accept_prob [B, L] float64, redraw_row [B] int32 (-1 if none),
      redraw_mode [B] int8 (0 none, 1 residual, 2 from p).
    """
    x = np.asarray(draft_tokens, dtype=np.int64)
    B, L = x.shape
    u = np.asarray(uniforms, dtype=np.float64)
    if u.shape != (B, L + 1):
        raise ValueError("uniforms must be [B, L+1]")
    z = _broadcast_lead(target_logits, B)
    d = _broadcast_lead(draft_logits, B)
    V = z.shape[-1]
    nb = 1 if has_bonus else 0
    if z.shape[1] < L + nb or d.shape[1] < L or d.shape[-1] != V:
        raise ValueError("logit shapes do not match the block")

    lp = log_softmax(z[:, :L + nb, :], temperature)      # log p_i
    lq = log_softmax(d[:, :L, :], temperature)           # log q_i

    valid = np.all((x >= 0) & (x < V), axis=1)
    xs = np.where((x >= 0) & (x < V), x, 0)
    bz = np.arange(B) if lp.shape[0] == B else np.zeros(B, dtype=np.int64)
    bd = np.arange(B) if lq.shape[0] == B else np.zeros(B, dtype=np.int64)
    ii = np.arange(L)
    lp_x = lp[bz[:, None], ii[None, :], xs]
    lq_x = lq[bd[:, None], ii[None, :], xs]
    a = acceptance_probability(lp_x, lq_x)               # [B, L]
    accept = u[:, :L] < a
    rejected = ~accept
    n_acc = np.where(np.any(rejected, axis=1), np.argmax(rejected, axis=1), L)

    out = np.full((B, L + 1), -1, dtype=np.int64)
    n_emit = np.where(n_acc < L, n_acc + 1, L + nb).astype(np.int64)
    mode = np.zeros(B, dtype=np.int8)
    row = np.full(B, -1, dtype=np.int64)

    for i in range(L):
        keep = n_acc > i
        out[keep, i] = x[keep, i]

    rej = np.nonzero((n_acc < L) & valid)[0]
    if rej.size:
        j = n_acc[rej]
        r, zero = residual_weights(lp[bz[rej], j, :], lq[bd[rej], j, :], with_fallback=True)
        out[rej, j] = inverse_cdf(r, u[rej, L])
        mode[rej] = np.where(zero, 2, 1)
        row[rej] = j
    if has_bonus:
        bon = np.nonzero((n_acc == L) & valid)[0]
        if bon.size:
            out[bon, L] = inverse_cdf(np.exp(lp[bz[bon], L, :]), u[bon, L])
            mode[bon] = 2
            row[bon] = L

    n_acc = np.where(valid, n_acc, -1)
    n_emit = np.where(valid, n_emit, 0)
    out[~valid] = -1
    mode[~valid] = 0
    row[~valid] = -1
    return {
        "n_accepted": n_acc.astype(np.int32),
        "out_tokens": out.astype(np.int32),
        "n_emitted": n_emit.astype(np.int32),
        "accept_prob": a,
        "redraw_row": row.astype(np.int32),
        "redraw_mode": mode,
    }


def draft_sample(draft_logits, uniforms, temperature=1.0):
    """Draw one draft token per row from q = softmax(d / T) by inverse CDF.

    "The Ψ-Spec Sampler" (aifromscratch.in page): the diffusion pathway
    proposes the block's tokens in parallel, one candidate per position for
    the linear sampler.  draft_logits: [..., V]; uniforms: [...].
    """
    q = np.exp(log_softmax(draft_logits, temperature))
    return inverse_cdf(q, uniforms).astype(np.int32)
