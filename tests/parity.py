"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerance rules (written here once, used by every parity test):

* GEMM outputs: max over elements of |y - y_ref| / max(|y_ref|, rms of the
  reference row), the elementwise error floored by the row's RMS so that
  cancellation to near-zero entries does not make the metric meaningless.
  bf16 bound 2e-2 (fp32 accumulation, bf16 inputs and output, the adapter's
  intermediate rounded once to bf16); fp32 bound 1e-4.
* Sampler outputs (accepted lengths, emitted tokens, sampled tokens): exact,
  except where the oracle's decision lies within 1e-6 of the uniform that
  drove it -- an acceptance test with |u - a| <= 1e-6, or a draw whose
  uniform sits within 1e-6 of every normalised CDF boundary between the two
  tokens.  Such ties are excused, counted and reported; anything else fails.
"""

import numpy as np

import oracle

TIE = 1e-6
BF16_TOL = 2e-2
F32_TOL = 1e-4


def floored_rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - ref) / den)) if y.size else 0.0


def _boundaries_within(weights, u, tok_a, tok_b, tie=TIE):
    """True iff every normalised CDF boundary between the two tokens is within tie of u."""
    lo, hi = min(tok_a, tok_b), max(tok_a, tok_b)
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    c = c / c[-1]
    bounds = c[lo:hi]                      # C_lo .. C_{hi-1}
    return bool(np.all(np.abs(bounds - u) <= tie))


def compare_verify(gpu, ref, z, d, u, temperature, has_bonus):
    """Compare GPU (n_acc, out_tokens, n_emitted) with the oracle's result dict.

    z, d: the logits the oracle saw ([B or 1, rows, V]); u: [B, L+1] float64.
    Returns (n_exact, n_excused, failures) where failures is a list of strings.
    """
    g_acc, g_tok, g_emit = (np.asarray(t) for t in gpu)
    r_acc, r_tok, r_emit = ref["n_accepted"], ref["out_tokens"], ref["n_emitted"]
    B, L = ref["accept_prob"].shape
    exact, excused, fails = 0, 0, []
    for s in range(B):
        if g_acc[s] == r_acc[s] and np.array_equal(g_tok[s], r_tok[s]) and g_emit[s] == r_emit[s]:
            exact += 1
            continue
        if r_acc[s] < 0 or g_acc[s] < 0:
            fails.append(f"seq {s}: sentinel mismatch gpu {g_acc[s]} oracle {r_acc[s]}")
            continue
        if g_acc[s] != r_acc[s]:
            i = int(min(g_acc[s], r_acc[s]))
            a = float(ref["accept_prob"][s, i])
            if abs(float(u[s, i]) - a) <= TIE:
                excused += 1
            else:
                fails.append(f"seq {s}: n_acc gpu {g_acc[s]} oracle {r_acc[s]}; u={u[s, i]!r} a={a!r}")
            continue
        j = int(r_acc[s])
        if not np.array_equal(g_tok[s, :j], r_tok[s, :j]) or g_emit[s] != r_emit[s]:
            fails.append(f"seq {s}: prefix/emit mismatch")
            continue
        if g_tok[s, j] == r_tok[s, j] or not (np.all(g_tok[s, j + 1:] == -1) and np.all(r_tok[s, j + 1:] == -1)):
            fails.append(f"seq {s}: tokens differ outside the drawn slot: gpu {g_tok[s]} oracle {r_tok[s]}")
            continue
        # same accepted prefix, different drawn token
        bz = s if z.shape[0] > 1 else 0
        bd = s if d.shape[0] > 1 else 0
        lp = oracle.log_softmax(z[bz, j], temperature)
        if j < L:
            w = oracle.residual_weights(lp, oracle.log_softmax(d[bd, j], temperature))
        else:
            w = np.exp(lp)
        if _boundaries_within(w, float(u[s, L]), int(g_tok[s, j]), int(r_tok[s, j])):
            excused += 1
        else:
            fails.append(f"seq {s}: drawn token gpu {g_tok[s, j]} oracle {r_tok[s, j]} u={u[s, L]!r}")
    return exact, excused, fails


def compare_samples(gpu_tok, ref_tok, d, u, temperature):
    """Compare sampled draft tokens [rows] with the oracle's; d: [rows, V] logits."""
    exact, excused, fails = 0, 0, []
    for i in range(len(ref_tok)):
        if int(gpu_tok[i]) == int(ref_tok[i]):
            exact += 1
            continue
        w = np.exp(oracle.log_softmax(d[i], temperature))
        if _boundaries_within(w, float(u[i]), int(gpu_tok[i]), int(ref_tok[i])):
            excused += 1
        else:
            fails.append(f"row {i}: gpu {gpu_tok[i]} oracle {ref_tok[i]} u={u[i]!r}")
    return exact, excused, fails
