"""Workload definitions and host-side (NumPy) input generators.

Five workloads, named by what they are:

* ``tiny``        one 512->512 projection (r=128, fp32) over 2 sequences of
                  [8 verify | 4 draft] rows; verify over V=64, block 4, fp32
                  logits z ~ N(0,1), draft d = z + N(0, 0.5^2), T = 1.
* ``layer_b1``    the 7 projections of an 8B-shaped layer (bf16) over one
                  sequence of [16 verify | 16 draft] rows; verify one block
                  of 16 over V=128256, z ~ N(0, 3^2), d = z + N(0, 1).
* ``layer_b64``   the same layer over 64 sequences x [16 | 16] rows; verify
                  64 blocks of 16, draft noise sigma in {0.25, 1, 4}.
* ``serve_b256``  the up (4096->14336) and down (14336->4096) projections
                  over 256 sequences x [32 | 32] rows; verify 256 blocks of
                  32, Zipf-skewed logits, T in {0.6, 1.0}.
* ``stack32_b32`` 32 layers x 7 projections over 32 sequences x [16 | 16]
                  rows; verify 32 blocks of 16, sigma = 1.

Weights follow the tiny workload's recipe at every size: W_AR and A have
N(0, 1/d_in) entries, B has N(0, 1/r) entries, x is N(0, 1); bf16 workloads
round every array to bf16 (round to nearest even) after sampling.
"""

from dataclasses import dataclass, field

import numpy as np

HIDDEN = 4096
KV_DIM = 1024
FFN = 14336
VOCAB = 128256
RANK = 128
ALPHA = 256

# (name, d_in, d_out) for the seven projections of one 8B-shaped layer.
LAYER_PROJECTIONS = (
    ("q", HIDDEN, HIDDEN),
    ("k", HIDDEN, KV_DIM),
    ("v", HIDDEN, KV_DIM),
    ("o", HIDDEN, HIDDEN),
    ("gate", HIDDEN, FFN),
    ("up", HIDDEN, FFN),
    ("down", FFN, HIDDEN),
)


def layer_shapes():
    """The seven (name, K, N) projection shapes of one layer."""
    return LAYER_PROJECTIONS


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_seq: int                 # sequences in the mixed batch
    verify_rows: int           # g = 0 rows per sequence
    draft_rows: int            # g = 1 rows per sequence
    projections: tuple         # ((name, K, N), ...) per layer
    layers: int
    gemm_dtype: str            # "f32" or "bf16"
    vocab: int
    block: int                 # L, drafted positions per sequence
    logits: str                # "normal" or "zipf"
    target_sigma: float        # std of target logits ("normal")
    draft_sigmas: tuple        # std of draft noise around the target
    temperatures: tuple
    logits_dtype: str          # "f32" or "bf16"
    extra: dict = field(default_factory=dict)

    @property
    def rows(self):
        return self.n_seq * (self.verify_rows + self.draft_rows)


WORKLOADS = {
    "tiny": Workload("tiny", 1001, 2, 8, 4, (("proj", 512, 512),), 1, "f32",
                     64, 4, "normal", 1.0, (0.5,), (1.0,), "f32",
                     {"trials": 1_000_000}),
    "layer_b1": Workload("layer_b1", 1002, 1, 16, 16, LAYER_PROJECTIONS, 1, "bf16",
                         VOCAB, 16, "normal", 3.0, (1.0,), (1.0,), "bf16"),
    "layer_b64": Workload("layer_b64", 1003, 64, 16, 16, LAYER_PROJECTIONS, 1, "bf16",
                          VOCAB, 16, "normal", 3.0, (0.25, 1.0, 4.0), (1.0,), "bf16"),
    "serve_b256": Workload("serve_b256", 1004, 256, 32, 32,
                           (("up", HIDDEN, FFN), ("down", FFN, HIDDEN)), 1, "bf16",
                           VOCAB, 32, "zipf", 0.0, (0.5,), (0.6, 1.0), "bf16",
                           {"zipf_slope": 1.1}),
    "stack32_b32": Workload("stack32_b32", 1005, 32, 16, 16, LAYER_PROJECTIONS, 32, "bf16",
                            VOCAB, 16, "normal", 3.0, (1.0,), (1.0,), "bf16"),
}


def bf16_round(a):
    """Round float32 values to the nearest bf16 value (ties to even); float32 out."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    finite = np.isfinite(a)
    r = np.where(finite, r, a.view(np.uint32) & np.uint32(0xFFFF0000))
    return r.view(np.float32).reshape(a.shape)


def bf16_bits(a):
    """The bf16 bit patterns (uint16) of float32 values already on the bf16 grid."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def gate_vector(n_seq, verify_rows, draft_rows):
    """Row gates for n_seq sequences laid out as [verify rows | draft rows] each."""
    one = np.concatenate([np.zeros(verify_rows, np.uint8), np.ones(draft_rows, np.uint8)])
    return np.tile(one, n_seq)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def gemm_inputs(M, K, N, r, seed, dtype="bf16", gate=None):
    """x [M,K], w [N,K], a [r,K], b [N,r] (float32 holding the stored values) and gate.

    x ~ N(0,1); w, a ~ N(0, 1/K); b ~ N(0, 1/r).  bf16 rounds each array.
    """
    g = _rng(seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    a = g.standard_normal((r, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
    b = g.standard_normal((N, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    if dtype == "bf16":
        x, w, a, b = (bf16_round(t) for t in (x, w, a, b))
    elif dtype != "f32":
        raise ValueError(dtype)
    if gate is None:
        gate = (g.random(M) < 0.5).astype(np.uint8)
    return {"x": x, "w": w, "a": a, "b": b, "gate": np.asarray(gate, np.uint8)}


def verify_inputs(B, L, V, seed, kind="normal", target_sigma=3.0, draft_sigma=1.0,
                  has_bonus=False, dtype="bf16", zipf_slope=1.1):
    """Target logits [B, L+has_bonus, V] and draft logits [B, L, V] (float32 values).

    normal: z ~ N(0, target_sigma^2), d = z + N(0, draft_sigma^2) on the first L rows.
    zipf:   per-row random ranks 1..V shared by both sides;
            z = -slope*log(rank) + N(0, draft_sigma^2), d likewise with its own noise.
    """
    g = _rng(seed)
    rows_t = L + (1 if has_bonus else 0)
    if kind == "normal":
        z = g.standard_normal((B, rows_t, V), dtype=np.float32) * np.float32(target_sigma)
        d = z[:, :L, :] + g.standard_normal((B, L, V), dtype=np.float32) * np.float32(draft_sigma)
    elif kind == "zipf":
        ranks = np.argsort(g.random((B, rows_t, V), dtype=np.float32), axis=-1).astype(np.float32) + 1.0
        base = np.float32(-zipf_slope) * np.log(ranks)
        z = base + g.standard_normal((B, rows_t, V), dtype=np.float32) * np.float32(draft_sigma)
        d = base[:, :L, :] + g.standard_normal((B, L, V), dtype=np.float32) * np.float32(draft_sigma)
    else:
        raise ValueError(kind)
    if dtype == "bf16":
        z, d = bf16_round(z), bf16_round(d)
    elif dtype != "f32":
        raise ValueError(dtype)
    return np.ascontiguousarray(z, np.float32), np.ascontiguousarray(d, np.float32)


def _exact_scale(K):
    """2^-e with 2^e the power of two nearest sqrt(K)."""
    return float(2.0 ** -round(0.5 * np.log2(max(K, 1))))


def lm_head_inputs(B, L, V, K, seed, has_bonus=False, kind="normal", logit_sigma=3.0, draft_noise=0.3):
    """Inputs of the LM head + verification: stacked hidden rows
    [B (L + has_bonus) + B L, K] (target rows, then draft rows), the head
    w [V, K], draft tokens [B, L] int32 and uniforms [B, L + 1] float32.

    normal: target hidden ~ N(0, 1); each draft row is the target row of the
            same position plus N(0, draft_noise^2); w ~ N(0, logit_sigma^2 / K),
            so logits have a spread of about logit_sigma.  bf16 rounds hidden and w.
    exact:  small integers, so that every fp32 sum of products is exact
            whatever the order: target hidden in [-3, 3], draft = target plus
            [-1, 1], w in [-2, 2] times 2^-e with 2^e near sqrt(K).
    Tokens are uniform over [0, V); uniforms uniform on [0, 1).
    """
    g = _rng(seed)
    nb = 1 if has_bonus else 0
    if kind == "normal":
        ht = g.standard_normal((B, L + nb, K), dtype=np.float32)
        hd = ht[:, :L] + g.standard_normal((B, L, K), dtype=np.float32) * np.float32(draft_noise)
        w = g.standard_normal((V, K), dtype=np.float32) * np.float32(logit_sigma / np.sqrt(K))
        ht, hd, w = bf16_round(ht), bf16_round(hd), bf16_round(w)
    elif kind == "exact":
        ht = g.integers(-3, 4, (B, L + nb, K)).astype(np.float32)
        hd = ht[:, :L] + g.integers(-1, 2, (B, L, K)).astype(np.float32)
        w = g.integers(-2, 3, (V, K)).astype(np.float32) * np.float32(_exact_scale(K))
    else:
        raise ValueError(kind)
    hidden = np.concatenate([ht.reshape(B * (L + nb), K), hd.reshape(B * L, K)])
    tokens = g.integers(0, V, (B, L)).astype(np.int32)
    uniforms = g.random((B, L + 1), dtype=np.float32)
    return {"hidden": np.ascontiguousarray(hidden), "w": np.ascontiguousarray(w), "tokens": tokens,
            "uniforms": uniforms}
