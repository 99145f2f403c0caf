"""Tree verification (the tree sampler) on the GPU vs the fp64 oracle.

Trees are built here from per-depth top-K candidate sets (breadth-first, so
every parent is numbered below its children): each node at depth d has the
K top tokens of a per-depth base logit vector as children, and each node's
AR logits are that depth's base plus noise, so that walks go several levels
deep.  Outputs must match the oracle exactly, except a draw whose uniform
lies within 1e-6 of every CDF boundary between the two tokens (tests/parity.py),
counted and excused.  Uniforms come from the oracle's Philox.
"""

import numpy as np
import pytest
import torch

import lossless_speculative_drafting_amd as uno
import oracle
from gpu_util import say, to_dev, to_host
from parity import _boundaries_within


def topk_tree(base, K, D):
    """Parents and tokens of the K-ary prefix tree of depth D over per-depth top-K sets."""
    parents, tokens, depth = [-1], [0], [0]
    frontier = [0]
    for d in range(D):
        top = np.argsort(-base[d], kind="stable")[:K]
        nxt = []
        for v in frontier:
            for t in top:
                parents.append(v)
                tokens.append(int(t))
                depth.append(d + 1)
                nxt.append(len(parents) - 1)
        frontier = nxt
    return np.array(parents), np.array(tokens), np.array(depth)


def tree_inputs(B, K, D, V, seed, noise=1.0, sigma=3.0):
    rng = np.random.default_rng(seed)
    par, tok, depth = topk_tree(np.zeros((D, V)), K, D)  # shape only; tokens per sequence below
    N = len(par)
    parents = np.tile(par, (B, 1))
    tokens = np.zeros((B, N), np.int64)
    z = np.zeros((B, N, V), np.float32)
    for s in range(B):
        base = rng.standard_normal((D + 1, V)) * sigma
        p_, t_, d_ = topk_tree(base, K, D)
        tokens[s] = t_
        z[s] = (base[d_] + rng.standard_normal((N, V)) * noise).astype(np.float32)
    return z, parents, tokens


def _compare(gpu, ref, z, parents, tokens, u, T):
    g_acc, g_tok, g_emit, g_last = gpu
    exact, excused, fails = 0, 0, []
    for s in range(len(g_acc)):
        same = (g_acc[s] == ref["n_accepted"][s] and g_emit[s] == ref["n_emitted"][s] and
                g_last[s] == ref["last_node"][s] and np.array_equal(g_tok[s], ref["out_tokens"][s]))
        if same:
            exact += 1
            continue
        if ref["n_accepted"][s] < 0 or g_acc[s] < 0:
            fails.append(f"seq {s}: sentinel gpu {g_acc[s]} oracle {ref['n_accepted'][s]}")
            continue
        # first differing draw: the same node reached by the common prefix
        d = int(np.argmax(g_tok[s] != ref["out_tokens"][s]))
        v = 0
        for j in range(d):
            v = [c for c in range(v + 1, parents.shape[1])
                 if parents[s, c] == v and tokens[s, c] == ref["out_tokens"][s, j]][0]
        w = np.exp(oracle.log_softmax(z[s, v], T))
        if _boundaries_within(w, float(u[s, d]), int(g_tok[s, d]), int(ref["out_tokens"][s, d])):
            excused += 1
        else:
            fails.append(f"seq {s}: depth {d} gpu {g_tok[s, d]} oracle {ref['out_tokens'][s, d]} u={u[s, d]!r}")
    return exact, excused, fails


def _run(z, parents, tokens, u, T, dtype):
    out = uno.tree_verify(to_dev(z, dtype), to_dev(parents, "i32"), to_dev(tokens, "i32"), to_dev(u, "f32"), T)
    torch.cuda.synchronize()
    return tuple(to_host(t) for t in out)


CASES = [  # B, K, D, V, dtype, T
    (8, 2, 5, 1000, "bf16", 1.0),    # 63 nodes
    (5, 4, 3, 997, "f32", 0.7),      # 85 nodes, V % 8 != 0
    (3, 3, 4, 520, "bf16", 1.3),     # 121 nodes
    (40, 1, 6, 64, "bf16", 1.0),     # chains
    (6, 8, 1, 2048, "f32", 1.0),     # one level, eight siblings
    (2, 2, 2, 300000, "bf16", 1.0),  # rows past the walk's LDS staging: every node drawn either way
    (2, 2, 2, 240000, "bf16", 1.0),  # the walk's largest staging (15000 segments: masses and maxima)
    (2, 2, 10, 256, "bf16", 1.0),    # 2047 nodes: the walk reads the tree from memory, not LDS
]


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["walk", "nodes"])
@pytest.mark.parametrize("B,K,D,V,dtype,T", CASES)
def test_topk_trees_match_the_oracle(B, K, D, V, dtype, T, path, monkeypatch):
    monkeypatch.setenv("UNO_TREE_PATH", path)
    z, parents, tokens = tree_inputs(B, K, D, V, seed=B * 13 + K * 7 + D + V, noise=0.7)
    if dtype == "bf16":
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
    N = parents.shape[1]
    u = oracle.philox_uniforms(3, 0, 0, B * N).reshape(B, N)
    say("tree verify", path, B, K, D, V, dtype, T, "nodes", N)
    gpu = _run(z, parents, tokens, u, T, dtype)
    ref = oracle.tree.tree_verify(z, parents, tokens, u.astype(np.float64), T)
    exact, excused, fails = _compare(gpu, ref, z, parents, tokens, u, T)
    print(f"  exact {exact} excused {excused} mean accepted {np.mean(ref['n_accepted']):.2f}", flush=True)
    assert not fails, fails[:5]
    assert excused <= 1


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["walk", "nodes"])
def test_degenerate_trees(path, monkeypatch):
    monkeypatch.setenv("UNO_TREE_PATH", path)
    V = 16
    # root only; a certain chain; a malformed tree; duplicate siblings
    N = 4
    par = np.array([[-1, 0, 1, 2], [-1, 0, 1, 2], [-1, 0, 3, 1], [-1, 0, 0, 1]])
    tok = np.array([[0, 3, 1, 4], [0, 3, 1, 4], [0, 3, 1, 4], [0, 2, 2, 2]])
    z = np.zeros((4, N, V), np.float32)
    z[1] = -np.inf
    z[1, 0, 3] = z[1, 1, 1] = z[1, 2, 4] = z[1, 3, 9] = 0.0
    z[3] = -np.inf
    z[3, :, 2] = 0.0
    u = oracle.philox_uniforms(4, 0, 0, 4 * N).reshape(4, N)
    say("tree verify degenerate")
    gpu = _run(z, par, tok, u, 1.0, "f32")
    ref = oracle.tree.tree_verify(z, par, tok, u.astype(np.float64), 1.0)
    exact, excused, fails = _compare(gpu, ref, z, par, tok, u, 1.0)
    assert not fails and excused == 0
    assert list(gpu[0][1:]) == [3, -1, 2]     # certain chain, malformed tree, duplicate siblings
    assert list(gpu[3][1:]) == [3, -1, 3]     # (the duplicates are walked through node 1, the lower one)

    one = np.array([[-1]])
    out = _run(z[:1, :1], one, np.zeros((1, 1), np.int64), u[:1, :1], 1.0, "f32")
    assert out[0][0] == 0 and out[2][0] == 1 and out[3][0] == 0   # root only: the bonus draw


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deep_chain_walk_past_the_lds_tree(dtype, monkeypatch):
    """A chain of 1200 nodes whose every drafted child is certain: the walk goes to the leaf,
    reading parents, tokens and the depths' uniforms from memory past depth 1024."""
    monkeypatch.setenv("UNO_TREE_PATH", "walk")
    B, N, V = 2, 1200, 64
    rng = np.random.default_rng(21)
    par = np.tile(np.arange(-1, N - 1), (B, 1))
    tok = rng.integers(0, V, (B, N))
    tok[:, 0] = 0
    z = rng.standard_normal((B, N, V)).astype(np.float32)
    for s in range(B):
        for c in range(1, N):
            z[s, c - 1, :] = -np.inf
            z[s, c - 1, tok[s, c]] = 0.0   # the child's token is the only one with mass
    if dtype == "bf16":
        z = torch.from_numpy(z).to(torch.bfloat16).float().numpy()
    u = oracle.philox_uniforms(6, 0, 0, B * N).reshape(B, N)
    say("tree verify deep chain", B, N, V, dtype)
    gpu = _run(z, par, tok, u, 1.0, dtype)
    ref = oracle.tree.tree_verify(z, par, tok, u.astype(np.float64), 1.0)
    exact, excused, fails = _compare(gpu, ref, z, par, tok, u, 1.0)
    assert not fails and excused == 0
    assert np.all(gpu[0] == N - 1) and np.all(gpu[2] == N) and np.all(gpu[3] == N - 1)
    np.testing.assert_array_equal(gpu[1][:, :N - 1], tok[:, 1:])


@pytest.mark.gpu
@pytest.mark.parametrize("path", ["walk", "nodes"])
def test_full_vocabulary_trees_sampled_against_the_oracle(path, monkeypatch):
    monkeypatch.setenv("UNO_TREE_PATH", path)
    B, K, D, V, T = 32, 2, 5, 128256, 1.0
    N = 2 ** (D + 1) - 1
    say("tree verify full size", B, N, V)
    g = torch.Generator(device="cuda").manual_seed(11)
    base = torch.randn((B, D + 1, V), generator=g, device="cuda") * 3.0
    par0, _, depth = topk_tree(np.zeros((D, V)), K, D)
    parents = np.tile(par0, (B, 1))
    tokens = np.zeros((B, N), np.int64)
    base_host = base.cpu().numpy()
    for s in range(B):
        tokens[s] = topk_tree(base_host[s], K, D)[1]
    dep = torch.from_numpy(depth).cuda()
    z = (base[:, dep, :] + torch.randn((B, N, V), generator=g, device="cuda") * 0.7).to(torch.bfloat16).contiguous()
    u = oracle.philox_uniforms(5, 0, 0, B * N).reshape(B, N)
    out = uno.tree_verify(z, to_dev(parents, "i32"), to_dev(tokens, "i32"), to_dev(u, "f32"), T)
    torch.cuda.synchronize()
    gpu = tuple(to_host(t) for t in out)
    seqs = [0, 9, 21, 31]
    zh = z[seqs].float().cpu().numpy()
    ref = oracle.tree.tree_verify(zh, parents[seqs], tokens[seqs], u[seqs].astype(np.float64), T)
    exact, excused, fails = _compare(tuple(a[seqs] for a in gpu), ref, zh, parents[seqs], tokens[seqs], u[seqs], T)
    print(f"  sampled exact {exact} excused {excused}; mean accepted (all) {gpu[0].mean():.2f}", flush=True)
    assert not fails, fails[:5]
    assert np.all(gpu[2] == gpu[0] + 1)
