"""Pins of the CPU oracle against things other than itself.

Every oracle function is checked against at least one of: a hand-derived
fixture under tests/golden/, a closed form, an invariant, brute force on tiny
inputs, or an independent library routine (torch fp64 CPU).  The last test
plants typical mistakes into copies of the oracle's source and checks that
some pin fails for each one.
"""
import inspect
import itertools
import json
import math
import os
import textwrap
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import sparsevila as ov
import synthetic

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        if x == "ln2":
            return math.log(2.0)
        return float(Fraction(x))
    if isinstance(x, list):
        return [_num(v) for v in x]
    return float(x)


def _arr(x):
    return np.array(_num(x), dtype=np.float64)


# ---------------------------------------------------------------- fixtures
def test_golden_retrieval(golden_dir):
    g = _load(golden_dir, "retrieval_gqa.json")
    q, K = _arr(g["q"]), _arr(g["K"])
    s = oracle.retrieval_scores(q, K)
    np.testing.assert_array_equal(s[0], np.array(g["expected_scores"], dtype=np.float64))
    for k, want in g["expected_topk"].items():
        got = oracle.retrieve(q, K, int(k))
        assert got[0].tolist() == want, (k, got)


def test_golden_attention(golden_dir):
    g = _load(golden_dir, "attention_sparse.json")
    out = oracle.sparse_decode_attn(_arr(g["q"]), _arr(g["k_vis"]), _arr(g["v_vis"]),
                                    np.array(g["idx"]), _arr(g["k_txt"]), _arr(g["v_txt"]),
                                    np.array(g["txt_len"]))
    np.testing.assert_allclose(out, _arr(g["expected"]), rtol=1e-14, atol=1e-14)


def test_golden_salience(golden_dir):
    g = _load(golden_dir, "salience_3tok.json")
    Q, K = _arr(g["Q"]), _arr(g["K"])
    s, idx = oracle.salience_prune(Q, K, g["keep"])
    np.testing.assert_allclose(s[0], _arr(g["expected"]), rtol=1e-14, atol=1e-15)
    assert idx[0].tolist() == g["expected_keep_idx"]


# ---------------------------------------------------------------- retrieval
def _loop_scores(q, K):
    """Python-loop scores with math.fsum (brute force)."""
    B, Tq, Hq, D = q.shape
    N, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    s = np.zeros((B, N))
    for b in range(B):
        for t in range(N):
            s[b, t] = math.fsum(float(q[b, tau, h, d]) * float(K[b, t, h // G, d])
                                for tau in range(Tq) for h in range(Hq) for d in range(D))
    return s


@pytest.mark.parametrize("Tq,Hq,Hkv", [(1, 4, 4), (1, 6, 2), (3, 4, 1)])
def test_retrieval_bruteforce(Tq, Hq, Hkv):
    rng = np.random.default_rng(7 + Tq + Hq)
    B, N, D = 2, 8, 5
    q = rng.standard_normal((B, Tq, Hq, D))
    K = rng.standard_normal((B, N, Hkv, D))
    s = oracle.retrieval_scores(q, K)
    np.testing.assert_allclose(s, _loop_scores(q, K), rtol=1e-12, atol=1e-12)
    for k in range(N + 1):
        idx = oracle.retrieve(q, K, k)
        for b in range(B):
            best = max(itertools.combinations(range(N), k), key=lambda c: math.fsum(s[b, list(c)]))
            assert idx[b].tolist() == sorted(best)


def test_topk_matches_torch():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((5, 1000))
    for k in (1, 17, 250, 1000):
        ref = torch.topk(torch.from_numpy(s), k, dim=1).indices.numpy()
        got = oracle.topk_ascending(s, k)
        for r in range(5):
            assert set(got[r].tolist()) == set(ref[r].tolist())
            assert np.all(np.diff(got[r]) > 0)


def test_topk_ties_and_edges():
    s = np.array([[1.0, 3.0, 3.0, 3.0, 0.0, 3.0]])
    assert oracle.topk_ascending(s, 2)[0].tolist() == [1, 2]
    assert oracle.topk_ascending(s, 4)[0].tolist() == [1, 2, 3, 5]
    assert oracle.topk_ascending(s, 0).shape == (1, 0)
    assert oracle.topk_ascending(s, 6)[0].tolist() == list(range(6))
    # -0.0 and +0.0 are equal values: the lower index wins
    z = np.array([[-0.0, 0.0, -1.0]])
    assert oracle.topk_ascending(z, 1)[0].tolist() == [0]
    with pytest.raises(ValueError):
        oracle.topk_ascending(s, 7)
    with pytest.raises(ValueError):
        oracle.topk_ascending(s, -1)


def test_retrieval_planted_image576():
    """Planted keys (K += 3 q/|q| per head) dominate by construction."""
    w = synthetic.DECODE["image576_fp32"]
    for seed in (0, 1, 2):
        d = synthetic.make_decode_layer(w, seed)
        planted = set(d["planted"][0].tolist())
        got = oracle.retrieve(d["q"], d["k_vis"], w.planted)
        assert set(got[0].tolist()) == planted
        got = oracle.retrieve(d["q"], d["k_vis"], w.k)
        assert planted <= set(got[0].tolist())


def test_retrieval_planted_llava_layer():
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=2)
    d = synthetic.make_decode_layer(w, 0, layer=3)
    got = oracle.retrieve(d["q"], d["k_vis"], w.k)
    for b in range(w.B):
        assert set(d["planted"][b].tolist()) <= set(got[b].tolist())


def test_retrieval_invariances():
    rng = np.random.default_rng(11)
    B, N, Hq, Hkv, D = 2, 64, 6, 2, 16
    q = rng.standard_normal((B, 1, Hq, D))
    K = rng.standard_normal((B, N, Hkv, D))
    k = 13
    base = oracle.retrieve(q, K, k)
    # common vector added to every key shifts every score equally
    u = rng.standard_normal((1, 1, Hkv, D))
    assert np.array_equal(oracle.retrieve(q, K + u, k), base)
    # positive rescaling of the query
    assert np.array_equal(oracle.retrieve(2.5 * q, K, k), base)
    # token permutation permutes the indices
    perm = rng.permutation(N)
    got = oracle.retrieve(q, K[:, perm], k)
    for b in range(B):
        assert sorted(perm[got[b]].tolist()) == base[b].tolist()
    # equal query heads inside each group: s = G * (q_g . K_g) summed over groups
    qe = np.repeat(q[:, :, ::3], 3, axis=2)
    s = oracle.retrieval_scores(qe, K)
    want = 3.0 * np.einsum("bgd,bngd->bn", qe[:, 0, ::3], K)
    np.testing.assert_allclose(s, want, rtol=1e-12)
    # several query tokens: the scores add
    q2 = rng.standard_normal((B, 2, Hq, D))
    np.testing.assert_allclose(oracle.retrieval_scores(q2, K),
                               oracle.retrieval_scores(q2[:, :1], K)
                               + oracle.retrieval_scores(q2[:, 1:], K), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- attention
def _rand_attn(rng, B=2, N=40, Hq=4, Hkv=2, D=8, Tmax=10):
    q = rng.standard_normal((B, Hq, D))
    kv = rng.standard_normal((B, N, Hkv, D))
    vv = rng.standard_normal((B, N, Hkv, D))
    kt = rng.standard_normal((B, Tmax, Hkv, D))
    vt = rng.standard_normal((B, Tmax, Hkv, D))
    return q, kv, vv, kt, vt


def test_attention_k_equals_n_is_dense_bitwise():
    rng = np.random.default_rng(5)
    q, kv, vv, kt, vt = _rand_attn(rng)
    tl = np.array([7, 10])
    idx = np.tile(np.arange(kv.shape[1]), (2, 1))
    a = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    b = oracle.dense_decode_attn(q, kv, vv, kt, vt, tl)
    assert np.array_equal(a, b)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(6)
    q, kv, vv, kt, vt = _rand_attn(rng)
    tl = np.array([3, 10])
    idx = np.stack([np.sort(rng.choice(40, 12, replace=False)) for _ in range(2)])
    out = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    G = 2
    for b in range(2):
        KE = np.concatenate([kv[b, idx[b]], kt[b, :tl[b]]])
        VE = np.concatenate([vv[b, idx[b]], vt[b, :tl[b]]])
        for h in range(4):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h][None, None]), torch.from_numpy(KE[None, :, h // G]),
                torch.from_numpy(VE[None, :, h // G]))
            np.testing.assert_allclose(out[b, h], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    q, kv, vv, kt, vt = _rand_attn(rng)
    tl = np.array([4, 9])
    idx = np.stack([np.sort(rng.choice(40, 6, replace=False)) for _ in range(2)])
    # every V row equal -> out = v
    v = rng.standard_normal(8)
    out = oracle.sparse_decode_attn(q, kv, np.broadcast_to(v, vv.shape), idx, kt,
                                    np.broadcast_to(v, vt.shape), tl)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=1e-14, atol=1e-14)
    # every key equal -> mean of V over E
    kc = np.broadcast_to(rng.standard_normal(8), kv.shape)
    out = oracle.sparse_decode_attn(q, kc, vv, idx, np.broadcast_to(kc[0, 0, 0], kt.shape), vt, tl)
    for b in range(2):
        VE = np.concatenate([vv[b, idx[b]], vt[b, :tl[b]]])
        for h in range(4):
            np.testing.assert_allclose(out[b, h], VE[:, h // 2].mean(axis=0), rtol=1e-13, atol=1e-14)
    # |E| = 1 -> that V row
    out = oracle.sparse_decode_attn(q, kv, vv, idx[:, :1], kt, vt, np.array([0, 0]))
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[b, h], vv[b, idx[b, 0], h // 2])
    # permuting the visual entries leaves the output unchanged
    perm = rng.permutation(6)
    a = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    b_ = oracle.sparse_decode_attn(q, kv, vv, idx[:, perm], kt, vt, tl)
    np.testing.assert_allclose(a, b_, rtol=1e-13, atol=1e-14)


def test_attention_split_combine_algebra():
    """Chunked partials (m, l, acc) merged with max-rescaling equal the one-shot result."""
    rng = np.random.default_rng(9)
    D, E = 16, 37
    q = rng.standard_normal(D)
    K = rng.standard_normal((E, D)) * 2
    V = rng.standard_normal((E, D))
    z = K @ q / math.sqrt(D)
    parts = []
    for c in np.array_split(np.arange(E), 5):
        m = z[c].max()
        p = np.exp(z[c] - m)
        parts.append((m, p.sum(), p @ V[c]))
    M = max(m for m, _, _ in parts)
    num = sum(math.exp(m - M) * a for m, _, a in parts)
    den = sum(math.exp(m - M) * l for m, l, _ in parts)
    one = oracle.sparse_decode_attn(q[None, None], K[None, :, None], V[None, :, None],
                                    np.arange(E)[None], np.zeros((1, 0, 1, D)),
                                    np.zeros((1, 0, 1, D)), np.array([0]))
    np.testing.assert_allclose(num / den, one[0, 0], rtol=1e-13, atol=1e-14)


def _loop_attn(q, kv, vv, idx, kt, vt, tl):
    """Python-loop decode attention with math.fsum (brute force)."""
    B, Hq, D = q.shape
    G = Hq // kv.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        rows = [(kv[b, j], vv[b, j]) for j in idx[b]] + [(kt[b, t], vt[b, t]) for t in range(tl[b])]
        for h in range(Hq):
            z = [math.fsum(q[b, h, d] * kr[h // G, d] for d in range(D)) / math.sqrt(D) for kr, _ in rows]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = math.fsum(w)
            for d in range(D):
                out[b, h, d] = math.fsum(w[j] * rows[j][1][h // G, d] for j in range(len(rows))) / tot
    return out


def test_attention_bruteforce_gqa():
    rng = np.random.default_rng(19)
    q, kv, vv, kt, vt = _rand_attn(rng, B=2, N=9, Hq=6, Hkv=2, D=4, Tmax=3)
    idx, tl = np.array([[0, 3, 8], [2, 5, 7]]), np.array([3, 1])
    out = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    np.testing.assert_allclose(out, _loop_attn(q, kv, vv, idx, kt, vt, tl), rtol=1e-13, atol=1e-14)


def test_attention_bruteforce_loops():
    rng = np.random.default_rng(10)
    q, kv, vv, kt, vt = _rand_attn(rng, B=1, N=6, Hq=2, Hkv=1, D=3, Tmax=2)
    idx, tl = np.array([[1, 4]]), np.array([2])
    out = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    rows_k = [kv[0, 1, 0], kv[0, 4, 0], kt[0, 0, 0], kt[0, 1, 0]]
    rows_v = [vv[0, 1, 0], vv[0, 4, 0], vt[0, 0, 0], vt[0, 1, 0]]
    for h in range(2):
        z = [math.fsum(q[0, h, d] * r[d] for d in range(3)) / math.sqrt(3) for r in rows_k]
        w = [math.exp(x) for x in z]
        tot = math.fsum(w)
        for d in range(3):
            want = math.fsum(w[j] * rows_v[j][d] for j in range(4)) / tot
            assert abs(out[0, h, d] - want) < 1e-13


def test_attention_empty_set_raises():
    rng = np.random.default_rng(1)
    q, kv, vv, kt, vt = _rand_attn(rng, B=1)
    with pytest.raises(ValueError):
        oracle.sparse_decode_attn(q, kv, vv, np.zeros((1, 0), dtype=np.int64), kt, vt, np.array([0]))


# ---------------------------------------------------------------- summary-token salience

def test_summary_salience_all_tokens_is_the_intra_visual_mean():
    # Every token a summary token: the no-summary (SigLIP/QwenVL) definition.
    rng = np.random.default_rng(21)
    Q, K = _rand_sal(rng, F=2, H=3, N=12, D=8)
    np.testing.assert_allclose(oracle.summary_salience(Q, K, 12), oracle.salience(Q, K),
                               rtol=1e-13, atol=1e-16)


def test_summary_salience_one_token_is_scipy_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(22)
    Q, K = _rand_sal(rng, F=3, H=1, N=17, D=8)
    got = oracle.summary_salience(Q, K, 1)
    for f in range(3):
        want = softmax(K[f, 0] @ Q[f, 0, 0] / math.sqrt(8))
        np.testing.assert_allclose(got[f], want, rtol=1e-13)


def test_summary_salience_bruteforce_and_sums():
    rng = np.random.default_rng(23)
    F, H, N, D, S = 2, 2, 7, 4, 3
    Q, K = _rand_sal(rng, F=F, H=H, N=N, D=D)
    got = oracle.summary_salience(Q, K, S, scale=0.7)
    want = np.zeros((F, N))
    for f in range(F):
        for h in range(H):
            for s in range(S):
                z = [sum(Q[f, h, s, d] * K[f, h, j, d] for d in range(D)) * 0.7 for j in range(N)]
                e = [math.exp(v) for v in z]
                for j in range(N):
                    want[f, j] += e[j] / sum(e) / (S * H)
    np.testing.assert_allclose(got, want, rtol=1e-12)
    np.testing.assert_allclose(got.sum(axis=1), 1.0, rtol=1e-13)
    # rows S.. do not matter
    Q2 = Q.copy()
    Q2[:, :, S:] = rng.standard_normal(Q2[:, :, S:].shape)
    np.testing.assert_array_equal(oracle.summary_salience(Q2, K, S, scale=0.7), got)
    _, idx = oracle.summary_salience_prune(Q, K, S, 4, scale=0.7)
    assert idx.shape == (F, 4) and all(list(r) == sorted(r) for r in idx.tolist())
    with pytest.raises(ValueError):
        oracle.summary_salience(Q, K, 0)


# ---------------------------------------------------------------- dense packing

def _coded_cache(B, N, Hkv, D, tag):
    """Cache whose every value spells out its own (b, t, g, d) position."""
    b, t, g, d = np.meshgrid(np.arange(B), np.arange(N), np.arange(Hkv), np.arange(D),
                             indexing="ij")
    return tag * 1e7 + b * 1e5 + t * 1e2 + g * 1e1 + d * 1e0 + 0.25


def _pack_decodes(kp, vp, idx, N):
    """kp/vp hold, at (b, j, g, d), the code of (b, idx[b, j], g, d); zero if outside."""
    B, k, Hkv, D = kp.shape
    for b in range(B):
        for j in range(k):
            t = int(idx[b, j])
            for g in range(Hkv):
                for d in range(D):
                    want_k = 1e7 + b * 1e5 + t * 1e2 + g * 1e1 + d + 0.25 if 0 <= t < N else 0.0
                    want_v = 2e7 + b * 1e5 + t * 1e2 + g * 1e1 + d + 0.25 if 0 <= t < N else 0.0
                    if kp[b, j, g, d] != want_k or vp[b, j, g, d] != want_v:
                        return False
    return True


def test_pack_decodes_positions():
    B, N, Hkv, D = 3, 11, 2, 4
    K, V = _coded_cache(B, N, Hkv, D, 1), _coded_cache(B, N, Hkv, D, 2)
    idx = np.array([[0, 4, 10], [9, 1, 3], [10, -1, 11]])
    kp, vp = oracle.pack_selected(K, V, idx)
    assert kp.shape == (B, 3, Hkv, D) and vp.shape == (B, 3, Hkv, D)
    assert _pack_decodes(kp, vp, idx, N)


def test_pack_identity_reverse_and_torch():
    rng = np.random.default_rng(11)
    K, V = rng.standard_normal((2, 9, 3, 5)), rng.standard_normal((2, 9, 3, 5))
    ident = np.tile(np.arange(9), (2, 1))
    kp, vp = oracle.pack_selected(K, V, ident)
    assert np.array_equal(kp, K) and np.array_equal(vp, V)
    kp, vp = oracle.pack_selected(K, V, ident[:, ::-1])
    assert np.array_equal(kp, np.flip(K, axis=1)) and np.array_equal(vp, np.flip(V, axis=1))
    idx = np.array([[2, 3, 7, 8], [0, 1, 5, 6]])
    kp, _ = oracle.pack_selected(K, V, idx)
    tk = torch.from_numpy(K)
    want = torch.stack([tk[b].index_select(0, torch.from_numpy(idx[b])) for b in range(2)])
    assert np.array_equal(kp, want.numpy())
    kp, vp = oracle.pack_selected(K, V, np.zeros((2, 0), dtype=np.int64))
    assert kp.shape == (2, 0, 3, 5) and vp.shape == (2, 0, 3, 5)


def test_pack_then_attend_equals_sparse_attention_bitwise():
    # Attending the packed rows 0..k-1 is the attention over the selected set.
    rng = np.random.default_rng(12)
    q, kv, vv, kt, vt = _rand_attn(rng, B=2, N=30, Hq=6, Hkv=2, D=8, Tmax=5)
    idx, tl = np.array([[1, 4, 9, 29], [0, 2, 17, 18]]), np.array([5, 2])
    kp, vp = oracle.pack_selected(kv, vv, idx)
    a = oracle.sparse_decode_attn(q, kp, vp, np.tile(np.arange(4), (2, 1)), kt, vt, tl)
    b = oracle.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- salience
def _rand_sal(rng, F=2, H=3, N=20, D=8, std=1.0):
    return rng.standard_normal((F, H, N, D)) * std, rng.standard_normal((F, H, N, D)) * std


def test_salience_sums_to_one_and_is_positive():
    rng = np.random.default_rng(12)
    Q, K = _rand_sal(rng, std=2.0)
    s = oracle.salience(Q, K)
    np.testing.assert_allclose(s.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(s > 0)


def test_salience_uniform_cases():
    rng = np.random.default_rng(13)
    Q, K = _rand_sal(rng)
    np.testing.assert_allclose(oracle.salience(np.zeros_like(Q), K), 1 / 20, rtol=1e-14)
    Kc = np.broadcast_to(K[:, :, :1], K.shape)
    np.testing.assert_allclose(oracle.salience(Q, Kc), 1 / 20, rtol=1e-13)
    s1 = oracle.salience(Q[:, :, :1], K[:, :, :1])
    np.testing.assert_array_equal(s1, np.ones((2, 1)))


def test_salience_shift_and_permutation():
    rng = np.random.default_rng(14)
    Q, K = _rand_sal(rng)
    s = oracle.salience(Q, K)
    u = rng.standard_normal((2, 3, 1, 8))
    np.testing.assert_allclose(oracle.salience(Q, K + u), s, rtol=1e-12)
    perm = rng.permutation(20)
    np.testing.assert_allclose(oracle.salience(Q[:, :, perm], K[:, :, perm]), s[:, perm], rtol=1e-12)
    # Q rows alone permuted: the column means do not change
    np.testing.assert_allclose(oracle.salience(Q[:, :, perm], K), s, rtol=1e-12)


def test_salience_planted_sink_monotone():
    rng = np.random.default_rng(15)
    Q, K = _rand_sal(rng, F=1, H=1, N=16, D=8)
    Q = np.abs(Q)            # every query row then has q_i . u > 0, so the limit is 1
    u = Q[0, 0].mean(axis=0)
    u /= np.linalg.norm(u)
    vals = []
    for c in (0.0, 2.0, 5.0, 10.0, 40.0, 200.0):
        K2 = K.copy()
        K2[0, 0, 5] += c * u
        vals.append(oracle.salience(Q, K2)[0, 5])
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert vals[-1] > 0.99


def test_salience_matches_torch_softmax():
    rng = np.random.default_rng(16)
    Q, K = _rand_sal(rng, std=1.5)
    s = oracle.salience(Q, K)
    Qt, Kt = torch.from_numpy(Q), torch.from_numpy(K)
    A = torch.softmax(Qt @ Kt.transpose(-1, -2) / math.sqrt(8), dim=-1)
    ref = A.mean(dim=2).mean(dim=1).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-12)


def test_salience_bruteforce_loops():
    rng = np.random.default_rng(17)
    Q, K = _rand_sal(rng, F=1, H=2, N=5, D=3)
    s = oracle.salience(Q, K)
    for j in range(5):
        acc = []
        for h in range(2):
            for i in range(5):
                z = [math.fsum(Q[0, h, i, d] * K[0, h, jj, d] for d in range(3)) / math.sqrt(3)
                     for jj in range(5)]
                e = [math.exp(x) for x in z]
                acc.append(e[j] / math.fsum(e))
        assert abs(s[0, j] - math.fsum(acc) / 10) < 1e-15


def test_salience_prune_keep_and_ties():
    rng = np.random.default_rng(18)
    Q, K = _rand_sal(rng)
    s, idx = oracle.salience_prune(Q, K, 7)
    for f in range(2):
        kept = set(idx[f].tolist())
        assert len(kept) == 7 and np.all(np.diff(idx[f]) > 0)
        assert min(s[f, list(kept)]) >= max(s[f, [j for j in range(20) if j not in kept]])
    # all tokens tie (Q = 0): the lowest indices are kept
    _, idx0 = oracle.salience_prune(np.zeros_like(Q), K, 5)
    assert idx0.tolist() == [list(range(5))] * 2


def test_synthetic_salience_statistics():
    """The SigLIP-shaped workload: near-uniform attention, salience sums to 1."""
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=2)
    Q, K = synthetic.make_salience(w, 0)
    assert Q.shape == (2, 16, 729, 72) and Q.dtype == torch.bfloat16
    assert abs(Q.float().std().item() - 72 ** -0.25) < 0.01
    s = oracle.salience(Q, K)
    np.testing.assert_allclose(s.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.abs(s * 729 - 1) < 0.1)


# ---------------------------------------------------------------- prefill attention of a question chunk
def _prefill_inputs(B=2, Tq=5, Hq=4, Hkv=2, D=8, N=7, Tmax=9, seed=0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)  # noqa: E731
    return (r(B, Tq, Hq, D), r(B, N, Hkv, D), r(B, N, Hkv, D), r(B, Tmax, Hkv, D),
            r(B, Tmax, Hkv, D), np.array([Tmax, Tq + 2][:B]))


def test_prefill_last_token_is_dense_decode_bitwise():
    """The question's last token sees every text row: the dense decode attention."""
    q, kv, vv, kt, vt, tl = _prefill_inputs()
    out = oracle.prefill_attention(q, kv, vv, kt, vt, tl)
    dense = oracle.dense_decode_attn(q[:, -1], kv, vv, kt, vt, tl)
    np.testing.assert_array_equal(out[:, -1], dense)


def test_prefill_is_causal():
    """Text rows after a token's position cannot change its output; they do
    change the outputs of the tokens that see them."""
    q, kv, vv, kt, vt, tl = _prefill_inputs(B=1)
    tl = np.array([9])
    a = oracle.prefill_attention(q, kv, vv, kt, vt, tl)
    kt2, vt2 = kt.clone(), vt.clone()
    kt2[:, 7:] += 3.0                     # rows 7, 8: seen by tau = 3, 4 only (p = 4 + tau)
    vt2[:, 7:] -= 2.0
    b = oracle.prefill_attention(q, kv, vv, kt2, vt2, tl)
    np.testing.assert_array_equal(a[:, :3], b[:, :3])
    assert np.abs(a[:, 3:] - b[:, 3:]).min() > 0
    # rows past txt_len are never read
    kt3 = kt.clone()
    kt3[:, 9:] = float("nan")
    np.testing.assert_array_equal(a, oracle.prefill_attention(q, kv, vv, kt3, vt, tl))


def test_prefill_matches_torch_masked_softmax():
    """Against torch fp64: logits with an explicit mask (visual keys all visible,
    text keys causal) filled with -inf, torch.softmax, then a matmul with V."""
    B, Tq, Hq, Hkv, D, N, Tmax = 2, 6, 6, 3, 16, 11, 10
    q, kv, vv, kt, vt, _ = _prefill_inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=3)
    tl = np.array([10, 4])                # second sequence: the first two tokens see no text
    out = oracle.prefill_attention(q, kv, vv, kt, vt, tl)
    G = Hq // Hkv
    for b in range(B):
        K = torch.cat([kv[b], kt[b]], 0).repeat_interleave(G, dim=1).permute(1, 0, 2)
        V = torch.cat([vv[b], vt[b]], 0).repeat_interleave(G, dim=1).permute(1, 0, 2)
        mask = torch.zeros(Tq, N + Tmax, dtype=torch.bool)
        mask[:, :N] = True
        for tau in range(Tq):
            p = int(tl[b]) - Tq + tau
            mask[tau, N:N + max(p + 1, 0)] = True
        z = torch.matmul(q[b].permute(1, 0, 2), K.transpose(1, 2).contiguous()) / math.sqrt(D)
        z = z.masked_fill(~mask, float("-inf"))
        ref = torch.matmul(torch.softmax(z, dim=-1), V)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefill_bruteforce_loops():
    q, kv, vv, kt, vt, tl = _prefill_inputs(B=1, Tq=3, Hq=2, Hkv=1, D=3, N=2, Tmax=4, seed=5)
    tl = np.array([4])
    out = oracle.prefill_attention(q, kv, vv, kt, vt, tl)
    for tau in range(3):
        p = 4 - 3 + tau
        rows = [(kv[0, j], vv[0, j]) for j in range(2)] + [(kt[0, j], vt[0, j]) for j in range(p + 1)]
        for h in range(2):
            z = [sum(float(q[0, tau, h, d]) * float(K[0, d]) for d in range(3)) / math.sqrt(3)
                 for K, _ in rows]
            m = max(z)
            w = [math.exp(v - m) for v in z]
            tot = math.fsum(w)
            for d in range(3):
                want = math.fsum(w[j] * float(rows[j][1][0, d]) for j in range(len(rows))) / tot
                assert abs(out[0, tau, h, d] - want) < 1e-13

# ---------------------------------------------------------------- mutation check
_MUTANTS = [
    ("salience", "A.sum(axis=0) / N", "A.sum(axis=1) / N", "row mean instead of column mean"),
    ("salience", "Q[f, h] @ K[f, h].T", "K[f, h] @ Q[f, h].T", "transposed QK^T"),
    ("salience", "s[f] /= H", "s[f] /= 1", "heads summed, not averaged"),
    ("salience", "scale = 1.0 / math.sqrt(D)", "scale = 1.0", "missing 1/sqrt(D)"),
    ("retrieval_scores", "K[b, :, h // G, :]", "K[b, :, h % Hkv, :]", "wrong GQA head mapping"),
    ("retrieval_scores", "for tau in range(Tq)", "for tau in range(1)", "dropped query tokens"),
    ("topk_ascending", "np.lexsort((idx, -s[r]))", "np.lexsort((-idx, -s[r]))", "ties to the higher index"),
    ("sparse_decode_attn", "Kt[b, :T]", "Kt[b]", "text rows beyond txt_len"),
    ("sparse_decode_attn", "scale = 1.0 / math.sqrt(D)", "scale = 1.0", "missing 1/sqrt(D)"),
    ("sparse_decode_attn", "z = (KE[:, g, :] @ q[b, h]) * scale", "z = (KE[:, 0, :] @ q[b, h]) * scale",
     "every head reads KV head 0"),
    ("pack_selected", "vp[b, j] = Vv[b, t]", "vp[b, j] = Kv[b, t]", "pack copies K into V"),
    ("summary_salience", "Q[f, h, :S] @ K[f, h].T", "Q[f, h, 1:S + 1] @ K[f, h].T",
     "summary rows shifted by one"),
    ("summary_salience", "out[f] += A.sum(axis=0) / S", "out[f] += A.sum(axis=1).mean() / S",
     "row sums instead of column sums"),
    ("summary_salience", "out[f] /= H", "out[f] /= 1", "heads summed, not averaged"),
    ("pack_selected", "if 0 <= t < N:", "if 0 <= t < N - 1:", "pack drops the last token"),
    ("pack_selected", "kp[b, j] = Kv[b, t]", "kp[b, j] = Kv[0, t]", "pack reads sequence 0"),
    ("prefill_attention", "p = min(T - Tq + tau, T - 1)", "p = min(T - Tq + tau + 1, T - 1)",
     "prefill sees one text row too many"),
    ("prefill_attention", "p = min(T - Tq + tau, T - 1)", "p = T - 1",
     "prefill without the causal mask"),
    ("prefill_attention", "z = (KE[:, g, :] @ q[b, tau, h]) * scale",
     "z = (KE[:, g, :] @ q[b, 0, h]) * scale", "prefill uses the first token's query"),
]


def _mutant_module(fn_name, old, new):
    ns = dict(vars(ov))
    src = textwrap.dedent(inspect.getsource(getattr(ov, fn_name)))
    assert old in src, (fn_name, old)
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), ns)
    # functions defined in ns call each other through ns
    for name in ("retrieve", "dense_decode_attn", "salience_prune"):
        src2 = textwrap.dedent(inspect.getsource(getattr(ov, name)))
        exec(compile(src2, f"<copy {name}>", "exec"), ns)

    class M:
        pass

    m = M()
    for n in ov.__all__:
        setattr(m, n, ns[n])
    return m


def _loop_prefill(q, kv, vv, kt, vt, tl):
    """Causal prefill attention with Python loops and math.fsum (token tau at text
    position tl - Tq + tau sees every visual row and text rows up to it)."""
    B, Tq, Hq, D = q.shape
    N, Hkv = kv.shape[1], kv.shape[2]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for tau in range(Tq):
            last = int(tl[b]) - Tq + tau
            rows = [(kv[b, j], vv[b, j]) for j in range(N)]
            rows += [(kt[b, j], vt[b, j]) for j in range(0, max(last + 1, 0))]
            for h in range(Hq):
                z = [math.fsum(q[b, tau, h, d] * K[h // G, d] for d in range(D)) / math.sqrt(D)
                     for K, _ in rows]
                mx = max(z)
                w = [math.exp(v - mx) for v in z]
                tot = math.fsum(w)
                for d in range(D):
                    out[b, tau, h, d] = math.fsum(w[j] * rows[j][1][h // G, d]
                                                  for j in range(len(rows))) / tot
    return out


def _pins_pass(m, golden_dir):
    """Run a compact subset of the pins against module-like ``m``; True if all pass."""
    try:
        g = _load(golden_dir, "salience_3tok.json")
        s, idx = m.salience_prune(_arr(g["Q"]), _arr(g["K"]), g["keep"])
        if not np.allclose(s[0], _arr(g["expected"]), rtol=1e-14, atol=1e-15):
            return False
        if idx[0].tolist() != g["expected_keep_idx"]:
            return False
        g = _load(golden_dir, "retrieval_gqa.json")
        if not np.array_equal(m.retrieval_scores(_arr(g["q"]), _arr(g["K"]))[0],
                              np.array(g["expected_scores"], dtype=float)):
            return False
        for k, want in g["expected_topk"].items():
            if m.retrieve(_arr(g["q"]), _arr(g["K"]), int(k))[0].tolist() != want:
                return False
        rng = np.random.default_rng(7)
        q = rng.standard_normal((1, 3, 4, 5))
        K = rng.standard_normal((1, 8, 2, 5))
        if not np.allclose(m.retrieval_scores(q, K), _loop_scores(q, K), rtol=1e-12):
            return False
        q, kv, vv, kt, vt = _rand_attn(rng, B=2, N=9, Hq=6, Hkv=2, D=4, Tmax=3)
        idx, tl = np.array([[0, 3, 8], [2, 5, 7]]), np.array([3, 1])
        if not np.allclose(m.sparse_decode_attn(q, kv, vv, idx, kt, vt, tl),
                           _loop_attn(q, kv, vv, idx, kt, vt, tl), rtol=1e-12, atol=1e-13):
            return False
        from scipy.special import softmax
        Qs, Ks = rng.standard_normal((2, 2, 6, 4)), rng.standard_normal((2, 2, 6, 4))
        ss = m.summary_salience(Qs, Ks, 2)
        want = sum(softmax(Ks[0, h] @ Qs[0, h, s] / 2.0) for h in range(2) for s in range(2)) / 4
        if not np.allclose(ss[0], want, rtol=1e-12):
            return False
        Kc, Vc = _coded_cache(2, 7, 2, 3, 1), _coded_cache(2, 7, 2, 3, 2)
        pidx = np.array([[0, 6, 3], [6, 2, 7]])
        if not _pack_decodes(*m.pack_selected(Kc, Vc, pidx), pidx, 7):
            return False
        qp = rng.standard_normal((2, 3, 4, 3))
        kvp, vvp = rng.standard_normal((2, 2, 2, 3)), rng.standard_normal((2, 2, 2, 3))
        ktp, vtp = rng.standard_normal((2, 5, 2, 3)), rng.standard_normal((2, 5, 2, 3))
        tlp = np.array([5, 2])
        if not np.allclose(m.prefill_attention(qp, kvp, vvp, ktp, vtp, tlp),
                           _loop_prefill(qp, kvp, vvp, ktp, vtp, tlp), rtol=1e-12, atol=1e-13):
            return False
        g = _load(golden_dir, "attention_sparse.json")
        out = m.sparse_decode_attn(_arr(g["q"]), _arr(g["k_vis"]), _arr(g["v_vis"]),
                                   np.array(g["idx"]), _arr(g["k_txt"]), _arr(g["v_txt"]),
                                   np.array(g["txt_len"]))
        return bool(np.allclose(out, _arr(g["expected"]), rtol=1e-14, atol=1e-14))
    except Exception:
        return False


def test_pins_pass_on_oracle(golden_dir):
    assert _pins_pass(ov, golden_dir)


@pytest.mark.parametrize("fn,old,new,what", _MUTANTS, ids=[m[3] for m in _MUTANTS])
def test_pins_catch_planted_mistake(fn, old, new, what, golden_dir):
    assert not _pins_pass(_mutant_module(fn, old, new), golden_dir), what
