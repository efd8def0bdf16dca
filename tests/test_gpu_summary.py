"""GPU parity of summary-token salience (sv_summary_salience_prune) against the
fp64 CPU oracle: salience within 1e-4 relative per element and summing to 1
within 1e-5 per frame; kept sets exact up to swaps inside the 1e-5 relative
band at the keep-th value (tests/accept.py).
"""
import dataclasses

import numpy as np
import pytest
import torch

import accept
import oracle
import synthetic
import visual_token_sparsity_amd as sv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(name, F, H, N, D, seed=0):
    base = synthetic.SALIENCE["clip_l14_336_256f"]
    w = dataclasses.replace(base, name=name, F=F, H=H, N=N, D=D, std=D ** -0.25)
    return synthetic.make_salience(w, seed)


CASES = [
    # name, F, H, N, D, S, keep
    ("clip_l14_336", 3, 16, 577, 64, 1, 288),
    ("radio_4_summary", 2, 16, 1028, 64, 4, 514),
    ("max_logits_s16", 2, 4, 768, 128, 16, 100),
    ("max_n_4096", 1, 2, 4096, 72, 3, 1000),
    ("ragged_d8", 4, 3, 37, 8, 2, 5),
    ("d16_s5", 2, 3, 301, 16, 5, 77),
    ("d32_s2", 2, 5, 1000, 32, 2, 499),
    ("d96_row_per_lane", 2, 4, 333, 96, 3, 100),
    ("s1_d8", 2, 3, 257, 8, 1, 40),
    ("s1_d16", 2, 3, 300, 16, 1, 30),
    ("s1_d32", 2, 3, 1001, 32, 1, 500),
    ("s1_d128", 2, 3, 4096, 128, 1, 2048),
    ("s1_d72_row_per_lane", 2, 3, 729, 72, 1, 364),
    ("n_one", 3, 2, 1, 64, 1, 1),
    ("keep_zero", 2, 2, 50, 64, 1, 0),
]


@pytest.mark.parametrize("name,F,H,N,D,S,keep", CASES, ids=[c[0] for c in CASES])
def test_summary_salience_parity(name, F, H, N, D, S, keep):
    _say("summary salience", name, F, H, N, D, S, keep)
    Q, K = _inputs(name, F, H, N, D)
    sal, idx = sv.summary_salience_prune(Q.to(DEV), K.to(DEV), S, keep)
    torch.cuda.synchronize()
    ref = oracle.summary_salience(Q, K, S)
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), ref)
    assert ok, (rel, sm)
    if keep:
        ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), ref, keep)
        assert ok, msgs


def test_summary_all_tokens_matches_intra_visual_salience():
    """S = N: every token is a summary token, which is the no-summary definition."""
    F, H, N, D = 3, 4, 16, 64                 # S = N = 16, the largest S
    _say("summary S=N", F, H, N, D)
    Q, K = _inputs("s_eq_n", F, H, N, D, seed=1)
    sal, _ = sv.summary_salience_prune(Q.to(DEV), K.to(DEV), N, 0)
    sal2, _ = sv.salience_prune(Q.to(DEV), K.to(DEV), 0)
    torch.cuda.synchronize()
    ref = oracle.salience(Q, K)
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), ref)
    assert ok, (rel, sm)
    ok, rel, sm = accept.check_salience(sal2.cpu().numpy(), ref)
    assert ok, (rel, sm)


def test_summary_explicit_scale_workspace_reuse_and_rows_beyond_s_unread():
    F, H, N, D, S = 2, 3, 200, 64, 2
    _say("summary scale / workspace / rows beyond S", F, H, N, D, S)
    Q, K = _inputs("scale_ws", F, H, N, D, seed=2)
    ws = sv.new_workspace(sv.summary_salience_prune_workspace_bytes(F, H, N), DEV)
    a, ia = sv.summary_salience_prune(Q.to(DEV), K.to(DEV), S, 20, 0.3, workspace=ws)
    Q2 = Q.clone()
    Q2[:, :, S:] = 0
    b, ib = sv.summary_salience_prune(Q2.to(DEV), K.to(DEV), S, 20, 0.3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ia, ib)
    ok, rel, sm = accept.check_salience(a.cpu().numpy(), oracle.summary_salience(Q, K, S, scale=0.3))
    assert ok, (rel, sm)


@pytest.mark.parametrize("name,S", [("clip_l14_336_256f", 1), ("radio_1028_64f", 4)])
def test_summary_salience_full_bench_shapes_sampled(name, S):
    """The bench workloads at full size: sampled frames against the oracle, and
    properties of every frame (sums to 1, kept indices ascending and in range)."""
    sw = synthetic.SALIENCE[name]
    _say("summary full size", name, sw.F, sw.H, sw.N, sw.D, S, sw.keep)
    Q, K = synthetic.make_salience(sw, 0, device=DEV, gen_device="cuda")
    sal, idx = sv.summary_salience_prune(Q, K, S, sw.keep)
    torch.cuda.synchronize()
    s_all = sal.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s_all.sum(axis=1) - 1.0) < 1e-5)
    ix = idx.cpu().numpy()
    assert np.all(np.diff(ix, axis=1) > 0) and ix.min() >= 0 and ix.max() < sw.N
    for f in (0, sw.F // 3, sw.F - 1):
        ref = oracle.summary_salience(Q[f:f + 1], K[f:f + 1], S)
        ok, rel, sm = accept.check_salience(s_all[f:f + 1], ref)
        assert ok, (f, rel, sm)
        ok, _, msgs = accept.check_index_sets(ix[f:f + 1], ref, sw.keep)
        assert ok, (f, msgs)
