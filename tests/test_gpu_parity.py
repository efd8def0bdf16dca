"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Inputs come from the seeded generators in ``synthetic``; both sides see the
same stored bits.  Acceptance rules (tests/accept.py): index sets exact up to
swaps inside a 1e-5 relative band at the k-th value, attention within 2e-3
max-abs-relative per (b, h), salience within 1e-4 relative per element and
summing to 1 within 1e-5 per frame.
"""
import math

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


def _to(d, dev=DEV):
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in d.items()}


def _self_consistent(idx, scores, k):
    """The GPU's picks are exactly the top-k of its own fp32 scores (value desc, index asc)."""
    idx = idx.cpu().numpy()
    s = scores.cpu().numpy().astype(np.float64)
    for r in range(s.shape[0]):
        order = np.lexsort((np.arange(s.shape[1]), -s[r]))
        assert sorted(order[:k].tolist()) == idx[r].tolist(), f"row {r}"


# ---------------------------------------------------------------- retrieval
RETRIEVE_CASES = [
    # name, workload, overrides
    ("image576_fp32", "image576_fp32", {}),
    ("image576_fp32_k16", "image576_fp32", dict(k=16)),
    ("llava_b2", "llava_next_7b", dict(B=2)),
    ("qwen2_gqa_n4096", "qwen2_7b_video", dict(N=4096, k=512)),
    ("qwen2_gqa_ragged", "qwen2_7b_video", dict(N=3001, k=333)),
    ("multiturn_n8192", "multiturn_128k", dict(B=2, N=8192, k=256)),
    ("k_zero", "llava_next_7b", dict(B=1, N=77, k=0, planted=0)),
    ("k_one", "llava_next_7b", dict(B=3, N=77, k=1, planted=0)),
    ("k_all", "llava_next_7b", dict(B=1, N=77, k=77, planted=0)),
    ("n_one", "llava_next_7b", dict(B=2, N=1, k=1, planted=0)),
]


@pytest.mark.parametrize("name,wl,ov", RETRIEVE_CASES, ids=[c[0] for c in RETRIEVE_CASES])
def test_retrieve_parity(name, wl, ov):
    w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
    _say("retrieve", name, w)
    d = synthetic.make_decode_layer(w, seed=1)
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    g = _to(d)
    idx, sc = sv.retrieve(g["q"], g["k_vis"], w.k, scores=True)
    torch.cuda.synchronize()
    ok, swaps, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    # scores: fp32 accumulation of exact bf16/fp32 products
    scale = np.abs(s_ref).max(axis=1, keepdims=True) + 1e-30
    err = np.abs(sc.cpu().numpy() - s_ref) / scale
    assert err.max() < 1e-5, err.max()
    _self_consistent(idx, sc, w.k)
    if w.planted and w.k >= w.planted:
        for b in range(w.B):
            assert set(d["planted"][b].tolist()) <= set(idx[b].cpu().tolist())
    if w.k == w.planted and w.planted:
        for b in range(w.B):
            assert set(d["planted"][b].tolist()) == set(idx[b].cpu().tolist())


def test_retrieve_multi_token_query():
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], N=2048, k=100)
    _say("retrieve Tq=3", w)
    d = synthetic.make_decode_layer(w, seed=4)
    q = torch.randn(1, 3, 28, 128, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    s_ref = oracle.retrieval_scores(q, d["k_vis"])
    idx = sv.retrieve(q.to(DEV), d["k_vis"].to(DEV), w.k)
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]


def test_retrieve_strided_cache_and_determinism():
    """A cache view with spare capacity (token stride > row) and bit-identical reruns."""
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=2, N=600, k=150)
    _say("retrieve strided", w)
    d = synthetic.make_decode_layer(w, seed=2)
    big = torch.zeros(2, 700, 40, 128, dtype=torch.bfloat16)
    big[:, :600, :32] = d["k_vis"]
    view = big.to(DEV)[:, :600, :32]          # token stride 40*128, batch stride 700*40*128
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    a = sv.retrieve(d["q"].to(DEV), view, w.k)
    b = sv.retrieve(d["q"].to(DEV), view, w.k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ok, _, msgs = accept.check_index_sets(a.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]


def test_retrieve_ties_go_to_lower_index():
    """Identical key rows give exactly equal scores: the lowest indices must win."""
    B, N, H, D = 2, 300, 4, 64
    g = torch.Generator().manual_seed(21)
    q = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16)
    kv[:, 100:200] = kv[:, 100:101].clone()            # 100 bit-identical rows per sequence
    s_ref = oracle.retrieval_scores(q, kv)
    _say("retrieve ties")
    for b in range(B):
        order = np.lexsort((np.arange(N), -s_ref[b]))
        first = int(np.nonzero(order == 100)[0][0])      # rank of the tied group's first member
        for k in (first + 1, first + 37, first + 100):
            idx = sv.retrieve(q[b:b + 1].to(DEV), kv[b:b + 1].to(DEV), k).cpu().numpy()[0]
            want = np.sort(order[:k])
            assert idx.tolist() == want.tolist(), (b, k)


@pytest.mark.parametrize("mode", ["all_equal", "outlier", "tied_block_300", "two_values"])
def test_retrieve_select_edge_distributions(mode):
    """Score rows that defeat value binning: every score equal, one huge outlier,
    a tied block wider than the candidate limit, two distinct values.  The
    select must stay exact (ties to the lower index) on all of them."""
    B, N, H, D = 2, 1500, 4, 64
    g = torch.Generator().manual_seed(31)
    q = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16)
    if mode == "all_equal":
        kv[:] = kv[:, :1].clone()
    elif mode == "outlier":
        kv[:, 777] = (q[:, 0] * 1000).to(torch.bfloat16)
    elif mode == "tied_block_300":
        kv[:, 400:700] = kv[:, 400:401].clone()
    elif mode == "two_values":
        kv[:, ::2] = kv[:, :1].clone()
        kv[:, 1::2] = kv[:, 1:2].clone()
    s_ref = oracle.retrieval_scores(q, kv)
    _say("retrieve select edge", mode)
    for k in (1, 299, 750, N):
        idx = sv.retrieve(q.to(DEV), kv.to(DEV), k).cpu().numpy()
        for b in range(B):
            order = np.lexsort((np.arange(N), -s_ref[b]))
            # the GPU sums in fp32: compare as index sets with the tie band
            ok, _, msgs = accept.check_index_sets(idx[b:b + 1], s_ref[b:b + 1], k)
            assert ok, (mode, k, b, msgs[:2])
            if mode != "outlier":          # exact ties: the lowest indices must win
                assert idx[b].tolist() == np.sort(order[:k]).tolist(), (mode, k, b)


def test_retrieve_long_rows_multi_token_query():
    """Rows over 2048 tokens take the parallel select; a 3-token query (GQA 28/4)."""
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], N=4100, k=333)
    _say("retrieve long rows Tq=3", w)
    d = synthetic.make_decode_layer(w, seed=5)
    q = torch.randn(1, 3, 28, 128, generator=torch.Generator().manual_seed(19)).to(torch.bfloat16)
    s_ref = oracle.retrieval_scores(q, d["k_vis"])
    idx, sc = sv.retrieve(q.to(DEV), d["k_vis"].to(DEV), w.k, scores=True)
    torch.cuda.synchronize()
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    _self_consistent(idx, sc, w.k)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [(torch.float32, 8, 8, 128), (torch.bfloat16, 16, 2, 64),
                                             (torch.bfloat16, 32, 2, 128)])
def test_retrieve_long_rows_dtypes_and_groups(dtype, Hq, Hkv, D):
    """Long rows through sv_retrieve: fp32 caches, group size 8 (the parallel select) and
    group size 16 (beyond it: the single-workgroup select)."""
    B, N, k = 2, 3000, 400
    g = torch.Generator().manual_seed(53)
    q = torch.randn(B, 1, Hq, D, generator=g).to(dtype)
    kv = torch.randn(B, N, Hkv, D, generator=g).to(dtype)
    s_ref = oracle.retrieval_scores(q, kv)
    _say("retrieve long rows", dtype, Hq, Hkv, D)
    idx, sc = sv.retrieve(q.to(DEV), kv.to(DEV), k, scores=True)
    torch.cuda.synchronize()
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, k)
    assert ok, msgs[:3]
    _self_consistent(idx, sc, k)


@pytest.mark.parametrize("mode", ["all_equal", "outlier", "tied_block_300", "two_values"])
def test_retrieve_long_rows_edge_distributions(mode):
    """The parallel select (rows over 2048 tokens) on rows that send it to its
    fallbacks: one value everywhere, a tied block wider than the ranked bin,
    two values; and one outlier.  One workspace serves every k in turn."""
    B, N, H, D = 2, 5000, 4, 64
    g = torch.Generator().manual_seed(41)
    q = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16)
    if mode == "all_equal":
        kv[:] = kv[:, :1].clone()
    elif mode == "outlier":
        kv[:, 3777] = (q[:, 0] * 1000).to(torch.bfloat16)
    elif mode == "tied_block_300":
        kv[:, 2400:2700] = kv[:, 2400:2401].clone()
    elif mode == "two_values":
        kv[:, ::2] = kv[:, :1].clone()
        kv[:, 1::2] = kv[:, 1:2].clone()
    s_ref = oracle.retrieval_scores(q, kv)
    _say("retrieve long-row select edge", mode)
    qd, kd = q.to(DEV), kv.to(DEV)
    ws = sv.new_workspace(sv.retrieve_workspace_bytes(B, N, N), DEV)
    for k in (1, 777, 2500, N):
        idx = sv.retrieve(qd, kd, k, workspace=ws).cpu().numpy()
        for b in range(B):
            order = np.lexsort((np.arange(N), -s_ref[b]))
            ok, _, msgs = accept.check_index_sets(idx[b:b + 1], s_ref[b:b + 1], k)
            assert ok, (mode, k, b, msgs[:2])
            if mode != "outlier":          # exact ties: the lowest indices must win
                assert idx[b].tolist() == np.sort(order[:k]).tolist(), (mode, k, b)


# ---------------------------------------------------------------- attention
ATTN_CASES = [
    ("image576_fp32", "image576_fp32", {}),
    ("llava_b2", "llava_next_7b", dict(B=2)),
    ("qwen2_gqa7", "qwen2_7b_video", dict(N=4096, k=512, T=100, Tmax=128)),
    ("multiturn", "multiturn_128k", dict(B=2, N=8192, k=1024, T=130, Tmax=256)),
    ("text_only", "llava_next_7b", dict(B=2, N=50, k=0, planted=0)),
    ("visual_only", "llava_next_7b", dict(B=2, N=300, k=40, T=0, Tmax=0, planted=0)),
    ("ragged_small", "qwen2_7b_video", dict(N=37, k=5, T=3, Tmax=9)),
    # bf16 grouped-query heads on matrix cores: 2 and 8 query heads per KV
    # head at D = 64 (up to four 16-entry tiles per wave), 4 at D = 128.
    ("gqa2_d64", "qwen2_7b_video", dict(Hq=8, Hkv=4, D=64, N=700, k=200, T=40, Tmax=48)),
    ("gqa8_d64", "qwen2_7b_video", dict(Hq=32, Hkv=4, D=64, N=3000, k=1000, T=70, Tmax=80)),
    ("gqa4_d128_b3", "qwen2_7b_video", dict(B=3, Hq=16, Hkv=4, N=900, k=250, T=33, Tmax=40)),
]


@pytest.mark.parametrize("name,wl,ov", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_sparse_attn_parity(name, wl, ov):
    w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
    _say("attn", name, w)
    d = synthetic.make_decode_layer(w, seed=3)
    idx = oracle.retrieve(d["q"], d["k_vis"], w.k) if w.k else np.zeros((w.B, 0), np.int64)
    tl = torch.tensor([max(0, w.T - 3 * b) for b in range(w.B)], dtype=torch.int32) if w.Tmax else None
    ref = oracle.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx, d["k_txt"], d["v_txt"],
                                    tl if tl is not None else np.zeros(w.B, np.int64))
    g = _to(d)
    out = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"],
                                torch.from_numpy(idx).to(torch.int32).to(DEV),
                                g["k_txt"] if w.Tmax else None, g["v_txt"] if w.Tmax else None,
                                tl.to(DEV) if tl is not None else None)
    torch.cuda.synchronize()
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err


def test_sparse_attn_k_equals_n_matches_dense():
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], N=700, k=700, T=64, Tmax=64)
    _say("attn k=N", w)
    d = synthetic.make_decode_layer(w, seed=5)
    ref = oracle.dense_decode_attn(d["q"], d["k_vis"], d["v_vis"], d["k_txt"], d["v_txt"], d["txt_len"])
    g = _to(d)
    idx = torch.arange(700, dtype=torch.int32, device=DEV)[None]
    out = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"], idx, g["k_txt"], g["v_txt"], g["txt_len"])
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err


def test_sparse_attn_skips_bad_indices_and_empty_sets():
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=2, N=64, k=4, T=2, Tmax=4, planted=0)
    _say("attn bad idx / empty", w)
    d = synthetic.make_decode_layer(w, seed=6)
    g = _to(d)
    idx = torch.tensor([[3, -1, 70, 10], [-5, 64, 1000, -1]], dtype=torch.int32, device=DEV)
    tl = torch.tensor([2, 0], dtype=torch.int32, device=DEV)
    out = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"], idx, g["k_txt"], g["v_txt"], tl)
    torch.cuda.synchronize()
    ref0 = oracle.sparse_decode_attn(d["q"][:1], d["k_vis"][:1], d["v_vis"][:1], np.array([[3, 10]]),
                                     d["k_txt"][:1], d["v_txt"][:1], np.array([2]))
    ok, err = accept.check_attention(out[:1].cpu().numpy(), ref0)
    assert ok, err
    assert torch.count_nonzero(out[1]) == 0          # sequence 1 attends nothing


def test_decode_step_gpu_indices_end_to_end():
    """retrieve -> sparse attention with the GPU's own indices (config-2 layer shape)."""
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=4)
    _say("decode step e2e", w)
    d = synthetic.make_decode_layer(w, seed=7, layer=5)
    g = _to(d)
    idx = sv.retrieve(g["q"], g["k_vis"], w.k)
    out = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"], idx, g["k_txt"], g["v_txt"], g["txt_len"])
    torch.cuda.synchronize()
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    ref = oracle.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx.cpu().numpy(), d["k_txt"],
                                    d["v_txt"], d["txt_len"])
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err


# ---------------------------------------------------------------- salience
SAL_CASES = [
    ("siglip_4f", "siglip_256f", dict(F=4)),
    ("siglip_narrow_3f", "siglip_256f_narrow", dict(F=3)),
    ("n100_d64", "siglip_256f", dict(F=2, N=100, D=64, H=3, keep=50)),
    ("n17_d32", "siglip_256f", dict(F=2, N=17, D=32, H=2, keep=17)),
    ("n1", "siglip_256f", dict(F=2, N=1, D=72, H=2, keep=1)),
    ("n768_d96", "siglip_256f", dict(F=1, N=768, D=96, H=2, keep=0)),
    ("n300_d8", "siglip_256f", dict(F=2, N=300, D=8, H=1, keep=299)),
]


@pytest.mark.parametrize("name,wl,ov", SAL_CASES, ids=[c[0] for c in SAL_CASES])
def test_salience_parity(name, wl, ov):
    w = synthetic.scaled_salience(synthetic.SALIENCE[wl], **ov)
    _say("salience", name, w)
    Q, K = synthetic.make_salience(w, seed=2)
    s_ref = oracle.salience(Q, K)
    sal, idx = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep)
    torch.cuda.synchronize()
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), s_ref)
    assert ok, (rel, sm)
    ok, swaps, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.keep)
    assert ok, msgs[:3]
    _say("salience", name, "max rel", rel, "sum err", sm, "swaps", swaps)


def test_salience_explicit_scale_and_rerun():
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=2)
    Q, K = synthetic.make_salience(w, seed=3)
    _say("salience scale=0.3")
    s_ref = oracle.salience(Q, K, scale=0.3)
    a, ia = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep, scale=0.3)
    b, ib = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep, scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ia, ib)
    ok, rel, sm = accept.check_salience(a.cpu().numpy(), s_ref)
    assert ok, (rel, sm)


# ---------------------------------------------------------------- workspaces and graphs
def test_workspace_reuse_leaves_counters_zero():
    """One zero-filled workspace serves many calls; the completion counters return to zero."""
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], N=5000, k=300, T=40, Tmax=64)
    _say("workspace reuse", w)
    d = synthetic.make_decode_layer(w, seed=8)
    g = _to(d)
    ws_r = sv.new_workspace(sv.retrieve_workspace_bytes(w.B, w.N, w.k), DEV)
    ws_a = sv.new_workspace(sv.sparse_decode_attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.k, w.Tmax), DEV)
    outs = []
    for _ in range(3):
        idx = sv.retrieve(g["q"], g["k_vis"], w.k, workspace=ws_r)
        out = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"], idx, g["k_txt"], g["v_txt"],
                                    g["txt_len"], workspace=ws_a)
        outs.append((idx.clone(), out.clone()))
    torch.cuda.synchronize()
    for idx, out in outs[1:]:
        assert torch.equal(idx, outs[0][0]) and torch.equal(out, outs[0][1])
    # counters (one 128-byte line each) live after the 256-byte status line and
    # the scores / partials, 256-byte aligned; for these long rows the parallel
    # select's histograms and lists follow them
    n_scores = 256 + ((w.B * w.N * 4 + 255) // 256) * 256
    n_ctr = ((w.B * 128 + 255) // 256) * 256
    assert ws_r.numel() - n_scores >= n_ctr
    assert torch.count_nonzero(ws_r[n_scores:n_scores + n_ctr]) == 0
    assert torch.count_nonzero(ws_r[:256]) == 0        # no wait gave up
    tail = ws_a[-((w.B * w.Hkv * 128 + 255) // 256) * 256:]
    assert torch.count_nonzero(tail) == 0
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    ok, _, msgs = accept.check_index_sets(outs[0][0].cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]


def test_decode_step_graph_replays_match_eager():
    """A captured two-layer decode step, replayed with eager work in between, matches eager runs."""
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=3, L=2)
    _say("graph replay", w)
    layers = [_to(synthetic.make_decode_layer(w, seed=9, layer=l)) for l in range(w.L)]
    ws_r = sv.new_workspace(sv.retrieve_workspace_bytes(w.B, w.N, w.k), DEV)
    ws_a = sv.new_workspace(sv.sparse_decode_attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.k, w.Tmax), DEV)
    idx = [torch.empty((w.B, w.k), dtype=torch.int32, device=DEV) for _ in layers]
    out = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV) for _ in layers]

    def step():
        for l, d in enumerate(layers):
            sv.retrieve(d["q"], d["k_vis"], w.k, workspace=ws_r, out=idx[l])
            sv.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx[l], d["k_txt"], d["v_txt"],
                                  d["txt_len"], workspace=ws_a, out=out[l])

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref_idx = [t.clone() for t in idx]
    ref_out = [t.clone() for t in out]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    for rep in range(4):
        for t in idx + out:
            t.fill_(-7)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(w.L):
            assert torch.equal(idx[l], ref_idx[l]), (rep, l)
            assert torch.equal(out[l], ref_out[l]), (rep, l)
    for l, d in enumerate(layers):
        host = {k: v.cpu() for k, v in d.items()}
        ref = oracle.sparse_decode_attn(host["q"], host["k_vis"], host["v_vis"], ref_idx[l].cpu().numpy(),
                                        host["k_txt"], host["v_txt"], host["txt_len"])
        ok, err = accept.check_attention(ref_out[l].cpu().numpy(), ref)
        assert ok, err


def test_salience_graph_replays_match_eager():
    """A captured salience prune (row kernel, flagged-item pass, mean, top-keep), replayed
    with eager work in between, matches the eager call bit for bit; one item is flagged so
    both kernels write the column sums."""
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=3, H=2)
    Q, K = synthetic.make_salience(w, seed=13)
    Q = Q.float()
    Q[2, 1] *= 12.0
    Q = Q.to(torch.bfloat16)
    _say("salience graph replay")
    Qd, Kd = Q.to(DEV), K.to(DEV)
    ws = sv.new_workspace(sv.salience_prune_workspace_bytes(w.F, w.H, w.N), DEV)
    sal = torch.empty((w.F, w.N), dtype=torch.float32, device=DEV)
    keep = torch.empty((w.F, w.keep), dtype=torch.int32, device=DEV)

    def call():
        sv.salience_prune(Qd, Kd, w.keep, workspace=ws, salience_out=sal, idx_out=keep)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref_sal, ref_keep = sal.clone(), keep.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        call()
    for rep in range(4):
        sal.fill_(-7.0)                       # eager work between replays
        keep.fill_(-7)
        if rep == 2:
            ws.zero_()                        # a cleared workspace replays the same
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sal, ref_sal), rep
        assert torch.equal(keep, ref_keep), rep
    s_ref = oracle.salience(Q, K)
    ok, rel, sm = accept.check_salience(ref_sal.cpu().numpy(), s_ref)
    assert ok, (rel, sm)


@pytest.mark.parametrize("mode", ["all_rows", "some_rows"])
def test_salience_large_logits_use_exact_row_max(mode):
    """Rows whose Cauchy-Schwarz shift could underflow take the exact-max path."""
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=2, H=2)
    Q, K = synthetic.make_salience(w, seed=11)
    Q = Q.float()
    if mode == "all_rows":
        Q *= 12.0
    else:
        Q[:, :, 100:180] *= 12.0            # spans several 16-row blocks
    Q = Q.to(torch.bfloat16)
    K = (K.float() * 4.0).to(torch.bfloat16)
    _say("salience large logits", mode)
    s_ref = oracle.salience(Q, K)
    sal, idx = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep)
    torch.cuda.synchronize()
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), s_ref)
    assert ok, (rel, sm)
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.keep)
    assert ok, msgs[:3]


def test_salience_mixed_items_split_between_kernels():
    """One (frame, head) item with large logits among ordinary ones: the fp16
    row kernel computes the ordinary items and flags the large one for the fp32
    kernel; both write the same column-sum buffer."""
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=3, H=2)
    Q, K = synthetic.make_salience(w, seed=12)
    Q = Q.float()
    Q[1, 0] *= 12.0
    Q = Q.to(torch.bfloat16)
    _say("salience mixed items")
    s_ref = oracle.salience(Q, K)
    for _ in range(2):  # the flags are rewritten by every call
        sal, idx = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep)
        torch.cuda.synchronize()
        ok, rel, sm = accept.check_salience(sal.cpu().numpy(), s_ref)
        assert ok, (rel, sm)
        ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.keep)
        assert ok, msgs[:3]


@pytest.mark.parametrize("D", [64, 72, 80, 96])
@pytest.mark.parametrize("N", [32, 129, 196, 250, 256, 400, 576, 729])
def test_salience_head_dim_grid(D, N):
    """Every head dim of both on-chip kernels (the row kernel takes N in 193..208,
    241..256, 385..400, 561..576 and 721..736), with and without a ragged last tile."""
    w = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=1, H=2, N=N, D=D, keep=N // 2)
    _say("salience grid", N, D)
    Q, K = synthetic.make_salience(w, seed=3)
    s_ref = oracle.salience(Q, K)
    sal, idx = sv.salience_prune(Q.to(DEV), K.to(DEV), w.keep)
    torch.cuda.synchronize()
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), s_ref)
    assert ok, (rel, sm)
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.keep)
    assert ok, msgs[:3]
