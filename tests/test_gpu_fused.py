"""GPU parity of the one-launch decode layer (sv_retrieve_attend).

Against the fp64 oracle: the selected set (index-set rule of tests/accept.py)
and the attention output over the GPU's own selection (2e-3 max-abs-relative
per (b, h)).  Against the two-call path (sv_retrieve then
sv_sparse_decode_attn): identical scores and indices (the same scan and
select arithmetic) and outputs equal up to the summation order of the
attention splits (the fused launch uses finer splits).
"""
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


def _txt_lens(w):
    return torch.tensor([max(0, w.T - 3 * b) for b in range(w.B)], dtype=torch.int32)


FUSED_CASES = [
    # name, workload, overrides
    ("llava_b2", "llava_next_7b", dict(B=2)),
    ("llava_b8_full_layer", "llava_next_7b", {}),
    ("image576_fp32", "image576_fp32", {}),
    ("qwen2_gqa7_n4096", "qwen2_7b_video", dict(N=4096, k=512, T=100, Tmax=128)),
    ("qwen2_gqa7_ragged", "qwen2_7b_video", dict(N=3001, k=333, T=37, Tmax=40)),
    ("multiturn_n8192", "multiturn_128k", dict(B=2, N=8192, k=1024, T=130, Tmax=256)),
    # Long rows at full length: the parallel select over 13 and 64 chunks.
    ("qwen2_full_layer", "qwen2_7b_video", {}),
    ("multiturn_b1_n131072_h8", "multiturn_128k", dict(B=1, Hq=8, Hkv=8, T=130, Tmax=256)),
    ("long_k_equals_n", "qwen2_7b_video", dict(N=4100, k=4100, T=16, Tmax=16)),
    ("long_k_one", "multiturn_128k", dict(B=3, N=2049, k=1, Hq=4, Hkv=4, T=8, Tmax=8)),
    # Long fp32 rows of three chunks, GQA 4: the chunk attention items on the
    # vector front.
    ("fp32_long_rows_gqa4", "image576_fp32", dict(B=2, N=5000, k=700, Hq=16, Hkv=4, T=20,
                                                  Tmax=24, planted=0)),
    ("visual_only", "llava_next_7b", dict(B=2, N=300, k=40, T=0, Tmax=0, planted=0)),
    ("k_one", "llava_next_7b", dict(B=3, N=77, k=1, T=5, Tmax=8, planted=0)),
    ("n_one", "llava_next_7b", dict(B=2, N=1, k=1, T=4, Tmax=4, planted=0)),
    ("hkv28_rows448", "llava_next_7b", dict(B=2, N=500, k=64, Hq=28, Hkv=28, planted=0)),
    ("hkv25_d64_ragged", "llava_next_7b", dict(B=2, N=300, k=50, Hq=25, Hkv=25, D=64, T=20,
                                               Tmax=24, planted=0)),
    ("hkv25_d64_fp32", "image576_fp32", dict(N=200, k=20, Hq=25, Hkv=25, D=64, planted=0)),
    ("fp32_rows_two_segments", "image576_fp32", dict(N=130, k=30, T=10, Tmax=12, planted=0)),
    ("bf16_rows_two_segments", "llava_next_7b", dict(B=2, N=130, k=30, Hq=64, Hkv=64, T=10,
                                                     Tmax=12, planted=0)),
    # Matrix-core attention items in both row modes, D = 64.
    ("gqa8_d64_short_rows", "qwen2_7b_video", dict(B=2, Hq=32, Hkv=4, D=64, N=1500, k=300, T=50,
                                                   Tmax=64)),
    ("gqa2_d64_long_rows", "qwen2_7b_video", dict(Hq=4, Hkv=2, D=64, N=5000, k=700, T=20,
                                                  Tmax=24)),
]


@pytest.mark.parametrize("name,wl,ov", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_retrieve_attend_parity(name, wl, ov):
    w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
    _say("retrieve_attend", name, w)
    d = synthetic.make_decode_layer(w, seed=11)
    tl = _txt_lens(w)
    g = _to(d)
    out, idx, sc = sv.retrieve_attend(g["q"], g["k_vis"], g["v_vis"], w.k,
                                      g["k_txt"] if w.Tmax else None,
                                      g["v_txt"] if w.Tmax else None,
                                      tl.to(DEV) if w.Tmax else None, scores=True)
    torch.cuda.synchronize()
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    scale = np.abs(s_ref).max(axis=1, keepdims=True) + 1e-30
    assert (np.abs(sc.cpu().numpy() - s_ref) / scale).max() < 1e-5
    ref = oracle.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx.cpu().numpy(), d["k_txt"],
                                    d["v_txt"], tl.numpy() if w.Tmax else np.zeros(w.B, np.int64))
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err
    if w.planted and w.k >= w.planted:
        for b in range(w.B):
            assert set(d["planted"][b].tolist()) <= set(idx[b].cpu().tolist())

    # The two-call path: the same scores and selection, the same attention up
    # to the order of the split merge.
    idx2, sc2 = sv.retrieve(g["q"], g["k_vis"], w.k, scores=True)
    out2 = sv.sparse_decode_attn(g["q"], g["k_vis"], g["v_vis"], idx2,
                                 g["k_txt"] if w.Tmax else None, g["v_txt"] if w.Tmax else None,
                                 tl.to(DEV) if w.Tmax else None)
    torch.cuda.synchronize()
    assert torch.equal(sc, sc2)
    assert torch.equal(idx, idx2)
    scale = out2.abs().amax(dim=-1, keepdim=True) + 1e-30
    assert ((out - out2).abs() / scale).max().item() < 1e-5


def test_retrieve_attend_strided_caches():
    """Cache views with spare capacity (token stride > row, batch stride > N rows)."""
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=2, N=600, k=150, T=30, Tmax=40)
    _say("retrieve_attend strided", w)
    d = synthetic.make_decode_layer(w, seed=12)

    def pad(t, rows):
        big = torch.zeros(t.shape[0], rows, 40, t.shape[3], dtype=t.dtype)
        big[:, :t.shape[1], :t.shape[2]] = t
        return big.to(DEV)[:, :t.shape[1], :t.shape[2]]

    kv, vv = pad(d["k_vis"], 700), pad(d["v_vis"], 700)
    kt, vt = pad(d["k_txt"], 50), pad(d["v_txt"], 50)
    tl = d["txt_len"].to(DEV)
    out, idx = sv.retrieve_attend(d["q"].to(DEV), kv, vv, w.k, kt, vt, tl)
    torch.cuda.synchronize()
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    ref = oracle.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx.cpu().numpy(), d["k_txt"],
                                    d["v_txt"], d["txt_len"])
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err


def test_retrieve_attend_k_equals_n_matches_dense():
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], N=700, k=700, T=64, Tmax=64)
    _say("retrieve_attend k=N", w)
    d = synthetic.make_decode_layer(w, seed=13)
    g = _to(d)
    out, idx = sv.retrieve_attend(g["q"], g["k_vis"], g["v_vis"], w.k, g["k_txt"], g["v_txt"],
                                  g["txt_len"])
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [list(range(700))]
    ref = oracle.dense_decode_attn(d["q"], d["k_vis"], d["v_vis"], d["k_txt"], d["v_txt"],
                                   d["txt_len"])
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err


def test_retrieve_attend_workspace_reuse_and_graph_replay():
    """One zero-filled workspace across eager calls and graph replays of a two-layer step;
    every call leaves the control block zero and gives identical results."""
    w = synthetic.scaled_decode(synthetic.DECODE["llava_next_7b"], B=3, L=2, T=40, Tmax=64)
    _say("retrieve_attend reuse + graph", w)
    layers = [_to(synthetic.make_decode_layer(w, seed=14, layer=l)) for l in range(w.L)]
    nbytes = sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k, w.Tmax)
    ws = sv.new_workspace(nbytes, DEV)
    idx = [torch.empty((w.B, w.k), dtype=torch.int32, device=DEV) for _ in layers]
    out = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV) for _ in layers]

    def step():
        for l, d in enumerate(layers):
            sv.retrieve_attend(d["q"], d["k_vis"], d["v_vis"], w.k, d["k_txt"], d["v_txt"],
                               d["txt_len"], workspace=ws, out=out[l], idx_out=idx[l])

    # The tail of the workspace: control words (one 128-byte line each), then
    # the encoded index copy (B*k words), both zero between launches.
    ctl_bytes = (w.B * (3 + w.Hkv) * 128 + 255) // 256 * 256 + _al256(w.B * w.k * 4)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[-ctl_bytes:]) == 0
    ref_idx = [t.clone() for t in idx]
    ref_out = [t.clone() for t in out]
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    for l in range(w.L):
        assert torch.equal(idx[l], ref_idx[l]) and torch.equal(out[l], ref_out[l])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    for rep in range(4):
        for t in idx + out:
            t.fill_(-7)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[-ctl_bytes:]) == 0, rep
        for l in range(w.L):
            assert torch.equal(idx[l], ref_idx[l]), (rep, l)
            assert torch.equal(out[l], ref_out[l]), (rep, l)
    for l, d in enumerate(layers):
        host = {k: v.cpu() for k, v in d.items()}
        s_ref = oracle.retrieval_scores(host["q"], host["k_vis"])
        ok, _, msgs = accept.check_index_sets(ref_idx[l].cpu().numpy(), s_ref, w.k)
        assert ok, msgs[:3]
        ref = oracle.sparse_decode_attn(host["q"], host["k_vis"], host["v_vis"],
                                        ref_idx[l].cpu().numpy(), host["k_txt"], host["v_txt"],
                                        host["txt_len"])
        ok, err = accept.check_attention(ref_out[l].cpu().numpy(), ref)
        assert ok, err


# ---------------------------------------------------------------- long rows
LONG_EDGE = [
    # mode, N, ks.  all_equal at N > 16384 overflows the candidate list and
    # two_values the final bin: both take the whole-row fallback.  tied_top_100
    # puts the k-th key inside a block of 100 equal top scores (ranked by index
    # in the threshold item); tied_block_3000 spans chunk boundaries.
    ("gaussian", 20000, (1, 2047, 2048, 9999, 20000)),
    ("all_equal", 20000, (1, 5000, 20000)),
    ("two_values", 6000, (1, 2999, 3000, 3001, 6000)),
    ("tied_top_100", 9000, (1, 50, 99, 100, 101)),
    ("tied_block_3000", 9000, (100, 4000, 8000)),
    ("outlier", 9000, (1, 2, 4500)),
]


@pytest.mark.parametrize("mode,N,ks", LONG_EDGE, ids=[c[0] for c in LONG_EDGE])
def test_retrieve_attend_long_row_edges(mode, N, ks):
    """Exact selection on long rows whatever the score distribution: ties go to
    the lower index, both fallbacks agree with the single-workgroup select."""
    B, H, D = 2, 4, 64
    g = torch.Generator().manual_seed(41)
    q = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16)
    vv = torch.randn(B, N, H, D, generator=g).to(torch.bfloat16)
    if mode == "all_equal":
        kv[:] = kv[:, :1].clone()
    elif mode == "two_values":
        kv[:, ::2] = kv[:, :1].clone()
        kv[:, 1::2] = kv[:, 1:2].clone()
    elif mode == "tied_top_100":
        kv[:, 4000:4100] = (q[:, 0] * 4).unsqueeze(1).to(torch.bfloat16)
    elif mode == "tied_block_3000":
        kv[:, 1500:4500] = kv[:, 1500:1501].clone()
    elif mode == "outlier":
        kv[:, 7777] = (q[:, 0] * 1000).to(torch.bfloat16)
    s_ref = oracle.retrieval_scores(q, kv)
    gq, gk, gv = q.to(DEV), kv.to(DEV), vv.to(DEV)
    for k in ks:
        _say("retrieve_attend long edge", mode, "N", N, "k", k)
        out, idx = sv.retrieve_attend(gq, gk, gv, k, None, None, None)
        idx2 = sv.retrieve(gq, gk, k)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2), (mode, k)
        h = idx.cpu().numpy()
        ok, _, msgs = accept.check_index_sets(h, s_ref, k)
        assert ok, (mode, k, msgs[:2])
        if mode != "outlier" and mode != "gaussian":   # exact ties: the lowest indices win
            for b in range(B):
                order = np.lexsort((np.arange(N), -s_ref[b]))
                assert h[b].tolist() == np.sort(order[:k]).tolist(), (mode, k, b)
        kt0 = torch.zeros(B, 0, H, D, dtype=torch.bfloat16)
        ref = oracle.sparse_decode_attn(q, kv, vv, h, kt0, kt0, np.zeros(B, np.int64))
        ok, err = accept.check_attention(out.cpu().numpy(), ref)
        assert ok, (mode, k, err)


def _al256(n):
    return (n + 255) // 256 * 256


def _long_zero_span(B, N, total):
    """Byte range of the long-row control lines and histograms (zero between
    launches): the tail of the workspace is [control lines 6 per sequence]
    [scan count lines 16 per sequence][hist1 8 x 2048 words][hist2 2048 words]
    [candidates 16384 x 8 bytes][two arrays of ceil(N / 2048) words], each part
    256-byte aligned."""
    P = (N + 2047) // 2048
    zero = (_al256(B * 6 * 128) + _al256(B * 16 * 128) + _al256(B * 8 * 2048 * 4) +
            _al256(B * 2048 * 4))
    long_total = zero + _al256(B * 16384 * 8) + 2 * _al256(B * P * 4)
    start = total - long_total
    return start, start + zero


def test_retrieve_attend_long_rows_reuse_and_graph_replay():
    """Long rows: the control lines, counters and histograms are zero after every
    launch, and graph replays reproduce the eager results."""
    w = synthetic.scaled_decode(synthetic.DECODE["qwen2_7b_video"], B=2, L=2, N=6000, k=700,
                                T=40, Tmax=64)
    _say("retrieve_attend long reuse + graph", w)
    layers = [_to(synthetic.make_decode_layer(w, seed=15, layer=l)) for l in range(w.L)]
    nbytes = sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k, w.Tmax)
    ws = sv.new_workspace(nbytes, DEV)
    z0, z1 = _long_zero_span(w.B, w.N, nbytes)
    ctl_bytes = (w.B * (3 + w.Hkv) * 128 + 255) // 256 * 256 + _al256(w.B * w.k * 4)
    idx = [torch.empty((w.B, w.k), dtype=torch.int32, device=DEV) for _ in layers]
    out = [torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=DEV) for _ in layers]

    def step():
        for l, d in enumerate(layers):
            sv.retrieve_attend(d["q"], d["k_vis"], d["v_vis"], w.k, d["k_txt"], d["v_txt"],
                               d["txt_len"], workspace=ws, out=out[l], idx_out=idx[l])

    def zero_ok():
        return (torch.count_nonzero(ws[z0:z1]) == 0 and
                torch.count_nonzero(ws[z0 - ctl_bytes:z0]) == 0)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    assert zero_ok()
    ref_idx = [t.clone() for t in idx]
    ref_out = [t.clone() for t in out]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    for rep in range(4):
        for t in idx + out:
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert zero_ok(), rep
        for l in range(w.L):
            assert torch.equal(idx[l], ref_idx[l]), (rep, l)
            assert torch.equal(out[l], ref_out[l]), (rep, l)
    for l, d in enumerate(layers):
        host = {k: v.cpu() for k, v in d.items()}
        s_ref = oracle.retrieval_scores(host["q"], host["k_vis"])
        ok, _, msgs = accept.check_index_sets(ref_idx[l].cpu().numpy(), s_ref, w.k)
        assert ok, msgs[:3]
        ref = oracle.sparse_decode_attn(host["q"], host["k_vis"], host["v_vis"],
                                        ref_idx[l].cpu().numpy(), host["k_txt"], host["v_txt"],
                                        host["txt_len"])
        ok, err = accept.check_attention(ref_out[l].cpu().numpy(), ref)
        assert ok, err


def test_multiturn_rounds_reuse_the_visual_cache():
    """Rounds of decode steps over one visual cache (the multi-turn reuse): every step a
    fresh query and a text length that grows by one, then partial eviction back to the
    system entries between rounds.  One workspace serves every step; each step matches
    the oracle and the visual cache is bit-identical afterwards."""
    w = synthetic.scaled_decode(synthetic.DECODE["multiturn_128k"], B=2, N=4100, k=300, T=24,
                                Tmax=24)
    sched = synthetic.multiturn_text_lengths(rounds=2, steps=4, system=8, question=8)
    assert sched == [[17, 18, 19, 20], [17, 18, 19, 20]]
    _say("multiturn rounds", w, sched)
    d = synthetic.make_decode_layer(w, seed=14)
    g = _to(d)
    before = [g[n].clone() for n in ("k_vis", "v_vis", "k_txt", "v_txt")]
    ws = sv.new_workspace(sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k,
                                                             w.Tmax), DEV)
    gen = torch.Generator().manual_seed(15)
    for r, lens in enumerate(sched):
        for t, T in enumerate(lens):
            q = torch.randn(w.B, 1, w.Hq, w.D, generator=gen).to(w.dtype)
            tl = torch.full((w.B,), T, dtype=torch.int32)
            out, idx = sv.retrieve_attend(q.to(DEV), g["k_vis"], g["v_vis"], w.k, g["k_txt"],
                                          g["v_txt"], tl.to(DEV), workspace=ws)
            torch.cuda.synchronize()
            s_ref = oracle.retrieval_scores(q, d["k_vis"])
            ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
            assert ok, (r, t, msgs[:2])
            ref = oracle.sparse_decode_attn(q, d["k_vis"], d["v_vis"], idx.cpu().numpy(),
                                            d["k_txt"], d["v_txt"], tl.numpy())
            ok, err = accept.check_attention(out.cpu().numpy(), ref)
            assert ok, (r, t, err)
    for a_, n in zip(before, ("k_vis", "v_vis", "k_txt", "v_txt")):
        assert torch.equal(a_, g[n]), n


@pytest.mark.parametrize("wl,ov", [("llava_next_7b", dict(B=4)), ("qwen2_7b_video", {})],
                         ids=["short_rows", "long_rows"])
def test_wait_give_up_is_reported_and_every_kernel_finishes(wl, ov):
    """The host lowers the bound of the in-kernel waits to one poll, so waits give
    up (a select before its scores are complete, attention items before their
    indices, long-row items before their counters): every kernel still runs to
    completion, and the workspace's status word reports it.  With the default
    bound and a fresh workspace, the same layer matches the oracle and reports
    nothing."""
    w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
    _say("wait give-up", wl, w)
    d = synthetic.make_decode_layer(w, seed=21)
    g = _to(d)
    nbytes = sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k, w.Tmax)
    reported = 0
    prev = sv.set_wait_limit(1)
    try:
        for _ in range(3):
            ws = sv.new_workspace(nbytes, DEV)
            sv.retrieve_attend(g["q"], g["k_vis"], g["v_vis"], w.k, g["k_txt"], g["v_txt"],
                               g["txt_len"], workspace=ws)
            torch.cuda.synchronize()        # every kernel has finished
            try:
                sv.workspace_status(ws)
            except sv.SvError as e:
                assert e.status == 4 and "gave up" in str(e)
                reported += 1
    finally:
        sv.set_wait_limit(prev)
    assert reported > 0
    ws = sv.new_workspace(nbytes, DEV)
    out, idx = sv.retrieve_attend(g["q"], g["k_vis"], g["v_vis"], w.k, g["k_txt"], g["v_txt"],
                                  g["txt_len"], workspace=ws)
    torch.cuda.synchronize()
    sv.workspace_status(ws)
    s_ref = oracle.retrieval_scores(d["q"], d["k_vis"])
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, w.k)
    assert ok, msgs[:3]
    ref = oracle.sparse_decode_attn(d["q"], d["k_vis"], d["v_vis"], idx.cpu().numpy(), d["k_txt"],
                                    d["v_txt"], d["txt_len"])
    ok, err = accept.check_attention(out.cpu().numpy(), ref)
    assert ok, err
