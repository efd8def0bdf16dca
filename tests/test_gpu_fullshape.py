"""GPU parity at the stated full shapes of the salience and 131k multi-turn
workloads, where the launch shapes differ from the small cases: many
(frame, head) items per persistent salience workgroup, and B x P long-row
select items per decode launch.

Salience (SigLIP-shaped encoder, 256 frames x 729 tokens x 16 heads, D = 72):
sampled frames against the fp64 oracle (1e-4 relative, kept sets with the
tie band), properties of every frame.  Decode (131072-token multi-turn
cache, B = 4, 32 x 128, k = 4096): one sequence's scores, selection and
attention against the oracle (scores computed chunk by chunk over the
tokens in fp64), every sequence against the two-call path.
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


def _check_frames(sal, idx, Q, K, frames, keep, N):
    """Properties of every frame, then the sampled frames against the oracle."""
    s_all = sal.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(s_all.sum(axis=1) - 1.0) < 1e-5)
    ix = idx.cpu().numpy()
    assert np.all(np.diff(ix, axis=1) > 0) and ix.min() >= 0 and ix.max() < N
    for f in frames:
        ref = oracle.salience(Q[f:f + 1].cpu(), K[f:f + 1].cpu())
        ok, rel, sm = accept.check_salience(s_all[f:f + 1], ref)
        assert ok, (f, rel, sm)
        ok, _, msgs = accept.check_index_sets(ix[f:f + 1], ref, keep)
        assert ok, (f, msgs)


def test_salience_full_siglip_256f_sampled():
    """256 frames x 16 heads = 4096 items on at most 256 persistent workgroups
    (16 items each: key re-staging and flag reset per item)."""
    sw = synthetic.SALIENCE["siglip_256f"]
    _say("salience full size", sw)
    Q, K = synthetic.make_salience(sw, 0, device=DEV, gen_device="cuda")
    sal, idx = sv.salience_prune(Q, K, sw.keep)
    torch.cuda.synchronize()
    _check_frames(sal, idx, Q, K, (0, 85, sw.F - 1), sw.keep, sw.N)


def test_salience_late_item_flagged_for_fp32_pass():
    """More items than workgroups, with one late (frame, head) item whose
    logit bound exceeds the fp16 row kernel's: that item is recomputed by the
    fp32 kernel (its skip loop walks past every unflagged item)."""
    sw = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=40)
    _say("salience late flagged item", sw)
    Q, K = synthetic.make_salience(sw, 3, device=DEV, gen_device="cuda")
    f_bad, h_bad = 37, 9                      # item 37 * 16 + 9 = 601 of 640
    Q[f_bad, h_bad] = (Q[f_bad, h_bad].float() * 6.0).to(torch.bfloat16)
    sal, idx = sv.salience_prune(Q, K, sw.keep)
    torch.cuda.synchronize()
    _check_frames(sal, idx, Q, K, (0, 21, f_bad, sw.F - 1), sw.keep, sw.N)


def _log2_bound(Qf, Kf):
    """Largest per-row shift of the fp16 row kernel: |q_i| max_j |k_j| scale log2(e)."""
    q = Qf.float().cpu().numpy().astype(np.float64)
    k = Kf.float().cpu().numpy().astype(np.float64)
    D = q.shape[-1]
    qn = np.linalg.norm(q, axis=-1)            # [H][N]
    kn = np.linalg.norm(k, axis=-1).max(axis=-1, keepdims=True)
    return (qn * kn / np.sqrt(D) * np.log2(np.e)).max()


@pytest.mark.parametrize("shape", ["sink", "diagonal"])
def test_salience_just_below_fp16_bound(shape):
    """Peaked attention just inside the fp16-probability path (row shift below
    7 in log2 units, so probabilities reach down to about 2^-14): a planted
    sink key that most rows attend to, or keys equal to the queries (each row
    attends to itself most)."""
    sw = synthetic.scaled_salience(synthetic.SALIENCE["siglip_256f"], F=4)
    Q, K = synthetic.make_salience(sw, 5)
    Q, K = Q.float(), K.float()
    if shape == "sink":
        # every query gets a common component along u; key 123 points along u
        g = torch.Generator().manual_seed(6)
        u = torch.randn(sw.F, sw.H, 1, sw.D, generator=g)
        u = u / u.norm(dim=-1, keepdim=True)
        Q = (Q + 3.0 * u).to(torch.bfloat16).float()
        for f in range(sw.F):
            for h in range(sw.H):
                qmax = Q[f, h].norm(dim=-1).max()
                c = 6.8 / (qmax * (1.0 / np.sqrt(sw.D)) * np.log2(np.e))
                K[f, h, 123] = (u[f, h, 0] * c).to(torch.bfloat16).float()
    else:
        g = torch.Generator().manual_seed(6)
        K = Q + 0.05 * torch.randn(Q.shape, generator=g)
        # rescale both so that the largest row shift sits just below 7
        for f in range(sw.F):
            for h in range(sw.H):
                b = _log2_bound(Q[f, h].to(torch.bfloat16), K[f, h].to(torch.bfloat16))
                s = (6.8 / b) ** 0.5
                Q[f, h] *= s
                K[f, h] *= s
    Q, K = Q.to(torch.bfloat16), K.to(torch.bfloat16)
    for f in range(sw.F):
        for h in range(sw.H):
            b = _log2_bound(Q[f, h], K[f, h])
            assert 6.0 < b < 6.99, (f, h, b)
    _say("salience near fp16 bound", shape, sw)
    sal, idx = sv.salience_prune(Q.to(DEV), K.to(DEV), sw.keep)
    torch.cuda.synchronize()
    ref = oracle.salience(Q, K)
    if shape == "sink":
        assert (ref[:, 123] > 10.0 / sw.N).all()     # the sink takes a large share
    ok, rel, sm = accept.check_salience(sal.cpu().numpy(), ref)
    assert ok, (rel, sm)
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), ref, sw.keep)
    assert ok, msgs


def _scores_chunked(q, k_vis, chunk=8192):
    """oracle.retrieval_scores over token chunks (each score depends on its own
    token only, so chunking over tokens is exact), with host copies per chunk."""
    N = k_vis.shape[1]
    out = np.empty((k_vis.shape[0], N), dtype=np.float64)
    for t0 in range(0, N, chunk):
        out[:, t0:t0 + chunk] = oracle.retrieval_scores(q, k_vis[:, t0:t0 + chunk].cpu())
    return out


def test_multiturn_full_shape_round_steps():
    """B = 4, 32 x 128 heads, N = 131072, k = 4096 (64 chunks per row: 256
    candidate and 256 compaction items per launch): the first and the last step
    of a round (129 and 256 text entries).  Sequence 0 against the oracle;
    every sequence against sv_retrieve + sv_sparse_decode_attn."""
    w = synthetic.DECODE["multiturn_128k"]
    _say("multiturn full shape", w)
    d = synthetic.make_decode_layer(w, 0, device=DEV, gen_device="cuda")
    ws = sv.new_workspace(sv.retrieve_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.N, w.k,
                                                             w.Tmax), DEV)
    lens = synthetic.multiturn_text_lengths()[0]
    for step in (0, len(lens) - 1):
        T = lens[step]
        _say("multiturn full shape step", step, "T", T)
        q = synthetic.make_fresh_query(w, 0, 0, step, device=DEV, gen_device="cuda")
        tl = torch.full((w.B,), T, dtype=torch.int32, device=DEV)
        out, idx, sc = sv.retrieve_attend(q, d["k_vis"], d["v_vis"], w.k, d["k_txt"], d["v_txt"],
                                          tl, workspace=ws, scores=True)
        idx2, sc2 = sv.retrieve(q, d["k_vis"], w.k, scores=True)
        out2 = sv.sparse_decode_attn(q, d["k_vis"], d["v_vis"], idx2, d["k_txt"], d["v_txt"], tl)
        torch.cuda.synchronize()
        sv.workspace_status(ws)
        assert torch.equal(sc, sc2) and torch.equal(idx, idx2)
        scale = out2.abs().amax(dim=-1, keepdim=True) + 1e-30
        assert ((out - out2).abs() / scale).max().item() < 1e-5
        ix = idx.cpu().numpy()
        assert np.all(np.diff(ix, axis=1) > 0) and ix.min() >= 0 and ix.max() < w.N
        # sequence 0 against the oracle
        q0 = q[0:1].cpu()
        s_ref = _scores_chunked(q0, d["k_vis"][0:1])
        ok, swaps, msgs = accept.check_index_sets(ix[0:1], s_ref, w.k)
        assert ok, msgs[:3]
        rel = np.abs(sc[0].cpu().numpy() - s_ref[0]).max() / np.abs(s_ref[0]).max()
        assert rel < 1e-5, rel
        sel = torch.from_numpy(ix[0]).to(DEV).long()
        kv0 = d["k_vis"][0:1, sel].cpu()               # the selected rows, gathered
        vv0 = d["v_vis"][0:1, sel].cpu()
        ref = oracle.sparse_decode_attn(q0, kv0, vv0, np.arange(w.k)[None], d["k_txt"][0:1].cpu(),
                                        d["v_txt"][0:1].cpu(), np.array([T]))
        ok, err = accept.check_attention(out[0:1].cpu().numpy(), ref)
        assert ok, err
