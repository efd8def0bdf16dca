"""GPU parity of dense packing (sv_pack_selected) against the fp64 CPU oracle.

Packing moves bits, so the rule is exact equality with the oracle's gather,
element by element, on every case (zero rows for indices outside [0, N)).
The per-question flow -- retrieval over the question's tokens, one pack,
then decode steps over the packed rows plus the text entries -- is checked
against the oracle's sparse attention over the unpacked cache (2e-3
max-abs-relative per (b, h), as for the unpacked attention).
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


def _f64(t):
    return oracle.to_f64(t)


def _check_pack(kc, vc, idx):
    """Pack on the GPU and compare every element with the oracle."""
    kp, vp = sv.pack_selected(kc, vc, idx)
    torch.cuda.synchronize()
    want_k, want_v = oracle.pack_selected(kc, vc, idx)
    assert kp.dtype == kc.dtype and kp.shape == want_k.shape
    assert np.array_equal(_f64(kp), want_k)
    assert np.array_equal(_f64(vp), want_v)
    return kp, vp


def _cache(shape, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(synthetic.stream_seed(seed, "pack", *shape))
    return torch.randn(shape, generator=g, device=DEV).to(dtype)


CASES = [
    # name, B, N, Hkv, D, k, dtype
    ("llava_full_bf16", 8, 1440, 32, 128, 360, torch.bfloat16),
    ("qwen2_gqa_bf16", 2, 3001, 4, 128, 333, torch.bfloat16),
    ("qwen2_video_full_bf16", 1, 25088, 4, 128, 2048, torch.bfloat16),
    ("multiturn_scaled_bf16", 2, 8192, 32, 128, 256, torch.bfloat16),
    ("ragged_fp32", 3, 77, 2, 64, 33, torch.float32),
    ("tiny_rows_bf16", 5, 9, 1, 8, 7, torch.bfloat16),
    ("long_rows_fp32", 2, 50, 80, 128, 17, torch.float32),   # rows of 40 KB: sliced units
    ("k_one", 3, 10, 4, 64, 1, torch.bfloat16),
]


@pytest.mark.parametrize("name,B,N,Hkv,D,k,dt", CASES, ids=[c[0] for c in CASES])
def test_pack_bit_exact(name, B, N, Hkv, D, k, dt):
    _say("pack", name, B, N, Hkv, D, k, dt)
    kc, vc = _cache((B, N, Hkv, D), dt, 1), _cache((B, N, Hkv, D), dt, 2)
    g = torch.Generator().manual_seed(synthetic.stream_seed(3, "pack_idx", name))
    idx = torch.stack([torch.randperm(N, generator=g)[:k].sort().values for _ in range(B)])
    _check_pack(kc, vc, idx.to(torch.int32).to(DEV))


def test_pack_strided_cache_bad_and_repeated_indices():
    B, N, Hkv, D = 3, 40, 4, 64
    _say("pack strided / bad idx", B, N, Hkv, D)
    # token stride > row (head-padded rows) and batch stride > N rows
    big_k = _cache((B, N + 6, Hkv + 1, D), torch.bfloat16, 4)
    big_v = _cache((B, N + 6, Hkv + 1, D), torch.bfloat16, 5)
    kc, vc = big_k[:, :N, :Hkv], big_v[:, :N, :Hkv]
    idx = torch.tensor([[0, 39, 39, 5, -1, 40],
                        [2147483647, 7, 7, 7, 0, 1],
                        [-2147483648, 38, 12, 13, 14, 40]], dtype=torch.int32, device=DEV)
    kp, vp = _check_pack(kc, vc, idx)
    assert torch.count_nonzero(kp[0, 4]) == 0 and torch.count_nonzero(vp[2, 5]) == 0


def test_pack_into_given_buffers_overwrites_them():
    B, N, Hkv, D, k = 2, 30, 2, 64, 11
    _say("pack out=", B, N, Hkv, D, k)
    kc, vc = _cache((B, N, Hkv, D), torch.float32, 6), _cache((B, N, Hkv, D), torch.float32, 7)
    kp = torch.full((B, k, Hkv, D), float("nan"), device=DEV)
    vp = torch.full((B, k, Hkv, D), float("nan"), device=DEV)
    idx = torch.tensor([list(range(0, 22, 2)), list(range(29, 18, -1))], dtype=torch.int32,
                       device=DEV)
    sv.pack_selected(kc, vc, idx, out=(kp, vp))
    torch.cuda.synchronize()
    want_k, want_v = oracle.pack_selected(kc, vc, idx)
    assert np.array_equal(_f64(kp), want_k) and np.array_equal(_f64(vp), want_v)


@pytest.mark.parametrize("wl,ov", [
    ("llava_next_7b", dict(B=2)),
    ("qwen2_7b_video", dict(N=2000, k=250)),
], ids=["llava_b2", "qwen2_gqa"])
def test_question_retrieve_pack_then_decode_steps(wl, ov):
    """Retrieve once for a question of 8 tokens, pack, then attend packed + text per step."""
    w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
    _say("per-question flow", wl, w)
    d = synthetic.make_decode_layer(w, seed=8)
    gq = torch.Generator().manual_seed(synthetic.stream_seed(8, "question", wl))
    question = torch.randn((w.B, 8, w.Hq, w.D), generator=gq).to(w.dtype)
    g = {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in d.items()}
    idx = sv.retrieve(question.to(DEV), g["k_vis"], w.k)
    kp, vp = sv.pack_selected(g["k_vis"], g["v_vis"], idx)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy().astype(np.int64)
    want_k, want_v = oracle.pack_selected(d["k_vis"], d["v_vis"], idx_np)
    assert np.array_equal(_f64(kp), want_k) and np.array_equal(_f64(vp), want_v)
    ok, _, msgs = accept.check_index_sets(idx_np, oracle.retrieval_scores(question, d["k_vis"]), w.k)
    assert ok, msgs
    ar = torch.arange(w.k, dtype=torch.int32, device=DEV).expand(w.B, w.k).contiguous()
    for step in range(3):
        q = torch.randn((w.B, w.Hq, w.D), generator=gq).to(w.dtype)
        tl = torch.tensor([w.T - step - b for b in range(w.B)], dtype=torch.int32)
        out_p = sv.sparse_decode_attn(q.to(DEV), kp, vp, ar, g["k_txt"], g["v_txt"], tl.to(DEV))
        # No index list: the packed rows 0..k-1 themselves, the same entries in
        # the same order, so the same bits.
        out_r = sv.sparse_decode_attn(q.to(DEV), kp, vp, w.k, g["k_txt"], g["v_txt"], tl.to(DEV))
        out_s = sv.sparse_decode_attn(q.to(DEV), g["k_vis"], g["v_vis"], idx, g["k_txt"], g["v_txt"],
                                      tl.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(out_r, out_p), step
        ref = oracle.sparse_decode_attn(q, d["k_vis"], d["v_vis"], idx_np, d["k_txt"], d["v_txt"], tl)
        ok, err = accept.check_attention(out_p.cpu().numpy(), ref)
        assert ok, (step, err)
        ok, err = accept.check_attention(out_s.cpu().numpy(), ref)
        assert ok, (step, err)


def test_pack_graph_replays_match_oracle():
    """A captured pack, replayed with new index lists written between replays."""
    B, N, Hkv, D, k = 4, 300, 8, 128, 45
    _say("pack graph replays", B, N, Hkv, D, k)
    kc, vc = _cache((B, N, Hkv, D), torch.bfloat16, 9), _cache((B, N, Hkv, D), torch.bfloat16, 10)
    idx = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    kp = torch.empty((B, k, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sv.pack_selected(kc, vc, idx, out=(kp, vp))       # warm-up before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            sv.pack_selected(kc, vc, idx, out=(kp, vp))
    g = torch.Generator().manual_seed(synthetic.stream_seed(11, "pack_graph"))
    for rep in range(4):
        new = torch.stack([torch.randperm(N, generator=g)[:k].sort().values for _ in range(B)])
        idx.copy_(new.to(torch.int32).to(DEV))
        kp.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want_k, want_v = oracle.pack_selected(kc, vc, new.numpy())
        assert np.array_equal(_f64(kp), want_k), rep
        assert np.array_equal(_f64(vp), want_v), rep
