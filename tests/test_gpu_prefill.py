"""GPU parity of sv_prefill_attend_retrieve (causal prefill attention of a
question chunk with the query-aware retrieval fused into it) against the fp64
oracle: attention within 2e-3 max-abs-relative per (sequence, token, head),
retrieval scores within 1e-5 of the largest score, selected sets exact up to
swaps inside the 1e-5 relative band.
"""
import numpy as np
import pytest
import torch

import accept
import oracle
import visual_token_sparsity_amd as sv

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)  # noqa: E731
    return r(B, Tq, Hq, D), r(B, N, Hkv, D), r(B, N, Hkv, D), r(B, Tmax, Hkv, D), r(B, Tmax, Hkv, D)


CASES = [
    # name, B, Tq, Hq, Hkv, D, N, Tmax, txt_len, k
    ("llava_like_question", 2, 32, 32, 32, 128, 1440, 256, [256, 100], 360),
    ("gqa7_rows112", 1, 16, 28, 4, 128, 4096, 200, [200], 512),
    ("gqa7_rows280_three_chunks", 1, 40, 28, 4, 128, 2100, 120, [120], 300),
    ("d64_ragged_short_text", 2, 8, 8, 2, 64, 333, 50, [50, 5], 40),
    ("rows48_two_waves", 2, 6, 16, 2, 64, 777, 64, [64, 31], 100),
    ("one_token", 3, 1, 8, 8, 128, 500, 40, [40, 1, 0], 64),
    ("long_rows_select", 1, 4, 8, 8, 128, 5000, 16, [16], 700),
    ("k_equals_n", 1, 3, 4, 4, 64, 90, 10, [10], 90),
    # 192 (sequence, KV head) items: one key split each, normalised output
    # written by the attention items themselves (no combine).
    ("one_split_direct_output", 6, 4, 32, 32, 128, 300, 40, [40, 33, 4, 40, 0, 17], 100),
]


@pytest.mark.parametrize("name,B,Tq,Hq,Hkv,D,N,Tmax,tl,k", CASES, ids=[c[0] for c in CASES])
def test_prefill_attend_retrieve_parity(name, B, Tq, Hq, Hkv, D, N, Tmax, tl, k):
    _say("prefill", name, B, Tq, Hq, Hkv, D, N, Tmax, tl, k)
    q, kv, vv, kt, vt = _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=N + Tq)
    txt = torch.tensor(tl, dtype=torch.int32)
    out, idx, sc = sv.prefill_attend_retrieve(q.to(DEV), kv.to(DEV), vv.to(DEV), kt.to(DEV),
                                              vt.to(DEV), txt.to(DEV), k, scores=True)
    torch.cuda.synchronize()
    ref = oracle.prefill_attention(q, kv, vv, kt, vt, txt.numpy())
    ok, err = accept.check_attention(out.cpu().numpy().reshape(B * Tq, Hq, D),
                                     ref.reshape(B * Tq, Hq, D))
    assert ok, err
    s_ref = oracle.retrieval_scores(q, kv)
    scale = np.abs(s_ref).max(axis=1, keepdims=True)
    assert (np.abs(sc.cpu().numpy() - s_ref) / scale).max() < 1e-5
    ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), s_ref, k)
    assert ok, msgs[:3]


def test_prefill_visual_only_and_no_selection():
    B, Tq, Hq, Hkv, D, N = 2, 5, 8, 4, 128, 300
    _say("prefill visual only", B, Tq, Hq, Hkv, D, N)
    q, kv, vv, _, _ = _inputs(B, Tq, Hq, Hkv, D, N, 1, seed=3)
    out, _ = sv.prefill_attend_retrieve(q.to(DEV), kv.to(DEV), vv.to(DEV), None, None, None, 0)
    torch.cuda.synchronize()
    empty = torch.zeros(B, 0, Hkv, D, dtype=torch.bfloat16)
    ref = oracle.prefill_attention(q, kv, vv, empty, empty, np.zeros(B, np.int64))
    ok, err = accept.check_attention(out.cpu().numpy().reshape(B * Tq, Hq, D),
                                     ref.reshape(B * Tq, Hq, D))
    assert ok, err


def test_prefill_last_token_matches_decode_path_and_retrieve():
    """The question's last token attends everything: the same output as the
    decode attention with k = N; its retrieval equals sv_retrieve over the
    whole question (identical selection)."""
    B, Tq, Hq, Hkv, D, N, Tmax = 2, 12, 16, 4, 128, 900, 80
    _say("prefill vs decode path", B, Tq, Hq, Hkv, D, N, Tmax)
    q, kv, vv, kt, vt = _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=4)
    g = [t.to(DEV) for t in (q, kv, vv, kt, vt)]
    txt = torch.tensor([80, 50], dtype=torch.int32, device=DEV)
    out, idx = sv.prefill_attend_retrieve(*g, txt, 200)
    all_idx = torch.arange(N, dtype=torch.int32, device=DEV).expand(B, N).contiguous()
    dec = sv.sparse_decode_attn(g[0][:, -1].contiguous(), g[1], g[2], all_idx, g[3], g[4], txt)
    idx2 = sv.retrieve(g[0], g[1], 200)
    torch.cuda.synchronize()
    ok, err = accept.check_attention(out[:, -1].cpu().numpy(), dec.cpu().numpy().astype(np.float64))
    assert ok, err
    assert torch.equal(idx, idx2) or accept.check_index_sets(
        idx.cpu().numpy(), oracle.retrieval_scores(q, kv), 200)[0]


def test_prefill_strided_caches_and_workspace_reuse():
    B, Tq, Hq, Hkv, D, N, Tmax = 2, 9, 8, 2, 64, 400, 30
    _say("prefill strided + reuse", B, Tq, Hq, Hkv, D, N, Tmax)
    q, kv, vv, kt, vt = _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=5)

    def pad(t, rows):
        big = torch.zeros(t.shape[0], rows, 3, t.shape[3], dtype=t.dtype)
        big[:, :t.shape[1], :t.shape[2]] = t
        return big.to(DEV)[:, :t.shape[1], :t.shape[2]]

    txt = torch.tensor([30, 12], dtype=torch.int32)
    ws = sv.new_workspace(sv.prefill_attend_retrieve_workspace_bytes(B, Tq, Hq, Hkv, D, N, Tmax), DEV)
    a = sv.prefill_attend_retrieve(q.to(DEV), pad(kv, 420), pad(vv, 420), pad(kt, 40), pad(vt, 40),
                                   txt.to(DEV), 50, workspace=ws)
    b = sv.prefill_attend_retrieve(q.to(DEV), pad(kv, 420), pad(vv, 420), pad(kt, 40), pad(vt, 40),
                                   txt.to(DEV), 50, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ref = oracle.prefill_attention(q, kv, vv, kt, vt, txt.numpy())
    ok, err = accept.check_attention(a[0].cpu().numpy().reshape(B * Tq, Hq, D),
                                     ref.reshape(B * Tq, Hq, D))
    assert ok, err


def test_prefill_long_rows_workspace_reuse_new_inputs():
    """Rows over 2048 tokens take the parallel select, whose control words the
    call leaves at zero: a second call on the same workspace with other inputs
    selects its own top-k (stale threshold words would select the first
    call's)."""
    B, Tq, Hq, Hkv, D, N, Tmax, k = 1, 4, 8, 8, 128, 5000, 16, 700
    _say("prefill long rows, workspace reuse", B, Tq, Hq, Hkv, D, N, Tmax, k)
    ws = sv.new_workspace(sv.prefill_attend_retrieve_workspace_bytes(B, Tq, Hq, Hkv, D, N, Tmax), DEV)
    txt = torch.tensor([16], dtype=torch.int32)
    for seed in (11, 12, 13):
        q, kv, vv, kt, vt = _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=seed)
        _, idx = sv.prefill_attend_retrieve(q.to(DEV), kv.to(DEV), vv.to(DEV), kt.to(DEV),
                                            vt.to(DEV), txt.to(DEV), k, workspace=ws)
        torch.cuda.synchronize()
        ok, _, msgs = accept.check_index_sets(idx.cpu().numpy(), oracle.retrieval_scores(q, kv), k)
        assert ok, (seed, msgs[:3])


@pytest.mark.parametrize("N,k,Tq", [(1440, 360, 8), (5000, 700, 4)], ids=["rows_1440", "rows_5000"])
def test_prefill_scores_out_off_16_byte_alignment(N, k, Tq):
    """The sums of the partial retrieval scores use 16-byte loads and stores
    only when the score buffers are 16-byte aligned. A scores_out 4 bytes past
    a 16-byte boundary takes the 4-byte path (the one-launch select at 1440
    tokens, the long-row sum items at 5000) and gives the same scores and the
    same selection as the aligned buffer."""
    B, Hq, Hkv, D, Tmax = 2, 8, 8, 128, 40
    _say("prefill scores_out alignment", B, Tq, Hq, Hkv, D, N, Tmax, k)
    q, kv, vv, kt, vt = [t.to(DEV) for t in _inputs(B, Tq, Hq, Hkv, D, N, Tmax, seed=7)]
    txt = torch.tensor([40, 17], dtype=torch.int32, device=DEV)
    out_a, idx_a, sc_a = sv.prefill_attend_retrieve(q, kv, vv, kt, vt, txt, k, scores=True)
    buf = torch.zeros(B * N + 4, dtype=torch.float32, device=DEV)
    assert buf.data_ptr() % 16 == 0
    sc_b = buf[1:1 + B * N]
    out_b = torch.empty_like(out_a)
    idx_b = torch.empty_like(idx_a)
    ws = sv.new_workspace(sv.prefill_attend_retrieve_workspace_bytes(B, Tq, Hq, Hkv, D, N, Tmax), DEV)
    lib = sv.load()
    rc = lib.sv_prefill_attend_retrieve(
        q.data_ptr(), B, Tq, Hq, kv.data_ptr(), vv.data_ptr(), kv.stride(0), kv.stride(1), N, Hkv,
        D, kt.data_ptr(), vt.data_ptr(), kt.stride(0), kt.stride(1), txt.data_ptr(), Tmax,
        sv.SV_BF16, 0.0, k, out_b.data_ptr(), idx_b.data_ptr(), sc_b.data_ptr(), ws.data_ptr(),
        ws.numel() * ws.element_size(), sv._stream(torch.device(DEV)))
    torch.cuda.synchronize()
    assert rc == 0, lib.sv_last_error().decode()
    assert torch.equal(sc_b.view(B, N), sc_a)
    assert torch.equal(idx_b, idx_a)
    assert torch.equal(out_b, out_a)
