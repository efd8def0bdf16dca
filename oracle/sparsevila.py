"""CPU oracle for SparseVILA's decoupled visual sparsity -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct float64 NumPy definitions of what the hot path
computes.  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this module; the product path never does.  It
shares no code with the HIP library.

Sources (web pages on SparseVILA, arXiv 2510.17777):
  [summary]  velog summary "SparseVILA: Decoupling Visual Sparsity for
             Efficient VLM Inference" (Korean), sections 3.1, 3.2, 4.1, 4.5.
  [review]   xllm-io paper review of SparseVILA (Chinese), section
             "三、技术架构 / 核心公式" (salience and retrieval formulas) and
             section "五、代码实现分析" (pseudo-code).
  [abstract] sciencestack page for arXiv 2510.17777 (TL;DR, Fig. 4, Fig. 5).

Readings taken where the pages are silent or garbled (each is listed with
its reason in the design notes):
  * retrieval score = raw q.K logits, summed over every query token and over
    the query heads that share a KV head; one selected set per (sequence,
    layer); no 1/sqrt(D) (it cannot change the order);
  * top-k order is (score descending, index ascending); indices are returned
    in ascending order;
  * the review's salience formula, read literally as a row sum of a softmax,
    is 1/N for every token; it is read as the attention each token RECEIVES
    (column mean), averaged over heads;
  * the salience softmax uses scale 1/sqrt(D), full bidirectional attention
    within a frame, no mask;
  * decode attention attends the selected visual entries plus all txt_len[b]
    text entries with scale 1/sqrt(D); query head h uses KV head h // G;
  * summary-token salience (CLIP: one summary token, RADIO: several) is the
    attention the summary tokens pay to each token, averaged over the
    summary tokens and the heads; the summary tokens are the first S tokens
    of the frame, and every token (summary tokens included) is scored and
    can be kept;
  * dense packing keeps the order of the index list and copies every KV head
    of a selected token (one selected set per sequence); an index outside
    [0, N) gives a zero row.

Parity pins: every function here is pinned in tests/test_oracle.py against
hand-derived fixtures (tests/golden/), closed forms, invariants, brute force
on tiny inputs and independent library routines.  No function is unpinned.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "to_f64", "retrieval_scores", "topk_ascending", "retrieve",
    "sparse_decode_attn", "dense_decode_attn", "pack_selected", "salience", "salience_prune",
    "summary_salience", "summary_salience_prune", "prefill_attention",
]


def to_f64(x) -> np.ndarray:
    """Exact widening of a torch tensor (fp32 / bf16 / int) or array to NumPy.

    Floating inputs become float64 (bf16 and fp32 values are exactly
    representable); integer inputs become int64.
    """
    if hasattr(x, "detach"):                       # torch tensor, without importing torch
        x = x.detach().to("cpu")
        if x.is_floating_point() and x.element_size() < 4:
            x = x.float()                          # bf16 / fp16: exact in fp32
        x = x.numpy()
    x = np.asarray(x)
    if np.issubdtype(x.dtype, np.floating):
        return x.astype(np.float64)
    return x.astype(np.int64)


def retrieval_scores(q, k_vis) -> np.ndarray:
    """Query-aware relevance of every retained visual token.

    [summary] Sec. 3.2 "Query-Aware Token Selection": the text query acts as
    Query, the cached vision tokens as Key, and the aggregated attention
    strength between them ranks the tokens.  [review] 核心公式:
    Selected = TopK(Query . KV_Cache, k), and the pseudo-code's
    ``matmul(query, keys.T)``.

    q      [B][Tq][Hq][D]
    k_vis  [B][N][Hkv][D]
    returns s [B][N] float64 with
        s[b, t] = sum_{tau < Tq} sum_{h < Hq} q[b, tau, h, :] . K[b, t, h // G, :]
    computed head by head exactly as written (no pre-summed query).
    """
    q = to_f64(q)
    K = to_f64(k_vis)
    B, Tq, Hq, D = q.shape
    Bk, N, Hkv, Dk = K.shape
    assert B == Bk and D == Dk and Hq % Hkv == 0
    G = Hq // Hkv
    s = np.zeros((B, N), dtype=np.float64)
    for b in range(B):
        for tau in range(Tq):
            for h in range(Hq):
                s[b] += K[b, :, h // G, :] @ q[b, tau, h, :]
    return s


def topk_ascending(s, k: int) -> np.ndarray:
    """The k largest entries of each row, ties to the lower index, in ascending index order.

    [review] 核心公式 TopK(., k); order (value desc, index asc) and ascending
    output are readings (the pages fix neither).
    s [R][N] -> int64 [R][k].  Requires 0 <= k <= N.
    """
    s = np.asarray(s, dtype=np.float64)
    R, N = s.shape
    if not 0 <= k <= N:
        raise ValueError(f"k={k} outside [0, {N}]")
    out = np.empty((R, k), dtype=np.int64)
    idx = np.arange(N)
    for r in range(R):
        order = np.lexsort((idx, -s[r]))           # primary: -s, secondary: index
        out[r] = np.sort(order[:k])
    return out


def retrieve(q, k_vis, k: int) -> np.ndarray:
    """Indices [B][k] of the k visual tokens most relevant to the query."""
    return topk_ascending(retrieval_scores(q, k_vis), k)


def sparse_decode_attn(q, k_vis, v_vis, idx, k_txt, v_txt, txt_len,
                       scale: Optional[float] = None) -> np.ndarray:
    """Decode attention over the retrieved visual entries plus the text entries.

    [summary] Sec. 3.2: only the query-relevant subset of the cache is
    activated for attention; the rest stays cached but deactivated.  Sec. 4.5
    (decoding attention kernel): attention runs over the reduced effective
    KV cache.  Standard scaled-dot-product softmax attention over that set.

    q       [B][Hq][D] (or [B][1][Hq][D])
    k_vis, v_vis  [B][N][Hkv][D]
    idx     [B][k]  visual entries (any order; duplicates are not expected)
    k_txt, v_txt  [B][Tmax][Hkv][D], first txt_len[b] rows attended
    returns out [B][Hq][D] float64:
        E = idx[b] followed by text rows 0..txt_len[b]-1
        z_j = scale * q[b,h] . K_j[h // G];  p = softmax(z);  out = sum_j p_j V_j[h // G]
    scale defaults to 1/sqrt(D).
    """
    q = to_f64(q)
    if q.ndim == 4:
        assert q.shape[1] == 1
        q = q[:, 0]
    Kv, Vv = to_f64(k_vis), to_f64(v_vis)
    Kt, Vt = to_f64(k_txt), to_f64(v_txt)
    idx = to_f64(idx)
    tl = to_f64(txt_len)
    B, Hq, D = q.shape
    Hkv = Kv.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        T = int(tl[b])
        KE = np.concatenate([Kv[b, idx[b]], Kt[b, :T]], axis=0)     # [E][Hkv][D]
        VE = np.concatenate([Vv[b, idx[b]], Vt[b, :T]], axis=0)
        if KE.shape[0] == 0:
            raise ValueError("empty attention set")
        for h in range(Hq):
            g = h // G
            z = (KE[:, g, :] @ q[b, h]) * scale
            m = z.max()
            p = np.exp(z - m)
            out[b, h] = (p @ VE[:, g, :]) / p.sum()
    return out


def dense_decode_attn(q, k_vis, v_vis, k_txt, v_txt, txt_len,
                      scale: Optional[float] = None) -> np.ndarray:
    """Dense decode attention: every visual token (in order) plus the text entries.

    Same code path as ``sparse_decode_attn`` with idx = 0..N-1, so k = N gives
    a bit-identical result.
    """
    Kv = to_f64(k_vis)
    B, N = Kv.shape[:2]
    idx = np.tile(np.arange(N, dtype=np.int64), (B, 1))
    return sparse_decode_attn(q, k_vis, v_vis, idx, k_txt, v_txt, txt_len, scale)


def pack_selected(k_vis, v_vis, idx) -> Tuple[np.ndarray, np.ndarray]:
    """Dense packing of the selected visual KV entries into contiguous rows.

    [summary] Sec. 3.2 (decode side): the selected KV entries are gathered
    into contiguous memory, so that decode reads them with regular, coalesced
    accesses instead of scattered ones; Sec. 3.3, kernel table (decoding
    attention row): the packed, reduced cache is what decode attends.

    k_vis, v_vis  [B][N][Hkv][D]
    idx           [B][k] visual token indices
    returns (k_pack, v_pack), each [B][k][Hkv][D] in the input's value type:
        pack[b][j] = cache[b][idx[b][j]]   for 0 <= idx[b][j] < N,
        pack[b][j] = 0                     otherwise.
    Values are copied, never rounded (bit-exact).
    """
    Kv, Vv = np.asarray(to_f64(k_vis)), np.asarray(to_f64(v_vis))
    ix = np.asarray(to_f64(idx))
    B, N, Hkv, D = Kv.shape
    k = ix.shape[1]
    kp = np.zeros((B, k, Hkv, D), dtype=Kv.dtype)
    vp = np.zeros((B, k, Hkv, D), dtype=Vv.dtype)
    for b in range(B):
        for j in range(k):
            t = int(ix[b, j])
            if 0 <= t < N:
                kp[b, j] = Kv[b, t]
                vp[b, j] = Vv[b, t]
    return kp, vp


def salience(vis_q, vis_k, scale: Optional[float] = None) -> np.ndarray:
    """Query-agnostic salience of every vision-encoder token, no summary token.

    [summary] Sec. 3.1, salience table (SigLIP / QwenVL row): importance is
    the intra-visual attention averaged over all tokens.  [review] 核心公式
    Salience(t_i) = (1/N) sum_j Attention(t_i, t_j), read as the attention
    token i receives (column mean), averaged over heads.

    vis_q, vis_k [F][H][N][D] -> s [F][N] float64:
        A_h = row-softmax(scale * Q_h K_h^T)   (N x N, materialised)
        s[f, j] = (1/H) sum_h (1/N) sum_i A_h[i, j]
    Each frame sums to 1 over j.
    """
    Q, K = to_f64(vis_q), to_f64(vis_k)
    F, H, N, D = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = np.zeros((F, N), dtype=np.float64)
    for f in range(F):
        for h in range(H):
            S = (Q[f, h] @ K[f, h].T) * scale
            S = S - S.max(axis=1, keepdims=True)
            A = np.exp(S)
            A = A / A.sum(axis=1, keepdims=True)
            s[f] += A.sum(axis=0) / N
        s[f] /= H
    return s


def salience_prune(vis_q, vis_k, keep: int,
                   scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Salience per token and the ``keep`` most salient tokens per frame.

    [summary] Sec. 3.1: tokens with the lowest aggregated salience are pruned
    (really deleted before the cache is stored).  The review's pseudo-code
    thresholds the salience; a fixed keep count per frame (constant prefill
    sparsity, [summary] Sec. 4.1) is the top-``keep`` set.
    returns (s [F][N] float64, idx [F][keep] int64 ascending)
    """
    s = salience(vis_q, vis_k, scale)
    return s, topk_ascending(s, keep)


def summary_salience(vis_q, vis_k, S: int, scale: Optional[float] = None) -> np.ndarray:
    """Salience read off the attention of the summary tokens (CLIP, RADIO).

    [summary] Sec. 3.1, salience table: with one summary token (CLIP) a
    token's importance is the attention through which it feeds the global
    (summary) embedding; with several summary tokens (RADIO) it is that
    attention averaged over the summary tokens.  Read as the softmax rows of
    the summary tokens' queries: summary token s attends over all N tokens,
    and token j receives A_h[s, j].

    vis_q, vis_k [F][H][N][D]; the summary tokens are rows 0..S-1.
    returns s [F][N] float64:
        A_h = row-softmax(scale * Q_h[0:S] K_h^T)   (S x N)
        s[f, j] = (1/H) sum_h (1/S) sum_{s<S} A_h[s, j]
    Each frame sums to 1 over j.
    """
    Q, K = to_f64(vis_q), to_f64(vis_k)
    F, H, N, D = Q.shape
    if not 1 <= S <= N:
        raise ValueError("need 1 <= S <= N summary tokens")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((F, N), dtype=np.float64)
    for f in range(F):
        for h in range(H):
            Z = (Q[f, h, :S] @ K[f, h].T) * scale          # [S][N]
            Z = Z - Z.max(axis=1, keepdims=True)
            A = np.exp(Z)
            A = A / A.sum(axis=1, keepdims=True)
            out[f] += A.sum(axis=0) / S
        out[f] /= H
    return out


def summary_salience_prune(vis_q, vis_k, S: int, keep: int,
                           scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Summary-token salience and the ``keep`` most salient tokens per frame
    (ascending indices, ties toward the lower index), as ``salience_prune``."""
    s = summary_salience(vis_q, vis_k, S, scale)
    return s, topk_ascending(s, keep)


def prefill_attention(q, k_vis, v_vis, k_txt, v_txt, txt_len,
                      scale: Optional[float] = None) -> np.ndarray:
    """Attention of a chunk of query tokens (the current question) at prefill.

    [summary] Sec. 3.2 (query-aware retrieval, its implementation note): the
    retrieval salience of the question is computed while the question's
    tokens go through the ordinary (FlashAttention) prefill attention, whose
    logits against the visual keys are exactly the terms the retrieval score
    sums.  This is that attention: standard causal softmax attention of the
    question tokens over the whole context.

    q       [B][Tq][Hq][D]: the question's tokens, in order
    k_vis, v_vis  [B][N][Hkv][D]: the retained visual cache (earlier in the
            sequence than the question, so every question token sees every
            visual token)
    k_txt, v_txt  [B][Tmax][Hkv][D]: text cache; the first txt_len[b] rows are
            valid and the LAST Tq of them are the question's own rows (the
            caller has appended them)
    returns out [B][Tq][Hq][D] float64: question token tau (text position
        p = txt_len[b] - Tq + tau) attends E = all N visual tokens, then text
        rows 0..p (causal; none when p < 0):
        z_j = scale * q[b,tau,h] . K_j[h // G];  out = sum_j softmax(z)_j V_j[h // G]
    scale defaults to 1/sqrt(D).
    """
    q = to_f64(q)
    Kv, Vv = to_f64(k_vis), to_f64(v_vis)
    Kt, Vt = to_f64(k_txt), to_f64(v_txt)
    tl = to_f64(txt_len)
    B, Tq, Hq, D = q.shape
    Hkv = Kv.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Tq, Hq, D), dtype=np.float64)
    for b in range(B):
        T = int(tl[b])
        for tau in range(Tq):
            p = min(T - Tq + tau, T - 1)
            KE = np.concatenate([Kv[b], Kt[b, :max(p + 1, 0)]], axis=0)   # [E][Hkv][D]
            VE = np.concatenate([Vv[b], Vt[b, :max(p + 1, 0)]], axis=0)
            for h in range(Hq):
                g = h // G
                z = (KE[:, g, :] @ q[b, tau, h]) * scale
                m = z.max()
                w = np.exp(z - m)
                out[b, tau, h] = (w @ VE[:, g, :]) / w.sum()
    return out
