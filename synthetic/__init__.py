"""Seeded synthetic workloads for SparseVILA's decoupled visual sparsity.

This module only draws inputs. It holds none of the method's arithmetic
(no scoring, selection, softmax or salience): the CPU oracle and the HIP
library both consume what it produces, and neither imports the other.

Every tensor is drawn from its own ``torch.Generator`` whose seed is a
stable hash of (seed, workload, layer, tensor name), so any tensor can be
regenerated alone.  Floating tensors are drawn in fp32 and then rounded to
the workload's storage dtype (round-to-nearest-even for bf16); both sides
of a parity test see exactly those stored bits.

Workload shapes stand in for the pages' settings (no dataset items, no
weights): LLaVA-1.5-style 576-token images and LLaVA-NeXT-style 5x576
multi-crop images (SparseVILA review, image results table), LongVILA-style
256-frame video on a Qwen2-7B-shaped GQA backbone (SparseVILA review, video
results table; arXiv abstract page, Fig. 5), a SigLIP-shaped encoder with
27x27 patches per frame (SparseVILA summary, Sec. 3.1 salience table) and
multi-turn reuse of one visual cache (SparseVILA summary, Sec. 4.1).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import torch

__all__ = [
    "DecodeWorkload", "SalienceWorkload", "DECODE", "SALIENCE",
    "stream_seed", "make_decode_layer", "make_salience", "multiturn_text_lengths",
    "scaled_decode", "scaled_salience",
]


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Shape of one decode-side workload (retrieval + sparse attention)."""
    name: str
    B: int          # sequences
    L: int          # decoder layers (each has its own caches and query)
    Hq: int         # query heads
    Hkv: int        # key/value heads (GQA group size G = Hq // Hkv)
    D: int          # head dim
    N: int          # retained visual tokens in the cache
    T: int          # text entries attended at the measured step (incl. current token)
    Tmax: int       # text-cache capacity (>= T)
    k: int          # visual tokens retrieved per (sequence, layer)
    dtype: torch.dtype
    planted: int    # planted relevant tokens per (sequence, layer); 0 = pure Gaussian
    plant_gain: float = 3.0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


@dataclasses.dataclass(frozen=True)
class SalienceWorkload:
    """Shape of the prefill-side salience workload (one encoder layer)."""
    name: str
    F: int          # frames, each an independent attention
    N: int          # tokens per frame
    H: int          # encoder heads
    D: int          # head dim
    keep: int       # tokens kept per frame
    std: float      # standard deviation of Q and K entries
    dtype: torch.dtype = torch.bfloat16


# 576-token image, fp32, one layer: the correctness anchor.
# 16 planted tokens; k = 25% of 576.
DECODE: Dict[str, DecodeWorkload] = {
    "image576_fp32": DecodeWorkload(
        name="image576_fp32", B=1, L=1, Hq=32, Hkv=32, D=128, N=576, T=64, Tmax=64,
        k=144, dtype=torch.float32, planted=16),
    # LLaVA-NeXT-7B-shaped: 5x576 visual tokens pruned to 50% (1440) at prefill,
    # k = 360 per step, 256 text entries, 5% planted.
    "llava_next_7b": DecodeWorkload(
        name="llava_next_7b", B=8, L=32, Hq=32, Hkv=32, D=128, N=1440, T=256, Tmax=256,
        k=360, dtype=torch.bfloat16, planted=72),
    # Qwen2-7B GQA long video: 256 frames x 196 tokens = 50176, 50% retained.
    "qwen2_7b_video": DecodeWorkload(
        name="qwen2_7b_video", B=1, L=28, Hq=28, Hkv=4, D=128, N=25088, T=512, Tmax=512,
        k=2048, dtype=torch.bfloat16, planted=0),
    # Long-context multi-turn: 131072 retained tokens, one layer measured.
    # Text capacity: 64 system + 64 question + 128 generated entries.
    "multiturn_128k": DecodeWorkload(
        name="multiturn_128k", B=4, L=1, Hq=32, Hkv=32, D=128, N=131072, T=256, Tmax=256,
        k=4096, dtype=torch.bfloat16, planted=0),
}

# SigLIP-shaped encoder, 256 frames x 729 (27x27) tokens, 16 heads, D = 72, no
# summary token.  Q, K ~ N(0, variance 1/sqrt(72)), i.e. std = 72**-0.25.
# Keep floor(0.5 * 729) = 364 tokens per frame.
SALIENCE: Dict[str, SalienceWorkload] = {
    "siglip_256f": SalienceWorkload(
        name="siglip_256f", F=256, N=729, H=16, D=72, keep=364, std=72 ** -0.25),
    # Alternative reading of N(0, 1/sqrt(72)): standard deviation 1/sqrt(72).
    "siglip_256f_narrow": SalienceWorkload(
        name="siglip_256f_narrow", F=256, N=729, H=16, D=72, keep=364, std=72 ** -0.5),
    # Summary-token encoders: CLIP ViT-L/14 at 336 px (one CLS token + 24 x 24
    # patches, 16 heads of 64) and a RADIO-style encoder (4 summary tokens +
    # 32 x 32 patches, 16 heads of 64); same entry distribution as above.
    "clip_l14_336_256f": SalienceWorkload(
        name="clip_l14_336_256f", F=256, N=577, H=16, D=64, keep=288, std=64 ** -0.25),
    "radio_1028_64f": SalienceWorkload(
        name="radio_1028_64f", F=64, N=1028, H=16, D=64, keep=514, std=64 ** -0.25),
    # QwenVL-style encoder attending over one long visual input: 16384 tokens
    # (e.g. a 128 x 128 patch grid) in one attention, 16 heads of 80; keep 50%.
    "qwenvl_16k": SalienceWorkload(
        name="qwenvl_16k", F=1, N=16384, H=16, D=80, keep=8192, std=80 ** -0.25),
}

# Multi-turn schedule of the 131072-token workload: 3 rounds x 128 decode steps,
# 64 system entries kept across rounds, 64 question entries appended at round
# start, one entry appended per generated token.
MULTITURN = dict(rounds=3, steps=128, system=64, question=64)


def multiturn_text_lengths(rounds: int = 3, steps: int = 128, system: int = 64,
                           question: int = 64) -> List[List[int]]:
    """Text entries attended at each decode step of each round.

    The current token's K/V is appended before its attention, so step t of a
    round attends system + question + t + 1 entries.  At the end of a round the
    previous question and answer are evicted and the length returns to
    ``system`` (partial eviction; the visual cache is untouched).
    """
    return [[system + question + t + 1 for t in range(steps)] for _ in range(rounds)]


def scaled_decode(w: DecodeWorkload, *, B=None, L=None, N=None, T=None, Tmax=None,
                  k=None, planted=None, name=None, Hq=None, Hkv=None, D=None,
                  dtype=None) -> DecodeWorkload:
    """A smaller (or reshaped) copy of a workload, for tests the oracle finishes in seconds."""
    kw = dict(B=B, L=L, N=N, T=T, Tmax=Tmax, k=k, planted=planted, name=name, Hq=Hq, Hkv=Hkv,
              D=D, dtype=dtype)
    kw = {a: b for a, b in kw.items() if b is not None}
    if "T" in kw and "Tmax" not in kw:
        kw["Tmax"] = max(kw["T"], w.Tmax if w.Tmax >= kw["T"] else kw["T"])
    return dataclasses.replace(w, **kw)


def scaled_salience(w: SalienceWorkload, *, F=None, N=None, H=None, D=None, keep=None,
                    name=None) -> SalienceWorkload:
    kw = dict(F=F, N=N, H=H, D=D, keep=keep, name=name)
    return dataclasses.replace(w, **{a: b for a, b in kw.items() if b is not None})


def stream_seed(seed: int, *parts) -> int:
    """Stable 63-bit seed for one named tensor stream."""
    h = hashlib.sha256(("/".join([str(seed)] + [str(p) for p in parts])).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, *parts))
    return g


def _normal(shape, std, device, seed, *parts) -> torch.Tensor:
    g = _gen(device, seed, *parts)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def make_decode_layer(w: DecodeWorkload, seed: int, layer: int = 0,
                      device="cpu", gen_device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Inputs of one decode step at one layer.

    Returns (all on ``device``):
      q       [B][1][Hq][D]    current token's queries (post-RoPE), dtype w.dtype
      k_vis   [B][N][Hkv][D]   retained visual keys, token-major
      v_vis   [B][N][Hkv][D]
      k_txt   [B][Tmax][Hkv][D] text keys (first txt_len[b] rows valid)
      v_txt   [B][Tmax][Hkv][D]
      txt_len [B] int32        text entries attended (= w.T)
      planted [B][P] int64     planted visual token indices (P = w.planted)

    Planting (MHA only): for each planted token t and head h, the fp32 key
    row gets 3 * q_h / |q_h| added before rounding to the storage dtype, so
    the planted tokens dominate the retrieval score by construction.
    """
    gd = gen_device or device
    B, N, Hq, Hkv, D, Tmax = w.B, w.N, w.Hq, w.Hkv, w.D, w.Tmax
    tag = (w.name, layer)
    q32 = _normal((B, 1, Hq, D), 1.0, gd, seed, *tag, "q")
    k32 = _normal((B, N, Hkv, D), 1.0, gd, seed, *tag, "k_vis")
    planted = torch.zeros((B, w.planted), dtype=torch.int64)
    if w.planted:
        if Hq != Hkv:
            raise ValueError("planting is defined for MHA workloads only")
        pg = _gen("cpu", seed, *tag, "planted")
        planted = torch.stack([torch.randperm(N, generator=pg)[: w.planted] for _ in range(B)])
        qn = q32[:, 0] / q32[:, 0].norm(dim=-1, keepdim=True)          # [B][H][D]
        pl = planted.to(gd)
        for b in range(B):
            k32[b, pl[b]] += w.plant_gain * qn[b].unsqueeze(0)
    out = {
        "q": q32.to(w.dtype),
        "k_vis": k32.to(w.dtype),
        "v_vis": _normal((B, N, Hkv, D), 1.0, gd, seed, *tag, "v_vis").to(w.dtype),
        "k_txt": _normal((B, Tmax, Hkv, D), 1.0, gd, seed, *tag, "k_txt").to(w.dtype),
        "v_txt": _normal((B, Tmax, Hkv, D), 1.0, gd, seed, *tag, "v_txt").to(w.dtype),
        "txt_len": torch.full((B,), w.T, dtype=torch.int32),
        "planted": planted,
    }
    del k32, q32
    return {n: t.to(device) for n, t in out.items()}


def make_fresh_query(w: DecodeWorkload, seed: int, layer: int, step: int,
                     device="cpu", gen_device: Optional[str] = None) -> torch.Tensor:
    """A new query for decode step ``step`` (multi-turn workload: fresh q each step)."""
    gd = gen_device or device
    q = _normal((w.B, 1, w.Hq, w.D), 1.0, gd, seed, w.name, layer, "q_step", step)
    return q.to(w.dtype).to(device)


def make_text_rows(w: DecodeWorkload, seed: int, layer: int, tag, rows: int,
                   device="cpu", gen_device: Optional[str] = None):
    """``rows`` new text K/V entries per sequence, [B][rows][Hkv][D] each."""
    gd = gen_device or device
    shape = (w.B, rows, w.Hkv, w.D)
    k = _normal(shape, 1.0, gd, seed, w.name, layer, "k_txt_new", tag).to(w.dtype)
    v = _normal(shape, 1.0, gd, seed, w.name, layer, "v_txt_new", tag).to(w.dtype)
    return k.to(device), v.to(device)


def make_salience(w: SalienceWorkload, seed: int, device="cpu",
                  gen_device: Optional[str] = None, frames: Optional[range] = None):
    """Encoder Q and K, [F][H][N][D] in w.dtype, entries ~ N(0, w.std**2).

    ``frames`` selects a sub-range of frames; frame f is always drawn from the
    same stream, so a sub-range equals the matching slice of the full tensor.
    """
    gd = gen_device or device
    fr = range(w.F) if frames is None else frames
    qs, ks = [], []
    for f in fr:
        qs.append(_normal((w.H, w.N, w.D), w.std, gd, seed, w.name, "q", f).to(w.dtype))
        ks.append(_normal((w.H, w.N, w.D), w.std, gd, seed, w.name, "k", f).to(w.dtype))
    return torch.stack(qs).to(device), torch.stack(ks).to(device)


def flop_count_salience(w: SalienceWorkload) -> float:
    """Algorithmic QK^T flops of one salience pass (2*N*N*D per frame-head)."""
    return 2.0 * w.N * w.N * w.D * w.H * w.F


def bytes_per_elem(dtype: torch.dtype) -> int:
    return torch.tensor([], dtype=dtype).element_size()


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)
