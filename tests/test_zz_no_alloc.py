"""sv_retrieve_attend_noalloc (workspace in a static device array) against
sv_retrieve_attend (caller's workspace), called through the C ABI: the same
indices and the same outputs, bit for bit, on consecutive calls whose sizes
shrink (the array keeps the previous call's contents, so each call must
clear what it needs), and a clean status word after each.
"""
import ctypes

import pytest
import torch

import synthetic
import visual_token_sparsity_amd as sv

pytestmark = pytest.mark.gpu

DEV = "cuda"

# Largest first: each later call reuses scratch the earlier one dirtied.
CALLS = [
    ("long_rows_b2_n65536", "multiturn_128k", dict(B=2, N=65536, k=2048, T=200, Tmax=256)),
    ("llava_b8_full_layer", "llava_next_7b", {}),
    ("llava_b2_small", "llava_next_7b", dict(B=2, N=700, k=100, T=30, Tmax=40)),
]


def _noalloc(lib, w, g, out, idx, scores):
    B, Hq, D = g["q"].shape
    return lib.sv_retrieve_attend_noalloc(
        ctypes.c_void_p(g["q"].data_ptr()), B, Hq, ctypes.c_void_p(g["k_vis"].data_ptr()),
        ctypes.c_void_p(g["v_vis"].data_ptr()), ctypes.c_int64(g["k_vis"].stride(0)),
        ctypes.c_int64(g["k_vis"].stride(1)), w.N, w.Hkv, D, w.k,
        ctypes.c_void_p(g["k_txt"].data_ptr()), ctypes.c_void_p(g["v_txt"].data_ptr()),
        ctypes.c_int64(g["k_txt"].stride(0)), ctypes.c_int64(g["k_txt"].stride(1)),
        ctypes.c_void_p(g["txt_len"].data_ptr()), w.Tmax, sv.SV_BF16, ctypes.c_float(0.0),
        ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(scores.data_ptr()),
        ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point():
    lib = sv.load()
    lib.sv_retrieve_attend_noalloc.restype = ctypes.c_int
    for name, wl, ov in CALLS:
        w = synthetic.scaled_decode(synthetic.DECODE[wl], **ov)
        print("[case] noalloc", name, w, flush=True)
        g = synthetic.make_decode_layer(w, seed=31, device=DEV, gen_device="cuda")
        g["q"] = g["q"][:, 0].contiguous()
        out = torch.full((w.B, w.Hq, w.D), -7.0, dtype=torch.float32, device=DEV)
        idx = torch.full((w.B, w.k), -7, dtype=torch.int32, device=DEV)
        sc = torch.full((w.B, w.N), -7.0, dtype=torch.float32, device=DEV)
        st = _noalloc(lib, w, g, out, idx, sc)
        assert st == 0, lib.sv_last_error()
        ref_out, ref_idx, ref_sc = sv.retrieve_attend(g["q"], g["k_vis"], g["v_vis"], w.k,
                                                      g["k_txt"], g["v_txt"], g["txt_len"],
                                                      scores=True)
        torch.cuda.synchronize()
        assert lib.sv_workspace_status(None, ctypes.c_void_p(
            torch.cuda.current_stream().cuda_stream)) == 0, lib.sv_last_error()
        assert torch.equal(idx, ref_idx), name
        assert torch.equal(sc, ref_sc), name
        assert torch.equal(out, ref_out), name
        # and again on the scratch this call just used
        out.fill_(-7.0)
        idx.fill_(-7)
        assert _noalloc(lib, w, g, out, idx, sc) == 0, lib.sv_last_error()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx) and torch.equal(out, ref_out), name
