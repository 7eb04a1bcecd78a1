"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
F32_MAX_ABS = 1e-5
LSE_ABS = {"bf16": 1e-3, "f32": 1e-5}


def dev():
    return torch.device("cuda:0")


def to_np(t):
    return t.detach().cpu().numpy()


def as_f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def check_attention(o_gpu, o_ref, dtype, what=""):
    """o_gpu, o_ref: float64 arrays of the compared outputs."""
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite GPU output"
    diff = np.abs(o_gpu - o_ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    if dtype == "f32":
        assert max_abs <= F32_MAX_ABS, f"{what}: max-abs {max_abs:.3g} > {F32_MAX_ABS}"
        return max_abs, 0.0
    rel = float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    assert max_abs <= BF16_MAX_ABS, f"{what}: max-abs {max_abs:.3g} > {BF16_MAX_ABS}"
    assert rel <= BF16_REL_L2, f"{what}: rel-L2 {rel:.3g} > {BF16_REL_L2}"
    return max_abs, rel


def check_lse(l_gpu, l_ref, dtype, what=""):
    d = float(np.abs(l_gpu - l_ref).max()) if l_ref.size else 0.0
    assert d <= LSE_ABS[dtype], f"{what}: lse max-abs {d:.3g}"
    return d


def upload(x, device):
    return {
        "q": x.q.to(device), "k": x.k_pool.to(device), "v": x.v_pool.to(device),
        "prefix": x.prefix_len.to(device), "table": x.page_table.to(device),
        "root": x.root_token.to(device),
    }
