"""ctypes binding of ``libjt.so`` (the C ABI declared in include/jt.h).

Argument marshalling only: the functions below take torch tensors that live
on the GPU, allocate the outputs and the workspace with torch (torch is used
for device memory and streams), pass raw pointers and the current HIP stream
to the library, and raise on a non-OK status.  Every step of the computation
runs in the library's HIP kernels.  There is no fallback: if the library is
missing or the GPU is absent the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# JT_LIBRARY selects another build of the same library (e.g. the host-only
# sanitized one that the CPU checks of the C ABI's validation load)
LIB_PATH = os.environ.get("JT_LIBRARY") or os.path.join(HERE, "libjt.so")

JT_F32, JT_BF16 = 0, 1
JT_EXPAND_CANDIDATE, JT_EXPAND_NODE_BLOCK = 0, 1
JT_DRAFT_TOPW, JT_DRAFT_SAMPLED = 0, 1
JT_OK, JT_ERR_INVALID_ARG, JT_ERR_UNSUPPORTED, JT_ERR_WORKSPACE, JT_ERR_LAUNCH, JT_ERR_SCRATCH = (
    range(6))
ACCEPT_SCRATCH_BYTES = 4 << 20
DERR_BAD_LOGIT, DERR_BAD_PARENT, DERR_BAD_NNODES, DERR_BAD_PAGE, DERR_BAD_PREFIX, DERR_BAD_DEPTH = (
    1, 2, 4, 8, 16, 32)
DERR_BAD_TOKEN, DERR_BAD_PATH, DERR_BAD_UNIFORM = 64, 128, 256

_c_int, _c_size, _vp, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

SIGNATURES = {
    "jt_status_string": (ctypes.c_char_p, [_c_int]),
    "jt_version": (_c_int, []),
    "jt_build_tree_workspace": (_c_size, [_c_int] * 5),
    "jt_build_tree": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "jt_build_tree_variant": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       ctypes.c_double, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _c_size, _vp]),
    "jt_tree_meta": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp]),
    "jt_tree_attention_workspace": (_c_size, [_c_int] * 8),
    "jt_tree_attention": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_float, _vp, _vp,
                                   _vp, _vp, _c_size, _vp]),
    "jt_accept_workspace": (_c_size, [_c_int] * 3),
    "jt_accept": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _c_size, _vp]),
    "jt_accept_noalloc": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _vp]),
    "jt_accept_margin": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                  ctypes.c_double, ctypes.c_double, _vp, _vp, _vp, _vp, _vp,
                                  _c_size, _vp]),
    "jt_commit_kv": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _c_int,
                              _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "jt_accept_stochastic_workspace": (_c_size, [_c_int, _c_int]),
    "jt_accept_stochastic": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
                                      _vp, _vp, _c_float, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _c_size, _vp]),
}


class JTError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the library once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


# (the argtypes declare pointers as c_void_p, which takes a plain int or None)
def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int):
    if status != JT_OK:
        raise JTError(fn, status, load().jt_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return JT_F32
    if t.dtype == torch.bfloat16:
        return JT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _cuda(t: torch.Tensor, name: str):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def _workspace(nbytes: int, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _tree_outputs(b: int, T: int, dev, with_score: bool):
    out = {k: torch.empty((b, T), dtype=torch.int32, device=dev) for k in ("parent", "token", "depth")}
    out["score"] = torch.empty((b, T), dtype=torch.float64, device=dev) if with_score else None
    out["n_nodes"] = torch.empty((b,), dtype=torch.int32, device=dev)
    return out


def _check_tree_outputs(out: dict, b: int, T: int):
    for k in ("parent", "token", "depth"):
        t = out[k]
        if t.dtype != torch.int32 or tuple(t.shape) != (b, T) or not t.is_contiguous():
            raise ValueError(f"out[{k!r}] must be a contiguous int32 [{b}, {T}] tensor")
    sc = out.get("score")
    if sc is not None and (sc.dtype != torch.float64 or tuple(sc.shape) != (b, T)
                           or not sc.is_contiguous()):
        raise ValueError(f"out['score'] must be a contiguous float64 [{b}, {T}] tensor or None")
    nn = out["n_nodes"]
    if nn.dtype != torch.int32 or tuple(nn.shape) != (b,):
        raise ValueError(f"out['n_nodes'] must be an int32 [{b}] tensor")


def jt_build_tree(draft_logits: torch.Tensor, width_w: int, budget_b: int,
                  root_token: torch.Tensor, err: torch.Tensor | None = None,
                  with_score: bool = True, workspace: torch.Tensor | None = None,
                  out: dict | None = None):
    """Returns dict(parent, token, depth, score, n_nodes) for a [b, N, V] batch
    (written into `out` when given: the same keys, preallocated)."""
    lib = load()
    _cuda(draft_logits, "draft_logits")
    b, N, V = draft_logits.shape
    dev = draft_logits.device
    T = budget_b + 1
    if out is None:
        out = _tree_outputs(b, T, dev, with_score)
    else:
        _check_tree_outputs(out, b, T)
    ws = (workspace if workspace is not None
          else _workspace(lib.jt_build_tree_workspace(b, N, V, width_w, budget_b), dev))
    _check("jt_build_tree", lib.jt_build_tree(
        _ptr(draft_logits), _dtype_code(draft_logits), b, N, V, width_w, budget_b, _ptr(root_token),
        _ptr(out["parent"]), _ptr(out["token"]), _ptr(out["depth"]), _ptr(out["score"]),
        _ptr(out["n_nodes"]), _ptr(err), _ptr(ws), ws.numel(), _stream()))
    return out


def jt_build_tree_variant(draft_logits: torch.Tensor, width_w: int, budget_b: int,
                          root_token: torch.Tensor, expand: str = "candidate",
                          entropy_weight: float = 0.0, err: torch.Tensor | None = None,
                          with_score: bool = True, workspace: torch.Tensor | None = None):
    """Build-mode variants; expand is "candidate" or "node_block".  Same outputs as jt_build_tree."""
    lib = load()
    _cuda(draft_logits, "draft_logits")
    modes = {"candidate": JT_EXPAND_CANDIDATE, "node_block": JT_EXPAND_NODE_BLOCK}
    if expand not in modes:
        raise ValueError(f"unknown expand mode {expand!r}")
    b, N, V = draft_logits.shape
    dev = draft_logits.device
    T = budget_b + 1
    out = _tree_outputs(b, T, dev, with_score)
    ws = (workspace if workspace is not None
          else _workspace(lib.jt_build_tree_workspace(b, N, V, width_w, budget_b), dev))
    _check("jt_build_tree_variant", lib.jt_build_tree_variant(
        _ptr(draft_logits), _dtype_code(draft_logits), b, N, V, width_w, budget_b, modes[expand],
        float(entropy_weight), _ptr(root_token), _ptr(out["parent"]), _ptr(out["token"]),
        _ptr(out["depth"]), _ptr(out["score"]), _ptr(out["n_nodes"]), _ptr(err), _ptr(ws),
        ws.numel(), _stream()))
    return out


def jt_tree_meta(parent: torch.Tensor, n_nodes: torch.Tensor, err: torch.Tensor | None = None,
                 out: torch.Tensor | None = None):
    """Ancestor bitmasks [b, T, ceil(T/32)] as int32 words (uint32 bit patterns)."""
    lib = load()
    _cuda(parent, "parent")
    b, T = parent.shape
    if out is None:
        out = torch.empty((b, T, (T + 31) // 32), dtype=torch.int32, device=parent.device)
    _check("jt_tree_meta", lib.jt_tree_meta(_ptr(parent), _ptr(n_nodes), b, T, _ptr(out),
                                            _ptr(err), _stream()))
    return out


def jt_tree_attention(q, k_pool, v_pool, n_nodes, prefix_len, page_table, num_pages, anc_mask,
                      scale: float, err=None, with_lse: bool = True, out=None, lse=None,
                      workspace=None):
    """Paged tree attention; returns (out [b, T, Hq, D], lse [b, T, Hq] or None)."""
    lib = load()
    for t, nm in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool"), (page_table, "page_table")):
        _cuda(t, nm)
    b, T, hq, D = q.shape
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or k_pool.shape[3] != D:
        raise ValueError("k_pool and v_pool must both be [num_pages, Hkv, page_size, head_dim]")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q, k_pool and v_pool must share a dtype")
    hkv, ps = k_pool.shape[1], k_pool.shape[2]
    if page_table.dim() != 2 or page_table.shape[0] != b:
        raise ValueError("page_table must be [batch, max_pages]")
    maxp = page_table.shape[1]
    if not 1 <= int(num_pages) <= k_pool.shape[0]:
        raise ValueError(f"num_pages={num_pages} outside [1, {k_pool.shape[0]}] (the pool's pages)")
    for t, nm, shape in ((n_nodes, "n_nodes", (b,)), (prefix_len, "prefix_len", (b,)),
                         (page_table, "page_table", None),
                         (anc_mask, "anc_mask", (b, T, (T + 31) // 32))):
        _cuda(t, nm)
        if t.dtype != torch.int32 or t.device != q.device:
            raise TypeError(f"{nm} must be an int32 tensor on {q.device}")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{nm} has shape {tuple(t.shape)}, expected {shape}")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((b, T, hq), dtype=torch.float32, device=q.device)
    ws = (workspace if workspace is not None
          else _workspace(lib.jt_tree_attention_workspace(b, T, hq, hkv, D, maxp, ps, dt), q.device))
    _check("jt_tree_attention", lib.jt_tree_attention(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), dt, b, T, hq, hkv, D, _ptr(n_nodes),
        _ptr(prefix_len), _ptr(page_table), maxp, int(num_pages), ps, _ptr(anc_mask),
        float(scale), _ptr(out), _ptr(lse), _ptr(err), _ptr(ws), ws.numel(), _stream()))
    return out, lse


def _accept_outputs(b: int, depth_n: int, dev, out):
    if out is None:
        return (torch.empty((b,), dtype=torch.int32, device=dev),
                torch.empty((b, depth_n), dtype=torch.int32, device=dev),
                torch.empty((b,), dtype=torch.int32, device=dev))
    alen, anodes, bonus = out
    for t, nm, shape in ((alen, "accept_len", (b,)), (anodes, "accept_nodes", (b, depth_n)),
                         (bonus, "bonus_token", (b,))):
        if t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous int32 {list(shape)} tensor")
    return alen, anodes, bonus


def jt_accept(target_logits, depth_n: int, parent, token, depth, n_nodes, err=None,
              workspace=None, out=None):
    """Returns (accept_len [b], accept_nodes [b, depth_n], bonus_token [b])
    (written into `out` when given: that tuple, preallocated)."""
    lib = load()
    _cuda(target_logits, "target_logits")
    b, T, V = target_logits.shape
    dev = target_logits.device
    alen, anodes, bonus = _accept_outputs(b, depth_n, dev, out)
    ws = (workspace if workspace is not None
          else _workspace(lib.jt_accept_workspace(b, T, V), dev))
    _check("jt_accept", lib.jt_accept(
        _ptr(target_logits), _dtype_code(target_logits), b, T, V, depth_n, _ptr(parent),
        _ptr(token), _ptr(depth), _ptr(n_nodes), _ptr(alen), _ptr(anodes), _ptr(bonus),
        _ptr(err), _ptr(ws), ws.numel(), _stream()))
    return alen, anodes, bonus


def jt_accept_noalloc(target_logits, depth_n: int, parent, token, depth, n_nodes, accept_len,
                      accept_nodes, bonus_token, err=None):
    """jt_accept without a workspace (the library's static scratch instead);
    the caller passes every output, so nothing is allocated here either."""
    lib = load()
    _cuda(target_logits, "target_logits")
    b, T, V = target_logits.shape
    _check("jt_accept_noalloc", lib.jt_accept_noalloc(
        _ptr(target_logits), _dtype_code(target_logits), b, T, V, depth_n, _ptr(parent),
        _ptr(token), _ptr(depth), _ptr(n_nodes), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(bonus_token), _ptr(err), _stream()))
    return accept_len, accept_nodes, bonus_token


def jt_accept_margin(target_logits, depth_n: int, parent, token, depth, n_nodes,
                     theta: float, temperature: float = 1.0, err=None, workspace=None):
    """Margin acceptance: keep a token whose probability ratio to the top-1
    token, under softmax(logits / temperature), reaches theta in (0, 1].

    Returns (accept_len [b], accept_nodes [b, depth_n], bonus_token [b]).
    """
    lib = load()
    _cuda(target_logits, "target_logits")
    b, T, V = target_logits.shape
    dev = target_logits.device
    alen, anodes, bonus = _accept_outputs(b, depth_n, dev, None)
    ws = (workspace if workspace is not None
          else _workspace(lib.jt_accept_workspace(b, T, V), dev))
    _check("jt_accept_margin", lib.jt_accept_margin(
        _ptr(target_logits), _dtype_code(target_logits), b, T, V, depth_n, _ptr(parent),
        _ptr(token), _ptr(depth), _ptr(n_nodes), float(theta), float(temperature), _ptr(alen),
        _ptr(anodes), _ptr(bonus), _ptr(err), _ptr(ws), ws.numel(), _stream()))
    return alen, anodes, bonus


def jt_commit_kv(k_pool, v_pool, page_table, num_pages, n_nodes, max_nodes: int, accept_len,
                 accept_nodes, prefix_len, parent=None, err=None):
    """Moves the accepted rows next to the prefix in place; advances prefix_len in place.

    parent [b, max_nodes] int32 (optional): when given, accept_nodes must
    also form a root-to-node chain of that tree.
    """
    lib = load()
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool"), (page_table, "page_table"),
                  (accept_nodes, "accept_nodes"), (prefix_len, "prefix_len")):
        _cuda(t, nm)
    hkv, ps, D = k_pool.shape[1], k_pool.shape[2], k_pool.shape[3]
    b, maxp = page_table.shape
    depth_n = accept_nodes.shape[1]
    _check("jt_commit_kv", lib.jt_commit_kv(
        _ptr(k_pool), _ptr(v_pool), _dtype_code(k_pool), b, hkv, D, _ptr(page_table), maxp,
        int(num_pages), ps, _ptr(n_nodes), _ptr(parent), int(max_nodes), depth_n, _ptr(accept_len),
        _ptr(accept_nodes), _ptr(prefix_len), _ptr(err), _stream()))


def jt_accept_stochastic(target_logits, depth_n: int, parent, token, depth, n_nodes,
                         temperature: float, u_accept, u_sample, draft_logits=None,
                         draft_mode: str = "topw", err=None, workspace=None):
    """Lossless verification at temperature T > 0 with caller-supplied uniforms.

    draft_mode "topw": siblings are chosen tokens (jt_build_tree's trees);
    draft_logits is not used.  "sampled": every child was drawn i.i.d. from
    softmax(draft row / T); draft_logits [b, depth_n, V] is required.
    u_accept [b, max_nodes] f32, u_sample [b] f32, all in [0, 1).
    Returns (accept_len [b], accept_nodes [b, depth_n], bonus_token [b]).
    """
    lib = load()
    modes = {"topw": JT_DRAFT_TOPW, "sampled": JT_DRAFT_SAMPLED}
    if draft_mode not in modes:
        raise ValueError(f"unknown draft mode {draft_mode!r}")
    for t, nm in ((target_logits, "target_logits"), (u_accept, "u_accept"),
                  (u_sample, "u_sample")):
        _cuda(t, nm)
    b, T, V = target_logits.shape
    if draft_mode == "sampled":
        if draft_logits is None:
            raise ValueError("draft_mode='sampled' needs draft_logits")
        _cuda(draft_logits, "draft_logits")
        if draft_logits.dtype != target_logits.dtype:
            raise TypeError("target_logits and draft_logits must share a dtype")
        if tuple(draft_logits.shape) != (b, depth_n, V):
            raise ValueError("draft_logits must be [batch, depth_n, vocab]")
    if u_accept.dtype != torch.float32 or u_sample.dtype != torch.float32:
        raise TypeError("u_accept and u_sample must be float32")
    if tuple(u_accept.shape) != (b, T) or tuple(u_sample.shape) != (b,):
        raise ValueError("inconsistent shapes")
    dev = target_logits.device
    alen = torch.empty((b,), dtype=torch.int32, device=dev)
    anodes = torch.empty((b, depth_n), dtype=torch.int32, device=dev)
    bonus = torch.empty((b,), dtype=torch.int32, device=dev)
    ws = workspace if workspace is not None else _workspace(
        lib.jt_accept_stochastic_workspace(b, V), dev)
    dr = draft_logits if draft_mode == "sampled" else None
    _check("jt_accept_stochastic", lib.jt_accept_stochastic(
        _ptr(target_logits), _ptr(dr), _dtype_code(target_logits), b, T, V, depth_n,
        _ptr(parent), _ptr(token), _ptr(depth), _ptr(n_nodes), float(temperature),
        modes[draft_mode], _ptr(u_accept), _ptr(u_sample), _ptr(alen), _ptr(anodes), _ptr(bonus),
        _ptr(err), _ptr(ws), ws.numel(), _stream()))
    return alen, anodes, bonus
