"""jt_accept_noalloc (the entry point for callers that cannot allocate device
memory) against jt_accept on the same inputs: two calls in a row, the second
on a smaller input, so a result that leaned on the first call's scratch
contents would show; plus the host-side rejection of inputs beyond the
static scratch."""
import ctypes

import numpy as np
import pytest
import torch

from tree_causal_attention_amd import binding as B

pytestmark = pytest.mark.gpu

VOCAB = 151936


def _case(b, N, W, Bb, seed, dtype):
    """A tree from jt_build_tree on random draft rows, random target rows
    with the deepest path of every other sequence planted (+50 on the
    parent's row at the node's token), all on the device."""
    d = torch.device("cuda:0")
    g = torch.Generator(device=d).manual_seed(seed)
    draft = torch.randn((b, N, VOCAB), generator=g, device=d) * 4.0
    root = torch.randint(0, VOCAB, (b,), generator=g, device=d, dtype=torch.int32)
    tree = B.jt_build_tree(draft, W, Bb, root)
    T = Bb + 1
    target = torch.randn((b, T, VOCAB), generator=g, device=d) * 4.0
    par, tok, dep, nn = (tree[k].cpu().numpy() for k in ("parent", "token", "depth", "n_nodes"))
    for s in range(0, b, 2):
        u = int(np.argmax(dep[s][:nn[s]]))
        while u > 0:
            p = int(par[s][u])
            target[s, p, int(tok[s][u])] += 50.0
            u = p
    if dtype == "bf16":
        target = target.to(torch.bfloat16)
    return target, tree


def _outputs(b, N, d):
    return (torch.full((b,), -7, dtype=torch.int32, device=d),
            torch.full((b, N), -7, dtype=torch.int32, device=d),
            torch.full((b,), -7, dtype=torch.int32, device=d))


def _compare(target, tree, N):
    d = target.device
    b = target.shape[0]
    err_ref = torch.zeros(1, dtype=torch.int32, device=d)
    ref = B.jt_accept(target, N, tree["parent"], tree["token"], tree["depth"], tree["n_nodes"],
                      err=err_ref)
    err = torch.zeros(1, dtype=torch.int32, device=d)
    got = B.jt_accept_noalloc(target, N, tree["parent"], tree["token"], tree["depth"],
                              tree["n_nodes"], *_outputs(b, N, d), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == int(err_ref.item()) == 0
    for r, g_ in zip(ref, got):
        assert torch.equal(r, g_)
    assert (ref[0][0::2] >= 1).all()  # the planted paths were accepted


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_accept_twice_second_smaller(dtype):
    print(f"noalloc: batch 8 x 257 rows then batch 1 x 17 rows ({dtype})", flush=True)
    target, tree = _case(8, 16, 8, 256, 11, dtype)
    _compare(target, tree, 16)
    target, tree = _case(1, 8, 4, 16, 12, dtype)
    _compare(target, tree, 8)


def test_noalloc_rejects_inputs_beyond_scratch():
    lib = B.load()
    p = ctypes.c_void_p(1)
    # 300 x 1024 rows of 8 chunks need 19.7 MB of partials: refused on the host
    assert lib.jt_accept_workspace(300, 1024, VOCAB) > B.ACCEPT_SCRATCH_BYTES
    st = lib.jt_accept_noalloc(p, 0, 300, 1024, VOCAB, 16, p, p, p, p, p, p, p, None, None)
    assert st == B.JT_ERR_SCRATCH
    assert lib.jt_status_string(st).decode().startswith("inputs need more")
    assert lib.jt_accept_noalloc(p, 0, 300, 1025, VOCAB, 16, p, p, p, p, p, p, p, None,
                                 None) == B.JT_ERR_UNSUPPORTED
