"""gdn_project_bf16_noalloc, the projection for callers that cannot allocate, against
gdn_project_bf16 with a workspace of the caller's, through the C ABI.

The two run the same kernels with the same fixed summation order, so the outputs must
be equal bit for bit; the first is also held to the oracle at tol(1).  Two calls in a
row share the library's scratch buffer, the second with a smaller input than the
first (the buffer keeps the first call's partial blocks, which must not matter).  A
shape whose workspace exceeds the buffer is refused and leaves its output untouched."""
import numpy as np
import pytest

import gdn_workloads as W
import oracle
from gpu_harness import assert_close, dev, log

pytestmark = pytest.mark.gpu


def _w(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _operands(rows, k, n, seed):
    import gated_deltanet_mixer_gdn_amd as G
    x, w = W.make_proj(rows, k, n, seed=seed)
    return x, w, G.gdn_split_bf16(dev(x)), G.gdn_pack_bf16(_w(w))


def _with_workspace(xs, wp):
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    nbytes = G.gdn_project_workspace_bytes(xs.rows, xs.k, wp.n)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    return G.gdn_project_bf16(xs, wp, workspace=ws)


def test_noalloc_equals_the_workspace_form_on_two_calls_in_a_row():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    # the out projection at a decode batch (0.94 MiB of partial blocks), then a smaller
    # product that also splits its k range (0.25 MiB)
    shapes = [(32, 6144, 2560, 301), (8, 4096, 512, 302)]
    for rows, k, n, seed in shapes:
        need = G.gdn_project_workspace_bytes(rows, k, n)
        assert 0 < need <= 4 << 20
        log(f"noalloc rows={rows} k={k} n={n}: {need} bytes of scratch")
        x, w, xs, wp = _operands(rows, k, n, seed)
        ref = _with_workspace(xs, wp)
        out = torch.full((rows, n), 7.0, device="cuda")
        G.gdn_project_bf16_noalloc(xs, wp, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"rows={rows} k={k} n={n}: not bit for bit the workspace form's output"
        assert_close(f"noalloc rows={rows}", out.cpu().numpy(), oracle.project(x, w), 1)
    # the first shape again after the second: the scratch holds the smaller call's blocks
    rows, k, n, seed = shapes[0]
    x, w, xs, wp = _operands(rows, k, n, seed)
    out = torch.full((rows, n), 7.0, device="cuda")
    G.gdn_project_bf16_noalloc(xs, wp, out)
    torch.cuda.synchronize()
    assert torch.equal(out, _with_workspace(xs, wp))


def test_noalloc_shapes_without_workspace_and_too_large():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    # qkv at 64 rows needs no workspace: the plain launch
    x, w, xs, wp = _operands(64, 2560, 10240, 303)
    assert G.gdn_project_workspace_bytes(64, 2560, 10240) == 0
    out = torch.empty(64, 10240, device="cuda")
    G.gdn_project_bf16_noalloc(xs, wp, out)
    torch.cuda.synchronize()
    assert torch.equal(out, _with_workspace(xs, wp))
    # 256 rows x k 8192 x n 2560 needs 10 MiB of partial blocks: more than the buffer
    rows, k, n = 256, 8192, 2560
    assert G.gdn_project_workspace_bytes(rows, k, n) > 4 << 20
    xs = G.gdn_split_bf16(torch.zeros(rows, k, device="cuda"))
    wp = G.gdn_pack_bf16(torch.zeros(n, k, dtype=torch.int16, device="cuda"))
    out = torch.full((rows, n), 7.0, device="cuda")
    with pytest.raises(G.GdnError) as e:
        G.gdn_project_bf16_noalloc(xs, wp, out)
    assert e.value.code == G.GDN_ERR_ARG and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
