"""The hot path under HIP-graph capture, through the C ABI: the single-launch decode,
conv + the multi-token recurrence with device-resident slots and ragged token counts,
and the out projection with its k range split over workgroups (workspace passed in).

Each graph is replayed several times with new inputs copied into its buffers, with
eager work and a synchronisation between replays, and every replay is compared bit
for bit with the same calls made eagerly on a second pool that started from the same
state (the same kernels on the same inputs give the same bits).  None of these calls
records a memset or allocates, and the slot lists and token counts are read on the
device, so a captured step needs nothing from the host at replay time.
"""
import numpy as np
import pytest

import gdn_workloads as W
from gpu_harness import GpuMixer, dev, log

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _restore(gm, wl):
    gm.pool.state.copy_(dev(wl.state))
    gm.pool.conv.copy_(dev(wl.conv_state))


def test_graph_replays_single_launch_decode():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    B = 6
    wl = W.make("graph_decode", B, REPLAYS, seed=141, n_slots=16, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    g = wl.geom
    eager, graph = GpuMixer(wl), GpuMixer(wl)
    qkv = torch.zeros(B, g.channels, device="cuda")
    alpha = torch.zeros(B, g.h_v, device="cuda")
    beta_logit = torch.zeros(B, g.h_v, device="cuda")
    z = torch.zeros(B, g.value_dim, device="cuda")
    y = torch.empty(B, g.value_dim, device="cuda")

    def step():
        G.gdn_decode_fused(graph.pool, qkv, graph.conv_w, alpha, beta_logit, graph.dt, graph.ssm_a, z,
                           graph.norm_w, wl.eps, y, None, graph.slots)
    step()                      # first launch outside the capture, then back to the start state
    _restore(graph, wl)
    torch.cuda.synchronize()
    cg = _capture(step)
    state0 = eager.pool.state.clone()
    for t in range(REPLAYS):
        log(f"decode replay {t}")
        qkv.copy_(eager.qkv[:, t])
        alpha.copy_(eager.alpha[:, t])
        beta_logit.copy_(eager.beta_logit[:, t])
        z.copy_(eager.z[:, t])
        cg.replay()
        y_e = torch.empty_like(y)
        G.gdn_decode_fused(eager.pool, eager.qkv[:, t].contiguous(), eager.conv_w, eager.alpha[:, t].contiguous(),
                           eager.beta_logit[:, t].contiguous(), eager.dt, eager.ssm_a, eager.z[:, t].contiguous(),
                           eager.norm_w, wl.eps, y_e, None, eager.slots)
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {t}: y differs"
        assert torch.equal(graph.pool.state, eager.pool.state), f"replay {t}: state differs"
        assert torch.equal(graph.pool.conv, eager.pool.conv), f"replay {t}: conv history differs"
    assert not torch.equal(eager.pool.state, state0)


def test_graph_replays_ragged_multi_token_step():
    """conv + recurrence with the fused norm over T = 4 tokens, with a new set of
    per-sequence token counts (a device tensor the graph reads) on every replay."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    B, T = 5, 4
    wl = W.make("graph_multi", B, T, seed=142, n_slots=12, state_std=0.02, conv_std=1.0,
                slot_choice="random", ragged_max=T)
    g = wl.geom
    eager, graph = GpuMixer(wl), GpuMixer(wl)
    qkv = torch.zeros(B, T, g.channels, device="cuda")
    alpha = torch.zeros(B, T, g.h_v, device="cuda")
    beta_logit = torch.zeros(B, T, g.h_v, device="cuda")
    z = torch.zeros(B, T, g.value_dim, device="cuda")
    n_tok = torch.ones(B, dtype=torch.int32, device="cuda")
    h = torch.empty(B, T, g.channels, device="cuda")
    y = torch.empty(B, T, g.value_dim, device="cuda")

    def step():
        G.gdn_mixer(graph.pool, qkv, alpha, beta_logit, z, graph.conv_w, graph.dt, graph.ssm_a, graph.norm_w,
                    wl.eps, h, None, y, graph.slots, n_tok, fused=True)
    step()
    _restore(graph, wl)
    torch.cuda.synchronize()
    cg = _capture(step)
    for r in range(REPLAYS):
        inp = W.make("graph_multi_in", B, T, seed=150 + r, n_slots=12, ragged_max=T)
        log(f"multi-token replay {r}: n_tok {inp.n_tok.tolist()}")
        qkv.copy_(dev(inp.qkv))
        alpha.copy_(dev(inp.alpha))
        beta_logit.copy_(dev(inp.beta_logit))
        z.copy_(dev(inp.z))
        n_tok.copy_(dev(inp.n_tok))
        cg.replay()
        h_e = torch.empty_like(h)
        y_e = torch.empty_like(y)
        G.gdn_mixer(eager.pool, dev(inp.qkv), dev(inp.alpha), dev(inp.beta_logit), dev(inp.z), eager.conv_w,
                    eager.dt, eager.ssm_a, eager.norm_w, wl.eps, h_e, None, y_e, eager.slots, dev(inp.n_tok),
                    fused=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {r}: y differs"
        assert torch.equal(h, h_e), f"replay {r}: h differs"
        assert torch.equal(graph.pool.state, eager.pool.state), f"replay {r}: state differs"
        assert torch.equal(graph.pool.conv, eager.pool.conv), f"replay {r}: conv history differs"


def test_graph_replays_split_k_projection():
    """split of y + the out projection at one row, whose launch splits k 3 ways and adds
    the parts in a second kernel through the caller's workspace."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    k, n = W.PROJECTIONS["out"]
    rows = 1
    need = G.gdn_project_workspace_bytes(rows, k, n)
    assert need > 0, "the shape no longer splits its k range"
    _, w = W.make_proj(rows, k, n, seed=143)
    wp = G.gdn_pack_bf16(torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).cuda())
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x = torch.zeros(rows, k, device="cuda")
    xs = G.gdn_split_bf16(x)
    out = torch.empty(rows, n, device="cuda")

    def step():
        G.gdn_split_bf16(x, xs)
        G.gdn_project_bf16(xs, wp, out, workspace=ws)
    step()
    torch.cuda.synchronize()
    cg = _capture(step)
    for r in range(REPLAYS):
        log(f"projection replay {r}")
        xr, _ = W.make_proj(rows, k, 8, seed=160 + r)
        x.copy_(dev(xr))
        cg.replay()
        ref = G.gdn_project(dev(xr), wp)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}: out differs"
        assert out.abs().max().item() > 0


def test_graph_replays_commit_window():
    """gdn_commit_window (the conv launch with the history advance, then the round
    launch) captured once and replayed over several rounds: each replay commits a new
    window (run eagerly on each pool, so both pools hold the same window h) with new
    device-resident n_keep and window token counts, and is compared bit for bit with
    the eager call on the second pool."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    B, T0, T1 = 4, 3, 5
    wl = W.make("graph_round", B, T1, seed=144, n_slots=10, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    g = wl.geom
    eager, graph = GpuMixer(wl), GpuMixer(wl)
    prev = [torch.zeros(B, T0, n, device="cuda") for n in (g.channels, g.channels, g.h_v, g.h_v)]
    z0 = torch.zeros(B, T0, g.value_dim, device="cuda")
    y0 = torch.empty(B, T0, g.value_dim, device="cuda")
    n_keep = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_tok = torch.ones(B, dtype=torch.int32, device="cuda")
    qkv, alpha, beta_logit, z = (torch.zeros(B, T1, n, device="cuda")
                                 for n in (g.channels, g.h_v, g.h_v, g.value_dim))
    h = torch.empty(B, T1, g.channels, device="cuda")
    y = torch.empty(B, T1, g.value_dim, device="cuda")

    def window0(gm):
        G.gdn_verify_window(gm.pool, prev[0], gm.conv_w, prev[2], prev[3], gm.dt, gm.ssm_a, z0, gm.norm_w, wl.eps,
                            prev[1], y0, gm.slots)

    def step(gm, hh, yy):
        G.gdn_commit_window(gm.pool, tuple(prev), n_keep, qkv, gm.conv_w, alpha, beta_logit, gm.dt, gm.ssm_a, z,
                            gm.norm_w, wl.eps, hh, yy, gm.slots, n_tok)
    step(graph, h, y)
    _restore(graph, wl)
    torch.cuda.synchronize()
    cg = _capture(lambda: step(graph, h, y))
    for r in range(REPLAYS):
        w0 = W.make("graph_round_prev", B, T0, seed=170 + r, n_slots=10, ragged_max=T0)
        w1 = W.make("graph_round_next", B, T1, seed=180 + r, n_slots=10, ragged_max=T1)
        keep = np.random.default_rng(190 + r).integers(0, T0 + 1, B).astype(np.int32)
        log(f"round replay {r}: n_keep {keep.tolist()} n_tok {w1.n_tok.tolist()}")
        for t, a in zip(prev, (w0.qkv, None, w0.alpha, w0.beta_logit)):
            if a is not None:
                t.copy_(dev(a))
        z0.copy_(dev(w0.z))
        n_keep.copy_(dev(keep))
        for t, a in zip((qkv, alpha, beta_logit, z, n_tok), (w1.qkv, w1.alpha, w1.beta_logit, w1.z, w1.n_tok)):
            t.copy_(dev(a))
        window0(graph)                    # h of the window being committed, from the graph pool
        cg.replay()
        window0(eager)                    # the same from the eager pool (same state, same bits)
        h_e, y_e = torch.empty_like(h), torch.empty_like(y)
        step(eager, h_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y, y_e), f"replay {r}: y differs"
        assert torch.equal(h, h_e), f"replay {r}: h differs"
        assert torch.equal(graph.pool.state, eager.pool.state), f"replay {r}: state differs"
        assert torch.equal(graph.pool.conv, eager.pool.conv), f"replay {r}: conv history differs"
