"""Parity of the qkv / z / out projections (gdn_split_bf16 + gdn_project_bf16) with the
fp64 oracle on MI355X, through the C ABI.

Tolerance: the one bound of tests/parity.py.  A projection is one step, so its output
is held to tol(1) = 1e-4 x max |ref|; in the chains through the mixer every product
and every mixer token is one more step.  The split of x into bf16 hi + lo keeps each
activation to within 2^-16 |x| and the matrix cores sum in fp32, so the expected error
is near 1e-6 of max |ref|.
"""
import numpy as np
import pytest

import gdn_workloads as W
import oracle
from gpu_harness import GpuMixer, assert_close, assert_tokens, dev, log

pytestmark = pytest.mark.gpu


def _w(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _untile(data, rows, k, parts):
    """The library's tiled layout back to [parts][rows][k] (parts = 2 for split x, 1 for
    packed weights): tile (R, C), fragment (s, p, lane = i + 32h) holds the 8 values
    [32R + i][64C + 32h + 8s + j]."""
    r32, k64 = -(-rows // 32) * 32, -(-k // 64) * 64
    t = data.reshape(r32 // 32, k64 // 64, 4, parts, 2, 32, 8)          # R C s p h i j
    full = t.transpose(3, 0, 5, 1, 4, 2, 6).reshape(parts, r32, k64)   # p (R i) (C h s j)
    return full, full[:, :rows, :k]


def test_split_is_round_to_nearest_and_exact_to_2e16():
    """hi is the round-to-nearest-even bf16 of x (torch's own conversion decides), hi + lo
    equals x to within 2^-16 |x|, and the padding of the tiles is zero."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    rng = np.random.default_rng(90)
    rows, k = 37, 264
    x = (rng.standard_normal((rows, k)) * np.exp(rng.uniform(-20, 20, (rows, k)))).astype(np.float32)
    x[0, :8] = [0.0, -0.0, 1.0, -1.5, 3.3895314e38, -3.3895314e38, 1e-38, 65504.0]
    xd = dev(x)
    xs = G.gdn_split_bf16(xd)
    torch.cuda.synchronize()
    full, parts = _untile(xs.data.cpu().numpy().view(np.uint16), rows, k, 2)
    hi, lo = parts
    assert not full[:, rows:, :].any() and not full[:, :, k:].any()
    ref_hi = xd.to(torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    big = np.abs(x) >= 3.3e38   # values that round up to infinity are truncated instead
    np.testing.assert_array_equal(hi[~big], ref_hi[~big])
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(f(hi) + f(lo) - x.astype(np.float64))
    # relative bound while lo is a normal number; below that the error is under 2^-126
    bound = np.maximum(2.0 ** -16 * np.abs(x.astype(np.float64)), 2.0 ** -126)
    assert (err <= bound).all(), np.argwhere(err > bound)[:5]


def test_pack_is_a_permutation_with_zero_padding():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    n, k = 70, 200
    w = np.random.default_rng(89).integers(0, 1 << 16, (n, k), dtype=np.uint16)
    wp = G.gdn_pack_bf16(_w(w))
    torch.cuda.synchronize()
    full, (back,) = _untile(wp.data.cpu().numpy().view(np.uint16), n, k, 1)
    np.testing.assert_array_equal(back, w)
    assert not full[:, n:, :].any() and not full[:, :, k:].any()


# (rows, k, n): a single row, ragged rows / columns / k, several tiles of each shape, and
# the tile shapes the launch picks by rows, k and n (one or two row tiles per
# workgroup, 1-3 column tiles per wave, k split over 1, 2 or 4 waves, and the
# ring-pipelined LDS form with 1, 2, 3 and 4 chunks, from 1 row up); the two-group LDS
# form, picked only for long k at more than 256 rows, and the k range split over
# workgroups, picked only for long k, have their own tests below
SHAPES = [(1, 64, 32), (3, 72, 40), (33, 136, 100), (64, 2560, 256), (70, 520, 300), (200, 520, 1030),
          (37, 6144, 96), (1, 2560, 10240), (16, 2560, 6144), (300, 128, 4100), (50, 200, 8200),
          (40, 136, 5000), (100, 264, 8300), (150, 136, 4500), (250, 72, 8250), (300, 200, 9000),
          (300, 136, 8200), (600, 64, 8192), (40, 64, 9000), (60, 120, 8300), (45, 136, 8200),
          (1, 200, 12300), (8, 2560, 16384)]


@pytest.mark.parametrize("rows,k,n", SHAPES)
def test_projection_matches_oracle(rows, k, n):
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    log(f"projection rows={rows} k={k} n={n}")
    x, w = W.make_proj(rows, k, n, seed=91 + rows + k + n)
    out = torch.full((rows, n), 7.0, device="cuda")
    G.gdn_project(dev(x), G.gdn_pack_bf16(_w(w)), out)
    torch.cuda.synchronize()
    assert_close("out", out.cpu().numpy(), oracle.project(x, w))


@pytest.mark.parametrize("name", ["qkv", "z", "out"])
def test_projection_full_size_sampled(name):
    """The pages' shapes at a 256-sequence decode batch; rows sampled across every row
    tile (first, last and in between), all n columns of each."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    k, n = W.PROJECTIONS[name]
    rows = 256
    log(f"projection {name} rows={rows} k={k} n={n}")
    x, w = W.make_proj(rows, k, n, seed={"qkv": 95, "z": 96, "out": 97}[name])
    out = G.gdn_project(dev(x), G.gdn_pack_bf16(_w(w)))
    torch.cuda.synchronize()
    pick = np.array([0, 1, 31, 32, 63, 64, 100, 127, 128, 191, 200, 223, 224, 254, 255])
    assert_close(name, out.cpu().numpy()[pick], oracle.project(x[pick], w))


@pytest.mark.parametrize("rows,k", [(512, 2560), (520, 2624)])
def test_projection_lds_form_sampled(rows, k):
    """More than 256 rows with a long k take the LDS-shared two-group tile (an even and an
    odd chunk count, a ragged last row tile); rows sampled across all row tiles."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    n = 10240
    log(f"projection (LDS form) rows={rows} k={k} n={n}")
    x, w = W.make_proj(rows, k, n, seed=110 + k)
    out = G.gdn_project(dev(x), G.gdn_pack_bf16(_w(w)))
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([np.linspace(0, rows - 1, 13).astype(int), [63, 64, 255, 256, rows - 1]]))
    assert_close("out", out.cpu().numpy()[pick], oracle.project(x[pick], w))


@pytest.mark.parametrize("rows,k,n1,n2", [(256, 2560, 10240, 6144), (37, 200, 100, 60), (300, 136, 8192, 40),
                                          (20, 4104, 3000, 1000)])
def test_two_outputs_equal_the_concatenated_projection(rows, k, n1, n2):
    """gdn_project2_bf16 (qkv and z in one launch) writes, column for column, what
    gdn_project_bf16 writes for the concatenated weights, and matches the oracle."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    log(f"two outputs rows={rows} k={k} n1={n1} n2={n2}")
    x, w = W.make_proj(rows, k, n1 + n2, seed=104 + rows)
    wp = G.gdn_pack_bf16(_w(w))
    xs = G.gdn_split_bf16(dev(x))
    o1, o2 = G.gdn_project2_bf16(xs, wp, n1)
    whole = G.gdn_project_bf16(xs, wp)
    torch.cuda.synchronize()
    assert torch.equal(o1, whole[:, :n1]) and torch.equal(o2, whole[:, n1:])
    pick = np.unique(np.linspace(0, rows - 1, 9).astype(int))
    ref = oracle.project(x[pick], w)
    assert_close("out1", o1.cpu().numpy()[pick], ref[:, :n1])
    assert_close("out2", o2.cpu().numpy()[pick], ref[:, n1:])


# (rows, k, n) whose launch splits the k range over 4, 3 or 2 workgroups per tile and
# adds the partial blocks in a second kernel: up to 64 rows with the tile the rules
# pick (one and two row tiles, ragged k, rows and columns), and above 64 rows with
# the 32 x 64 tiles the priced choice splits 4 and 3 ways (ragged rows and columns)
SPLIT_SHAPES = [(1, 6144, 2560), (5, 4104, 1000), (20, 4104, 4000), (50, 4096, 1500), (64, 6144, 4096),
                (70, 6144, 1000), (100, 6144, 1000), (200, 6144, 700)]


@pytest.mark.parametrize("rows,k,n", SPLIT_SHAPES)
def test_projection_split_k_matches_oracle(rows, k, n):
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    assert G.gdn_project_workspace_bytes(rows, k, n) > 0, "the shape no longer splits its k range"
    log(f"projection (k split) rows={rows} k={k} n={n}")
    x, w = W.make_proj(rows, k, n, seed=120 + rows + n)
    out = torch.full((rows, n), 7.0, device="cuda")
    G.gdn_project(dev(x), G.gdn_pack_bf16(_w(w)), out)
    torch.cuda.synchronize()
    assert_close("out", out.cpu().numpy(), oracle.project(x, w))


def test_projection_workspace_is_scratch():
    """A caller's workspace full of NaN gives, bit for bit, what a fresh one gives, and
    one workspace serves two calls in a row, the second with fewer rows."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    k, n = W.PROJECTIONS["out"]
    x, w = W.make_proj(32, k, n, seed=125)
    wp = G.gdn_pack_bf16(_w(w))
    ws = torch.full((G.gdn_project_workspace_bytes(32, k, n) // 4,), float("nan"), device="cuda")
    log(f"workspace of {ws.numel() * 4} bytes")
    ref32 = G.gdn_project(dev(x), wp)
    ref1 = G.gdn_project(dev(x[:1]), wp)
    a = G.gdn_project_bf16(G.gdn_split_bf16(dev(x)), wp, workspace=ws)
    b = G.gdn_project_bf16(G.gdn_split_bf16(dev(x[:1])), wp, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, ref32) and torch.equal(b, ref1)
    assert_close("out", a.cpu().numpy(), oracle.project(x, w))


# the layer input's four projections in one launch (qkv, z, alpha and beta logits) at
# a decode and a single-sequence batch, ragged small outputs, and a k-split launch
MULTI = [(256, 2560, (10240, 6144, 48, 48)), (1, 2560, (10240, 6144, 48, 48)), (37, 200, (100, 60, 7, 9)),
         (20, 4104, (3000, 900, 50, 50)), (5, 72, (40, 24, 8))]


@pytest.mark.parametrize("rows,k,cols", MULTI)
def test_multi_outputs_equal_the_stacked_projection(rows, k, cols):
    """gdn_project_multi_bf16 writes, column for column, what gdn_project_bf16 writes for
    the stacked weights, and matches the oracle (rows sampled at 256)."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    n = sum(cols)
    log(f"multi-output rows={rows} k={k} cols={cols}")
    x, w = W.make_proj(rows, k, n, seed=170 + rows + len(cols))
    wp = G.gdn_pack_bf16(_w(w))
    xs = G.gdn_split_bf16(dev(x))
    outs = G.gdn_project_multi_bf16(xs, wp, cols)
    whole = G.gdn_project_bf16(xs, wp)
    torch.cuda.synchronize()
    pick = np.unique(np.linspace(0, rows - 1, 9).astype(int))
    ref = oracle.project(x[pick], w)
    c0 = 0
    for o, c in zip(outs, cols):
        assert torch.equal(o, whole[:, c0:c0 + c]), f"columns {c0}..{c0 + c} differ"
        assert_close(f"out[{c0}:{c0 + c}]", o.cpu().numpy()[pick], ref[:, c0:c0 + c])
        c0 += c


@pytest.mark.parametrize("rows", [256, 1])
def test_projection_is_deterministic(rows):
    """Same inputs, same bits: the k-split launch (1 row) adds its parts in a fixed order."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    x, w = W.make_proj(rows, 6144, 2560, seed=98)
    xs = G.gdn_split_bf16(dev(x))
    wp = G.gdn_pack_bf16(_w(w))
    a = G.gdn_project_bf16(xs, wp)
    b = G.gdn_project_bf16(xs, wp)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_projection_empty_is_a_no_op():
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    x = torch.empty(0, 2560, device="cuda")
    out = G.gdn_project(x, G.gdn_pack_bf16(torch.zeros(64, 2560, dtype=torch.int16, device="cuda")))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


@pytest.mark.parametrize("B,geom", [(37, W.Geom()), (1, W.Geom()), (64, W.Geom()), (5, W.Geom(h_k=2, h_v=4)),
                                    (33, W.Geom(h_k=1, h_v=14))],
                         ids=lambda v: str(v) if isinstance(v, int) else f"hk{v.h_k}hv{v.h_v}")
def test_single_launch_decode_writes_the_split_of_y(B, geom):
    """gdn_decode_fused with ys writes, bit for bit, what gdn_split_bf16 writes for its y
    (the 32-row padding it leaves alone stays as it was: zero here), with and without
    y, for groups of 3 and 2 value heads per qk head and for the heads-in-turn form."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("ys", B, 1, seed=180 + B, geom=geom, n_slots=B + 3, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    vdim = geom.h_v * geom.s
    log(f"decode with ys B={B} h_k={geom.h_k} h_v={geom.h_v}")
    runs = []
    for with_y in (True, False):
        gm = GpuMixer(wl)
        y = torch.empty(B, vdim, device="cuda") if with_y else None
        ys = G.gdn_split_bf16(torch.zeros(B, vdim, device="cuda"))
        G.gdn_decode_fused(gm.pool, gm.qkv[:, 0].contiguous(), gm.conv_w, gm.alpha[:, 0].contiguous(),
                           gm.beta_logit[:, 0].contiguous(), gm.dt, gm.ssm_a, gm.z[:, 0].contiguous(), gm.norm_w,
                           wl.eps, y, None, gm.slots, ys=ys)
        runs.append((gm, y, ys))
    (ga, y, ys), (gb, _, ys_noy) = runs
    ref = G.gdn_split_bf16(y)
    torch.cuda.synchronize()
    assert y.abs().max().item() > 0
    assert torch.equal(ys.data, ref.data), "the fused split differs from gdn_split_bf16(y)"
    assert torch.equal(ys_noy.data, ys.data), "without y the split differs"
    assert torch.equal(ga.pool.state, gb.pool.state) and torch.equal(ga.pool.conv, gb.pool.conv)


def test_single_launch_decode_split_of_y_for_an_unknown_slot():
    """A sequence whose slot is unknown gets zero fragments; the others get the split of
    their y."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    wl = W.make("ys-bad", 3, 1, seed=185, n_slots=4, state_std=0.02, conv_std=1.0)
    gm = GpuMixer(wl)
    vdim = wl.geom.value_dim
    y = torch.empty(3, vdim, device="cuda")
    ys = G.gdn_split_bf16(torch.full((3, vdim), 5.0, device="cuda"))
    G.gdn_decode_fused(gm.pool, gm.qkv[:, 0].contiguous(), gm.conv_w, gm.alpha[:, 0].contiguous(),
                       gm.beta_logit[:, 0].contiguous(), gm.dt, gm.ssm_a, gm.z[:, 0].contiguous(), gm.norm_w,
                       wl.eps, y, None, dev(np.array([2, 9, 0], np.int32)), ys=ys)
    ref = G.gdn_split_bf16(y)
    torch.cuda.synchronize()
    _, got = _untile(ys.data.cpu().numpy().view(np.uint16), 3, vdim, 2)
    _, want = _untile(ref.data.cpu().numpy().view(np.uint16), 3, vdim, 2)
    assert not got[:, 1].any(), "the unknown slot's fragments are not zero"
    np.testing.assert_array_equal(got[:, [0, 2]], want[:, [0, 2]])


def test_projections_around_the_mixer():
    """x -> qkv, z, alpha, beta projections -> mixer -> out projection, against the
    oracle's projections and mixer on the same x (small geometry, 3 tokens)."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    geom = W.Geom(h_k=2, h_v=4)
    B, T, n_embd = 5, 3, 256
    wl = W.make("layer", B, T, seed=99, geom=geom, state_std=0.02, conv_std=1.0)
    xq, wqkv = W.make_proj(B * T, n_embd, geom.channels, seed=100)
    _, wgate = W.make_proj(1, n_embd, geom.value_dim, seed=101)
    _, wout = W.make_proj(1, geom.value_dim, n_embd, seed=102)
    ab = W.make_ab(B, T, seed=103, n_embd=n_embd, h_v=geom.h_v)
    ab.x = xq.reshape(B, T, n_embd)
    # the oracle's chain
    wl.qkv = oracle.project(xq, wqkv).reshape(B, T, -1).astype(np.float32)
    wl.z = oracle.project(xq, wgate).reshape(B, T, -1).astype(np.float32)
    ra, rb = oracle.ab_project(ab.x, ab.w_alpha, ab.w_beta)
    wl.alpha, wl.beta_logit = ra.astype(np.float32), rb.astype(np.float32)
    res = oracle.run_workload(wl)
    y_ref = np.stack([r["y"] for r in res])
    out_ref = oracle.project(y_ref.reshape(B * T, -1), wout)
    # the HIP chain
    gm = GpuMixer(wl)
    xs = G.gdn_split_bf16(dev(xq))
    # qkv and z in one launch over the concatenated weights
    wqkvz = G.gdn_pack_bf16(_w(np.concatenate([wqkv, wgate])))
    G.gdn_project2_bf16(xs, wqkvz, geom.channels, gm.qkv.view(B * T, -1), gm.z.view(B * T, -1))
    G.gdn_ab_project(dev(ab.x), _w(ab.w_alpha), _w(ab.w_beta), gm.alpha, gm.beta_logit)
    gm.run(fused=True)
    out = G.gdn_project(gm.y.view(B * T, -1), G.gdn_pack_bf16(_w(wout)))
    torch.cuda.synchronize()
    # qkv, z, alpha and beta come out of one product each: token t of y is t + 2 steps
    # from x, and the out projection adds one more
    assert_tokens("y", gm.y.cpu().numpy(), list(y_ref), [T] * B, first_step=2)
    assert_tokens("out", out.cpu().numpy().reshape(B, T, -1), list(out_ref.reshape(B, T, -1)), [T] * B,
                  first_step=3)


def test_four_launch_layer_decode_matches_the_oracle():
    """One decode token of a layer in 4 launches: split x -> qkv, z, alpha and beta logits
    in one launch -> the single-launch mixer writing y already split -> out projection,
    against the oracle's projections, mixer and out projection on the same x (a decode
    batch of 37 sequences, the model's geometry, random slots)."""
    import torch
    import gated_deltanet_mixer_gdn_amd as G
    geom = W.Geom()
    B, n_embd = 37, 2560
    wl = W.make("layer4", B, 1, seed=190, geom=geom, n_slots=48, state_std=0.02, conv_std=1.0,
                slot_choice="random")
    x, wqkv = W.make_proj(B, n_embd, geom.channels, seed=191)
    _, wgate = W.make_proj(1, n_embd, geom.value_dim, seed=192)
    _, wab = W.make_proj(1, n_embd, 2 * geom.h_v, seed=193)
    _, wout = W.make_proj(1, geom.value_dim, n_embd, seed=194)
    # the oracle's chain
    wl.qkv = oracle.project(x, wqkv).reshape(B, 1, -1).astype(np.float32)
    wl.z = oracle.project(x, wgate).reshape(B, 1, -1).astype(np.float32)
    ab = oracle.project(x, wab)
    wl.alpha = ab[:, :geom.h_v].reshape(B, 1, -1).astype(np.float32)
    wl.beta_logit = ab[:, geom.h_v:].reshape(B, 1, -1).astype(np.float32)
    res = oracle.run_workload(wl)
    y_ref = np.stack([r["y"] for r in res]).reshape(B, -1)
    out_ref = oracle.project(y_ref, wout)
    # the HIP chain
    gm = GpuMixer(wl)
    wp_in = G.gdn_pack_bf16(_w(np.concatenate([wqkv, wgate, wab])))
    wp_out = G.gdn_pack_bf16(_w(wout))
    xs = G.gdn_split_bf16(dev(x))
    qkv, z, alpha, beta = G.gdn_project_multi_bf16(xs, wp_in, (geom.channels, geom.value_dim, geom.h_v, geom.h_v))
    ys = G.gdn_split_bf16(torch.zeros(B, geom.value_dim, device="cuda"))
    G.gdn_decode_fused(gm.pool, qkv, gm.conv_w, alpha, beta, gm.dt, gm.ssm_a, z, gm.norm_w, wl.eps, None,
                       None, gm.slots, ys=ys)
    out = G.gdn_project_bf16(ys, wp_out)
    torch.cuda.synchronize()
    # x -> projections (1) -> one mixer token (2) -> out projection (3)
    assert_close("out", out.cpu().numpy(), out_ref, 3)
    for b in range(B):
        slot = int(wl.slots[b])
        assert_close(f"state[{b}]", gm.pool.state[slot].cpu().numpy(), res[b]["state"], 2)
