#!/usr/bin/env python3
"""Benchmark of the GDN decode mixer on one MI355X.

A step is one pass of the whole mixer (conv/SiLU/L2 -> gated delta rule -> gated
RMSNorm) over one batch: by default the bandwidth-bound decode of 256 sequences x
1 token (768 MiB of fp32 state), inputs already in HBM.  For one token per
sequence the timed step is the single launch gdn_decode_fused (conv, recurrence
and gated RMSNorm, writing y only), the fastest form; the two-launch form
(gdn_conv_silu_norm + gdn_decode_step_norm) and the three-call form are timed
beside it for context.  Workloads with several tokens per sequence time the
two-launch form.  Prints ONE JSON line on stdout; diagnostics go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config b256]
                  [--cpu-seconds S | --no-cpu-baseline] [--copy-probe-mib M]

The `roofline` object is for the dominant kernel of the timed step
(decode_fused_par_kernel<3> for the default workload): its algorithmic bytes per
launch over its average launch time, measured with HIP events recorded on the
stream the kernels run on: one pair around all timed launches when the step is that
one kernel, else around the kernels of every 8th step of the timed region.  `traffic` (HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
counters, scaled by a copy-kernel calibration) is read from
profiles/decode_fused_b256_traffic.txt and reported only while the kernel sources
it was measured on are unchanged.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E, published peak
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 matrix peak, published
# fp32 VALU without packed instructions (the library is compiled with them off):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz
VALU_PEAK_TFLOPS = 78.6
FLOP_PER_SEQ_HEAD_STEP = 7 * 128 * 128   # per state element: S^T k FMA, S^T q FMA, decay multiply, update FMA
# the sources the recurrence kernel is built from (its counter record is void once they change)
KERNEL_SRCS = [os.path.join(ROOT, "gated_deltanet_mixer_gdn_amd", "csrc", f)
               for f in ("gdn_recurrence.hip", "gdn_device.h", "gdn_kernels.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_fused_b256_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic():
    """(bytes per launch, note) if the committed counter summary matches this kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(wl):
    """Bytes each kernel must move at minimum (inputs read once, outputs written once).
    "step" is the recurrence writing o; "step_norm" the recurrence with the gated RMSNorm
    fused in, reading z and writing y only."""
    g = wl.geom
    C, S, hv = g.channels, g.s, g.h_v
    tok = int(wl.B * wl.T if wl.n_tok is None else wl.n_tok.sum())
    seqs = int(wl.B if wl.n_tok is None else (wl.n_tok > 0).sum())
    all_tok = wl.B * wl.T
    row = hv * S * 4                           # one token's o, z or y
    conv = tok * C * 4 + all_tok * C * 4 + seqs * C * (g.d_conv - 1) * 4 * 2 + C * g.d_conv * 4
    core = (seqs * hv * S * S * 4 * 2          # state read + write, once per call
            + tok * (C * 4 + 2 * hv * 4)       # h (q|k|v) and alpha / beta logits of each token
            + 2 * hv * 4)                      # dt, ssm_a
    step_norm = core + tok * row + all_tok * row + S * 4                  # z in, y out
    return {"conv": conv,
            "step": core + all_tok * row,                                  # o
            "norm": all_tok * row * 3 + S * 4,                             # o, z in; y out; weight
            "step_norm": step_norm,
            # single launch: conv without the h write, recurrence without the h read
            "one": conv - all_tok * C * 4 + step_norm - tok * C * 4}, tok * hv


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle, as it stands, on the host cores: whole batches of the same
    workload, repeated until `seconds` of wall time have passed."""
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    oracle.lib()
    units = sum(wl.tokens_of(b) for b in range(wl.B)) * wl.geom.h_v
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.run_workload(wl, threads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": units * reps / el, "unit": "seq-head-steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full passes of the {wl.name} workload ({units} seq-head-steps each, "
                      f"all {wl.B} sequences), fp64 C oracle, {cores} threads, {el:.1f} s"}


def copy_probe(mib: int, reps: int = 5):
    """A plain device copy of known size, for calibrating HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "reps": reps}))


def _card_dir():
    """sysfs directory of the amdgpu card that device 0 of this process is, matched by
    its PCI address, or None."""
    import glob
    import torch
    pr = torch.cuda.get_device_properties(0)
    try:
        want = "%04x:%02x:%02x." % (pr.pci_domain_id, pr.pci_bus_id, pr.pci_device_id)
    except AttributeError:
        return None
    for card in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if os.path.basename(os.path.realpath(card)).startswith(want):
            return card
    return None


def gpu_clocks(card):
    """The card's current shader and memory clock levels in MHz, read from the amdgpu
    driver's pp_dpm_sclk / pp_dpm_mclk files (the level marked '*'); None where they
    cannot be read.  A file read, so it is safe in any process (no child program)."""
    if card is None:
        return None
    out = {}
    for key, name in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
        try:
            with open(os.path.join(card, name)) as f:
                lines = f.read().splitlines()
        except OSError:
            continue
        cur = [ln for ln in lines if ln.rstrip().endswith("*")]
        m = re.search(r"(\d+)\s*mhz", cur[0], re.I) if cur else None
        if m:
            out[key] = int(m.group(1))
    return out or None


def projections_context(G, W, rows: int, stream, reps: int = 50):
    """Time the split of x, qkv + z in one launch, the split of y and the out projection
    at the pages' sizes; algorithmic flops are 2 * rows * k * n per projection."""
    import numpy as np
    import torch
    k_in, n_qkv = W.PROJECTIONS["qkv"]
    _, n_z = W.PROJECTIONS["z"]
    k_out, n_out = W.PROJECTIONS["out"]
    x, w_qkvz = W.make_proj(rows, k_in, n_qkv + n_z, seed=12)
    y, w_out = W.make_proj(rows, k_out, n_out, seed=13)
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    wp_qkvz, wp_out = G.gdn_pack_bf16(dev16(w_qkvz)), G.gdn_pack_bf16(dev16(w_out))
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    xs, ys = G.gdn_split_bf16(xd), G.gdn_split_bf16(yd)
    qkv, z = torch.empty(rows, n_qkv, device="cuda"), torch.empty(rows, n_z, device="cuda")
    out = torch.empty(rows, n_out, device="cuda")
    calls = {
        "split_x": lambda: G.gdn_split_bf16(xd, xs),
        "qkv_z": lambda: G.gdn_project2_bf16(xs, wp_qkvz, n_qkv, qkv, z),
        "split_y": lambda: G.gdn_split_bf16(yd, ys),
        "out": lambda: G.gdn_project_bf16(ys, wp_out, out),
    }
    us = {}
    for name, fn in calls.items():
        for _ in range(5):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        us[name] = ev[0].elapsed_time(ev[1]) / reps * 1000.0
    flops = {"qkv_z": 2.0 * rows * k_in * (n_qkv + n_z), "out": 2.0 * rows * k_out * n_out}
    tflops = {kname: flops[kname] / us[kname] / 1e6 for kname in flops}
    total_us = sum(us.values())
    log("projections: " + ", ".join(f"{kname}={v:.1f}us" for kname, v in us.items()) +
        f"; qkv+z {tflops['qkv_z']:.0f} TFLOP/s, out {tflops['out']:.0f} TFLOP/s")
    return {"rows": rows, "us": us, "us_total": total_us, "algorithmic_flops": flops, "tflops": tflops,
            "frac_of_bf16_peak": {kname: v / BF16_PEAK_TFLOPS for kname, v in tflops.items()},
            "note": "fp32 activations as bf16 hi+lo: two bf16 matrix ops per multiply-add"}


def layer_decode(G, batches, reps: int = 50):
    """One decode token of a whole GDN layer, x [B][n_embd] -> out [B][n_embd]: split of x,
    qkv, z and the alpha / beta logits in one launch, the single-launch mixer writing y
    already split for the out projection, and the out projection (4 launches),
    captured in a HIP graph and replayed (so the host's launch cost is not in it), at
    each batch size; plus each call timed eagerly with events, the 5-launch form
    (alpha / beta projection as a launch of its own, better from 64 rows) and the
    6-launch form (the split of y as a launch of its own too).  Seeded
    random weights (bf16) and inputs; one JSON line per batch size."""
    import torch
    n_embd, n_qkv, n_z = 2560, 10240, 6144
    geom = G.Geom()
    hv, s_ = geom.h_v, geom.s
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    rnd = lambda *shape, std=1.0: torch.randn(*shape, generator=gen, device="cuda") * std
    bf16 = lambda t: t.to(torch.bfloat16).view(torch.int16).contiguous()
    w_qkvz = bf16(rnd(n_qkv + n_z, n_embd, std=n_embd ** -0.5))
    w_alpha, w_beta = bf16(rnd(hv, n_embd, std=n_embd ** -0.5)), bf16(rnd(hv, n_embd, std=n_embd ** -0.5))
    wp_qkvz = G.gdn_pack_bf16(w_qkvz)
    wp_in = G.gdn_pack_bf16(torch.cat([w_qkvz, w_alpha, w_beta]).contiguous())
    cols_in = (n_qkv, n_z, hv, hv)
    wp_out = G.gdn_pack_bf16(bf16(rnd(n_embd, n_z, std=n_z ** -0.5)))
    conv_w, dt, norm_w = rnd(n_qkv, geom.d_conv, std=0.5), rnd(hv, std=0.5), 1.0 + rnd(s_, std=0.1)
    ssm_a = -torch.exp(torch.rand(hv, generator=gen, device="cuda") * 2.0 - 1.0)
    weight_bytes = (n_qkv + n_z) * n_embd * 2 + 2 * hv * n_embd * 2 + n_embd * n_z * 2
    for B in batches:
        pool = G.StatePool(B, geom)
        pool.state.copy_(rnd(*pool.state.shape, std=0.02))
        pool.conv.copy_(rnd(*pool.conv.shape))
        x = rnd(B, n_embd)
        xs = G.gdn_split_bf16(x)
        qkv, z = torch.empty(B, n_qkv, device="cuda"), torch.empty(B, n_z, device="cuda")
        alpha, beta_logit = torch.empty(B, hv, device="cuda"), torch.empty(B, hv, device="cuda")
        y, out = torch.empty(B, n_z, device="cuda"), torch.empty(B, n_embd, device="cuda")
        ys = G.gdn_split_bf16(y.zero_())
        ws = torch.empty(max(G.gdn_project_workspace_bytes(B, n_z, n_embd), 16), dtype=torch.uint8,
                         device="cuda")
        calls = {
            "split_x": lambda: G.gdn_split_bf16(x, xs),
            "qkv_z_alpha_beta": lambda: G.gdn_project_multi_bf16(xs, wp_in, cols_in, (qkv, z, alpha, beta_logit),
                                                                 workspace=ws),
            "mixer_ys": lambda: G.gdn_decode_fused(pool, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z, norm_w,
                                                   1e-6, None, ys=ys),
            "out": lambda: G.gdn_project_bf16(ys, wp_out, out, workspace=ws),
        }
        separate_ab = {"split_x": calls["split_x"],
                       "qkv_z": lambda: G.gdn_project2_bf16(xs, wp_qkvz, n_qkv, qkv, z, workspace=ws),
                       "alpha_beta": lambda: G.gdn_ab_project(x, w_alpha, w_beta, alpha, beta_logit),
                       "mixer": lambda: G.gdn_decode_fused(pool, qkv, conv_w, alpha, beta_logit, dt, ssm_a, z,
                                                           norm_w, 1e-6, y),
                       "split_y": lambda: G.gdn_split_bf16(y, ys),
                       "out": calls["out"]}
        eager = {}
        for name, fn in {**calls, **separate_ab}.items():
            for _ in range(3):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(reps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            eager[name] = ev[0].elapsed_time(ev[1]) / reps * 1000.0
        def graph_us(fns):
            step = lambda: [fn() for fn in fns.values()]
            step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            graph.replay()
            torch.cuda.synchronize()
            best = None
            for _ in range(5):
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record()
                for _ in range(reps):
                    graph.replay()
                ev[1].record()
                torch.cuda.synchronize()
                us = ev[0].elapsed_time(ev[1]) / reps * 1000.0
                best = us if best is None else min(best, us)
            return best
        five = {"split_x": calls["split_x"], "qkv_z": separate_ab["qkv_z"], "alpha_beta": separate_ab["alpha_beta"],
                "mixer_ys": calls["mixer_ys"], "out": calls["out"]}
        best = graph_us(calls)
        best_five = graph_us(five)
        best_separate = graph_us(separate_ab)   # 6 launches
        state_bytes = 2 * B * hv * s_ * s_ * 4
        print(json.dumps({"layer_decode": {
            "B": B, "graph_us_per_token": best, "graph_us_five_launches": best_five,
            "graph_us_six_launches": best_separate,
            "eager_us": eager,
            "weight_bytes": weight_bytes, "state_bytes_read_written": state_bytes,
            "gbps_weights_and_state": (weight_bytes + state_bytes) / best / 1e3,
            "note": "seeded random bf16 weights and fp32 inputs; n_embd 2560, h_k 16, h_v 48, S 128"}}),
            flush=True)
        del pool


def small_batches(G, batches, reps: int = 200):
    """One decode token at each batch size, in the single launch and in the two launches
    (conv, then the recurrence with the fused norm), each call repeated `reps` times
    back to back.  Seeded random inputs of the decode shapes.  At small batches an eager
    call costs more host time than kernel time, so the per-call event figure printed
    here is host-bound; the kernel durations come from a rocprofv3 kernel trace of
    this run, grouped by grid size."""
    import torch
    geom = G.Geom()
    C, hv, vd = geom.channels, geom.h_v, geom.h_v * geom.s
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    rnd = lambda *shape, std=1.0: torch.randn(*shape, generator=gen, device="cuda") * std
    conv_w, dt, norm_w = rnd(C, geom.d_conv, std=0.5), rnd(hv, std=0.5), 1.0 + rnd(geom.s, std=0.1)
    ssm_a = -torch.exp(torch.rand(hv, generator=gen, device="cuda") * 2.0 - 1.0)
    for B in batches:
        pool = G.StatePool(B, geom)
        pool.state.copy_(rnd(*pool.state.shape, std=0.02))
        pool.conv.copy_(rnd(*pool.conv.shape))
        pool.flags.zero_()
        qkv, alpha, bl, z = rnd(B, 1, C), rnd(B, 1, hv), rnd(B, 1, hv), rnd(B, 1, vd)
        h, y = torch.empty(B, 1, C, device="cuda"), torch.empty(B, 1, vd, device="cuda")
        forms = {
            "single_launch": lambda: G.gdn_decode_fused(pool, qkv[:, 0], conv_w, alpha[:, 0], bl[:, 0], dt, ssm_a,
                                                        z[:, 0], norm_w, 1e-6, y[:, 0]),
            "two_launches": lambda: G.gdn_mixer(pool, qkv, alpha, bl, z, conv_w, dt, ssm_a, norm_w, 1e-6, h, None, y,
                                                fused=True),
        }
        out = {"B": B}
        for name, fn in forms.items():
            fn()
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(reps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            out[f"{name}_us_per_call_eager"] = ev[0].elapsed_time(ev[1]) / reps * 1000.0
        print(json.dumps({"small_batch_decode": out}), flush=True)
        del pool


def verify_round(G, W, B: int, T: int, reps: int = 20):
    """One speculative round at batch B: gdn_verify_window over T drafted tokens from the
    untouched pool (writes h and y, persists nothing), then gdn_commit of n_keep ~
    U{1..T} tokens per sequence (conv history and state advance).  Seeded synthetic
    inputs of the decode shapes; one JSON line with the two calls' event-timed mean
    durations and algorithmic bytes.  The window's h between its two kernels is not
    counted (the decode step's accounting); the commit reads it as an input.  Also
    timed: gdn_commit_window, the commit of one window fused with the next window (a
    second set of window buffers), which reads each state tile and history once."""
    import numpy as np
    import torch
    wl = W.make(f"verify_b{B}_t{T}", B, T, seed=31, state_std=0.02, conv_std=1.0)
    g = wl.geom
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pool = G.StatePool(wl.n_slots)
    pool.state.copy_(dev(wl.state))
    pool.conv.copy_(dev(wl.conv_state))
    pool.flags.zero_()
    n_keep_h = np.random.default_rng(32).integers(1, T + 1, B).astype(np.int32)
    qkv, alpha, bl, z = dev(wl.qkv), dev(wl.alpha), dev(wl.beta_logit), dev(wl.z)
    conv_w, dt, ssm_a, norm_w = dev(wl.conv_w), dev(wl.dt), dev(wl.ssm_a), dev(wl.norm_w)
    n_keep = dev(n_keep_h)
    h = torch.empty(B, T, g.channels, device="cuda")
    y = torch.empty(B, T, g.value_dim, device="cuda")
    window = lambda: G.gdn_verify_window(pool, qkv, conv_w, alpha, bl, dt, ssm_a, z, norm_w, wl.eps, h, y)
    commit = lambda: G.gdn_commit(pool, qkv, h, alpha, bl, dt, ssm_a, n_keep)
    qkv2, alpha2, bl2, z2 = qkv.clone(), alpha.clone(), bl.clone(), z.clone()
    h2, y2 = torch.empty_like(h), torch.empty_like(y)
    fused = lambda: G.gdn_commit_window(pool, (qkv, h, alpha, bl), n_keep, qkv2, conv_w, alpha2, bl2, dt, ssm_a,
                                        z2, norm_w, wl.eps, h2, y2)

    def mean_us(fn):
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps * 1000.0
    window()
    win_us = mean_us(window)
    com_us = mean_us(commit)
    fused_us = mean_us(fused)
    C, V, hv = g.channels, g.value_dim, g.h_v
    state = B * hv * g.s * g.s * 4
    hist = B * C * (g.d_conv - 1) * 4
    kept = int(n_keep_h.sum())
    adv = int(np.minimum(n_keep_h, g.d_conv - 1).sum())    # raw rows that end up in the history
    win_bytes = B * T * C * 4 + hist + state + 2 * B * T * V * 4 + 2 * B * T * hv * 4 + C * g.d_conv * 4
    com_bytes = 2 * hist + adv * C * 4 + 2 * state + kept * C * 4 + 2 * kept * hv * 4 + C * g.d_conv * 4
    fused_bytes = win_bytes + com_bytes - state - hist   # one state read and one history read fewer
    print(json.dumps({"verify_round": {
        "B": B, "T": T, "tokens_kept": kept, "history_rows_read": adv, "window_us": win_us, "commit_us": com_us,
        "round_us": win_us + com_us,
        "window_gbps": win_bytes / win_us / 1e3, "commit_gbps": com_bytes / com_us / 1e3,
        "round_gbps": (win_bytes + com_bytes) / (win_us + com_us) / 1e3,
        "frac_of_hbm_peak": (win_bytes + com_bytes) / (win_us + com_us) / 1e3 / HBM_PEAK_GBPS,
        "window_bytes": win_bytes, "commit_bytes": com_bytes,
        "commit_window_us": fused_us, "commit_window_bytes": fused_bytes,
        "commit_window_gbps": fused_bytes / fused_us / 1e3,
        "commit_window_frac_of_hbm_peak": fused_bytes / fused_us / 1e3 / HBM_PEAK_GBPS,
        "note": "seeded synthetic inputs of the decode shapes; n_keep ~ U{1..T}; event-timed means"}}),
        flush=True)


def _algorithmic(geom, B, T, n_tok=None):
    """algorithmic_bytes for a batch described by its shape alone."""
    from types import SimpleNamespace
    return algorithmic_bytes(SimpleNamespace(geom=geom, B=B, T=T, n_tok=n_tok))


def _event_span(stream, fn, reps):
    """Mean microseconds of fn over reps calls, one HIP event pair on the launch stream
    around all of them (the calls are queued back to back)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps * 1000.0


def _kernel_events(stream, launches, reps):
    """Mean microseconds of each launch of a several-launch step, each bracketed by its
    own HIP event pair on every one of reps steps (an event record costs a few
    microseconds, under 1% of the kernels timed this way)."""
    import numpy as np
    import torch
    names = list(launches)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    for e in evs:
        e[0].record(stream)
        for i, name in enumerate(names):
            launches[name]()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    return {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1000.0
            for i, name in enumerate(names)}


def config_blocks(G, W, stream, steps: int, warmup: int):
    """Every workload of the mixer at one GPU, timed on inputs drawn on the device with
    the workloads' distributions (seeded torch generator; the ragged slot list and token
    counts from a seeded numpy generator): qkv, alpha, beta logits, z ~ N(0, 1),
    conv_w ~ N(0, 0.5), dt ~ N(0, 0.5), ssm_a = -exp(U(-1, 1)), norm_w ~ 1 + N(0, 0.1),
    filled states ~ N(0, 0.02) and histories ~ N(0, 1).  Parity on the numpy-drawn
    workloads is the tests' job; these numbers only need the shapes and value ranges.
      tiny_b1_t8      8 sequential single-launch decode tokens of one sequence, captured
                      in one HIP graph and replayed: microseconds per token (launch- and
                      latency-bound; GB/s of its algorithmic bytes for reference)
      decode_b64      one single-launch decode token of 64 sequences: effective GB/s
                      (its 192 MiB of state can sit in the 256 MB Infinity Cache)
      decode_b256     the same at 256 sequences (the headline's configuration)
      prefill         16 sequences x 512 tokens in one call of the two-launch form: the
                      recurrence kernel in TFLOP/s against the fp32 VALU peak
      ragged          1024 sequences at random slots of a 2048-slot pool, U{1..8}
                      tokens each, in one call of the two-launch form: GB/s"""
    import numpy as np
    import torch
    geom = G.Geom()
    C, hv, vd, S = geom.channels, geom.h_v, geom.h_v * geom.s, geom.s
    eps = 1e-6
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    rnd = lambda *shape, std=1.0: torch.randn(*shape, generator=gen, device="cuda") * std
    conv_w, dt, norm_w = rnd(C, geom.d_conv, std=0.5), rnd(hv, std=0.5), 1.0 + rnd(S, std=0.1)
    ssm_a = -torch.exp(torch.rand(hv, generator=gen, device="cuda") * 2.0 - 1.0)
    out = {}

    def pool_of(n_slots, state_std, conv_std):
        pool = G.StatePool(n_slots, geom)
        if state_std:
            pool.state.normal_(0.0, state_std, generator=gen)
        else:
            pool.state.zero_()
        if conv_std:
            pool.conv.normal_(0.0, conv_std, generator=gen)
        else:
            pool.conv.zero_()
        pool.flags.zero_()
        return pool

    # tiny: 8 sequential decode tokens of one sequence, one graph of 8 launches
    T = 8
    pool = pool_of(1, 0.0, 0.0)
    qkv, alpha, bl, z = rnd(T, 1, C), rnd(T, 1, hv), rnd(T, 1, hv), rnd(T, 1, vd)
    y = torch.empty(T, 1, vd, device="cuda")
    tokens = lambda: [G.gdn_decode_fused(pool, qkv[t], conv_w, alpha[t], bl[t], dt, ssm_a, z[t], norm_w, eps, y[t])
                      for t in range(T)]
    for _ in range(3):
        tokens()
    torch.cuda.synchronize()
    eager_us = _event_span(stream, tokens, max(steps // 4, 10)) / T
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tokens()
    graph.replay()
    torch.cuda.synchronize()
    graph_us = _event_span(torch.cuda.current_stream(), graph.replay, max(steps // 4, 10)) / T
    nb, _ = _algorithmic(geom, 1, 1)
    out["tiny_b1_t8"] = {
        "form": "gdn_decode_fused, 8 sequential calls of B=1, captured in one HIP graph",
        "us_per_token_graph": graph_us, "us_per_token_eager": eager_us,
        "algorithmic_bytes_per_token": nb["one"],
        "roofline": {"bound": "latency", "achieved": nb["one"] / graph_us / 1e3, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": nb["one"] / graph_us / 1e3 / HBM_PEAK_GBPS,
                     "note": "16 workgroups, one per qk head: one workgroup's latency sets the time"}}
    log(f"tiny_b1_t8: {graph_us:.1f} us per token in a graph, {eager_us:.1f} us eager")
    del pool

    # single-launch decode at 64 and 256 sequences
    for B in (64, 256):
        pool = pool_of(B, 0.02, 1.0)
        qkv, alpha, bl, z = rnd(B, C), rnd(B, hv), rnd(B, hv), rnd(B, vd)
        y = torch.empty(B, vd, device="cuda")
        fn = lambda: G.gdn_decode_fused(pool, qkv, conv_w, alpha, bl, dt, ssm_a, z, norm_w, eps, y)
        for _ in range(warmup):
            fn()
        us = _event_span(stream, fn, steps)
        nb, units = _algorithmic(geom, B, 1)
        gbps = nb["one"] / us / 1e3
        out[f"decode_b{B}"] = {
            "form": "gdn_decode_fused (one launch)", "us_per_step": us, "seq_head_steps_per_s": units / us * 1e6,
            "algorithmic_bytes": nb["one"],
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS,
                         **({"note": "effective: the 192 MiB of state can sit in the 256 MB Infinity Cache"}
                            if B == 64 else {})}}
        log(f"decode_b{B}: {us:.1f} us per step, {gbps:.0f} GB/s")
        del pool

    # the two-launch form over many tokens: prefill and the ragged pool
    def two_launch(name, n_slots, B, T, state_std, conv_std, slots=None, n_tok=None, reps=None):
        pool = pool_of(n_slots, state_std, conv_std)
        qkv, alpha, bl, z = rnd(B, T, C), rnd(B, T, hv), rnd(B, T, hv), rnd(B, T, vd)
        h = torch.empty(B, T, C, device="cuda")
        y = torch.empty(B, T, vd, device="cuda")
        sl = None if slots is None else torch.from_numpy(slots).cuda()
        nt = None if n_tok is None else torch.from_numpy(n_tok).cuda()
        launches = {"conv": lambda: G.gdn_conv_silu_norm(pool, qkv, conv_w, eps, h, sl, nt),
                    "recurrence": lambda: G.gdn_decode_step_norm(pool, h, alpha, bl, dt, ssm_a, z, norm_w, eps, y,
                                                                 None, sl, nt)}
        for _ in range(max(warmup // 4, 2)):
            for f in launches.values():
                f()
        torch.cuda.synchronize()
        us = _kernel_events(stream, launches, reps)
        nb, units = _algorithmic(geom, B, T, n_tok)
        flags = int(pool.flags.item())
        if flags:
            raise SystemExit(f"bench.py: device flag word set ({flags:#x}) in {name}")
        del pool
        return us, nb, units

    reps = max(steps // 10, 10)
    us, nb, units = two_launch("prefill", 16, 16, 512, 0.0, 0.0, reps=reps)
    flops = units * FLOP_PER_SEQ_HEAD_STEP
    tflops = flops / us["recurrence"] / 1e6
    step_us = us["conv"] + us["recurrence"]
    out["prefill_b16_t512"] = {
        "form": "gdn_conv_silu_norm + gdn_decode_step_norm, 512 tokens per call",
        "kernel_us": us, "us_per_step": step_us, "tokens_per_s": 16 * 512 / step_us * 1e6,
        "algorithmic_flops_recurrence": flops, "algorithmic_bytes": {"conv": nb["conv"], "recurrence": nb["step_norm"]},
        "conv_gbps": nb["conv"] / us["conv"] / 1e3,
        "roofline": {"bound": "alu", "kernel": "decode_multi_kernel<fused norm>", "achieved": tflops,
                     "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / VALU_PEAK_TFLOPS,
                     "hbm_gbps": nb["step_norm"] / us["recurrence"] / 1e3}}
    log(f"prefill: conv {us['conv']:.1f} us, recurrence {us['recurrence']:.1f} us = {tflops:.1f} TFLOP/s")

    rng = np.random.default_rng(5)
    slots = rng.choice(2048, 1024, replace=False).astype(np.int32)
    n_tok = rng.integers(1, 9, 1024).astype(np.int32)
    us, nb, units = two_launch("ragged", 2048, 1024, 8, 0.02, 1.0, slots, n_tok, reps=reps)
    gbps = nb["step_norm"] / us["recurrence"] / 1e3
    step_us = us["conv"] + us["recurrence"]
    out["ragged_pool2048_b1024"] = {
        "form": "gdn_conv_silu_norm + gdn_decode_step_norm, per-sequence token counts, 8 tokens per call",
        "tokens": int(n_tok.sum()), "kernel_us": us, "us_per_step": step_us,
        "seq_head_steps_per_s": units / step_us * 1e6,
        "algorithmic_bytes": {"conv": nb["conv"], "recurrence": nb["step_norm"]},
        "step_gbps": (nb["conv"] + nb["step_norm"]) / step_us / 1e3,
        "roofline": {"bound": "hbm", "kernel": "decode_multi_kernel<fused norm>", "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS}}
    log(f"ragged: conv {us['conv']:.1f} us, recurrence {us['recurrence']:.1f} us = {gbps:.0f} GB/s")
    return out


def trace_summary(path: str, skip: int):
    """Per-kernel dispatch durations from a rocprofv3 kernel trace (csv): the first `skip`
    dispatches of each kernel (warm-up) are dropped, and the count, median, mean, min and
    max of the rest are printed, one kernel per line, longest median first.  Kernels
    with the same name and grid are one group."""
    import csv
    import statistics
    groups = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Kind", "KERNEL_DISPATCH") != "KERNEL_DISPATCH":
                continue
            key = (row["Kernel_Name"], row.get("Grid_Size_X", ""), row.get("Grid_Size_Y", ""))
            groups.setdefault(key, []).append((int(row["Start_Timestamp"]),
                                               (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0))
    lines = []
    for (name, gx, gy), rows in groups.items():
        rows.sort()
        us = [d for _, d in rows[skip:]]
        if not us:
            continue
        lines.append((statistics.median(us), f"{statistics.median(us):11.1f} us median  {statistics.mean(us):9.1f} mean  "
                                             f"{min(us):9.1f} min  {max(us):9.1f} max  x{len(us):<4d} (of {len(rows)})  "
                                             f"grid {gx}x{gy}  {name}"))
    for _, line in sorted(lines, reverse=True):
        print(line)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--trace-summary":
        tp = argparse.ArgumentParser()
        tp.add_argument("--trace-summary", required=True, help="a rocprofv3 kernel_trace.csv")
        tp.add_argument("--skip", type=int, default=0, help="warm-up dispatches of each kernel to drop")
        a = tp.parse_args()
        trace_summary(a.trace_summary, a.skip)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="b256", choices=["tiny", "b64", "b256", "prefill", "ragged"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--layer", default="",
                    help="comma-separated batch sizes: time one decode token of a whole layer "
                         "(projections + mixer) from a HIP graph, instead of the step")
    ap.add_argument("--verify", default="",
                    help="B,T: time one speculative round (verify window of T tokens + commit) "
                         "instead of the step")
    ap.add_argument("--batches", default="",
                    help="comma-separated batch sizes: one decode token per sequence in the single "
                         "launch and the two launches, for kernel traces, instead of the step")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record per-kernel HIP events on every N-th timed step")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload blocks (tiny, b64, b256, prefill, ragged) after the headline")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode mixer shards by sequence slots or head "
              "groups with no exchange inside the path, so a run on N GPUs is N independent "
              "copies of this one. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_mixer_gdn_amd as G
    import gdn_workloads as W

    if not os.path.exists(G.LIB_PATH):
        from gated_deltanet_mixer_gdn_amd import _build
        _build.build()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py: no GPU visible")
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.layer:
        layer_decode(G, [int(v) for v in args.layer.split(",")])
        return
    if args.batches:
        small_batches(G, [int(v) for v in args.batches.split(",")])
        return
    if args.verify:
        vb, vt = (int(v) for v in args.verify.split(","))
        verify_round(G, W, vb, vt)
        return

    wl = W.CONFIGS[args.config]()
    g = wl.geom
    log(f"workload {wl.name}: B={wl.B} T={wl.T} pool={wl.n_slots} slots")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pool = G.StatePool(wl.n_slots)
    pool.state.copy_(dev(wl.state))
    pool.conv.copy_(dev(wl.conv_state))
    pool.flags.zero_()
    qkv, alpha, bl, z = dev(wl.qkv), dev(wl.alpha), dev(wl.beta_logit), dev(wl.z)
    conv_w, dt, ssm_a, norm_w = dev(wl.conv_w), dev(wl.dt), dev(wl.ssm_a), dev(wl.norm_w)
    slots = dev(wl.slots)
    n_tok = dev(wl.n_tok) if wl.n_tok is not None else None
    h = torch.empty(wl.B, wl.T, g.channels, device="cuda")
    o = torch.empty(wl.B, wl.T, g.h_v, g.s, device="cuda")
    y = torch.empty(wl.B, wl.T, g.value_dim, device="cuda")
    stream = torch.cuda.current_stream()
    # the tiny configuration is T sequential decode calls of one token each (a step is
    # all T of them); every other configuration is one call per step.  Events of the
    # multi-kernel forms bracket the first call's kernels.
    seq = args.config == "tiny"
    calls = wl.T if seq else 1
    if seq:
        cut = lambda a, t: a[:, t:t + 1].contiguous()
        toks = [(cut(qkv, t), cut(alpha, t), cut(bl, t), cut(z, t), cut(h, t), cut(o, t), cut(y, t))
                for t in range(wl.T)]
    else:
        toks = [(qkv, alpha, bl, z, h, o, y)]

    def step_fused(ev=None):
        # the timed hot path: conv/SiLU/L2, then the recurrence with the gated RMSNorm
        # fused into its epilogue (y only, like the pages' fused step + norm kernel)
        for i, (qkv_, alpha_, bl_, z_, h_, o_, y_) in enumerate(toks):
            e = ev if i == 0 else None
            if e:
                e[0].record(stream)
            G.gdn_conv_silu_norm(pool, qkv_, conv_w, wl.eps, h_, slots, n_tok)
            if e:
                e[1].record(stream)
            G.gdn_decode_step_norm(pool, h_, alpha_, bl_, dt, ssm_a, z_, norm_w, wl.eps, y_, None, slots, n_tok)
            if e:
                e[2].record(stream)

    def step_one(ev=None):
        # single launch: conv/SiLU/L2, recurrence and gated RMSNorm for one token
        if ev:
            ev[0].record(stream)
        for qkv_, alpha_, bl_, z_, h_, o_, y_ in toks:
            G.gdn_decode_fused(pool, qkv_, conv_w, alpha_, bl_, dt, ssm_a, z_, norm_w, wl.eps, y_, None, slots)
        if ev:
            ev[1].record(stream)

    def step_three(ev=None):
        # the same pass as three separate calls (o goes through HBM)
        for i, (qkv_, alpha_, bl_, z_, h_, o_, y_) in enumerate(toks):
            e = ev if i == 0 else None
            if e:
                e[0].record(stream)
            G.gdn_conv_silu_norm(pool, qkv_, conv_w, wl.eps, h_, slots, n_tok)
            if e:
                e[1].record(stream)
            G.gdn_decode_step(pool, h_, alpha_, bl_, dt, ssm_a, o_, slots, n_tok)
            if e:
                e[2].record(stream)
            G.gdn_gated_rmsnorm(o_, z_, norm_w, wl.eps, y_)
            if e:
                e[3].record(stream)

    card = _card_dir()
    clocks = {}

    def timed(fn, n_ev, names):
        for _ in range(args.warmup):
            fn()
        # The timed region: K steps between two synchronisations, wall clock around it.
        # A step of one kernel: one pair of HIP events on the launch stream around all K
        # launches, so the kernel's average duration is the span over K (any gap between
        # the queued launches counts against it).  A step of several kernels: events
        # bracket every kernel of every `every`-th step of the same region (an event
        # record costs a few microseconds, so recording them on every step would
        # inflate the step time it is meant to explain).
        single_kernel = len(names) == 1
        every = max(1, args.event_every)
        sampled = [] if single_kernel else range(0, args.steps, every)
        evs = {k: [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for k in sampled}
        span = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        span[0].record(stream)
        for k in range(args.steps):
            fn(evs.get(k))
        span[1].record(stream)
        # the steps are queued and the GPU is still running them: sample its clocks
        clocks[fn.__name__] = gpu_clocks(card)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if single_kernel:
            return wall * 1000.0 / args.steps, {names[0]: span[0].elapsed_time(span[1]) / args.steps}, args.steps
        k_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs.values()]))
                for i, name in enumerate(names)}
        return wall * 1000.0 / args.steps, k_ms, len(evs)

    three_ms, three_k, _ = timed(step_three, 4, ("conv", "step", "norm"))
    single = (wl.T == 1 or seq) and wl.n_tok is None
    two_ms, two_k, two_n = timed(step_fused, 3, ("conv", "step_norm"))
    # the timed hot path: the single launch for one token per sequence (the fastest
    # form), else conv/SiLU/L2 + the recurrence with the norm fused (two launches)
    if single:
        one_ms, one_k, one_n = timed(step_one, 2, ("one",))
        one_k = {k: v / calls for k, v in one_k.items()}   # per launch
        ms_per_step, k_ms, n_samples, dominant = one_ms, one_k, one_n, "one"
    else:
        one_ms = one_k = None
        ms_per_step, k_ms, n_samples, dominant = two_ms, two_k, two_n, "step_norm"
    # context: the alpha / beta projections that feed this step (n_embd = 2560, bf16 weights)
    ab = W.make_ab(wl.B, wl.T, seed=11)
    ab_x = dev(ab.x)
    ab_wa = torch.from_numpy(ab.w_alpha.view(np.int16)).cuda()
    ab_wb = torch.from_numpy(ab.w_beta.view(np.int16)).cuda()
    ab_a, ab_b = torch.empty_like(alpha), torch.empty_like(bl)
    for _ in range(5):
        G.gdn_ab_project(ab_x, ab_wa, ab_wb, ab_a, ab_b)
    ae = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ae[0].record(stream)
    for _ in range(50):
        G.gdn_ab_project(ab_x, ab_wa, ab_wb, ab_a, ab_b)
    ae[1].record(stream)
    torch.cuda.synchronize()
    ab_us = ae[0].elapsed_time(ae[1]) / 50 * 1000.0
    ab_bytes = ab.x.nbytes + ab.w_alpha.nbytes + ab.w_beta.nbytes + 2 * ab_a.numel() * 4
    del ab_x, ab_a, ab_b

    # context: the dense projections around the mixer for the same rows (bf16 weights,
    # fp32 activations split once into bf16 hi + lo): qkv and z in one launch over the
    # layer input, out over the mixer output
    proj = projections_context(G, W, wl.B * wl.T, stream)

    # context: a plain device-to-device copy of the state's size on the same stream
    ref_src = pool.state.view(-1)
    ref_dst = torch.empty_like(ref_src)
    for _ in range(3):
        ref_dst.copy_(ref_src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    for _ in range(20):
        ref_dst.copy_(ref_src)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * ref_src.numel() * 4 * 20 / (ce[0].elapsed_time(ce[1]) / 1000.0) / 1e9
    del ref_dst
    flags = int(pool.flags.item())
    if flags:
        raise SystemExit(f"bench.py: device flag word set ({flags:#x})")

    nbytes, units = algorithmic_bytes(dataclasses.replace(wl, T=1) if seq else wl)   # per call
    units *= calls                                                                     # per step
    value = units / (ms_per_step / 1000.0)
    achieved = nbytes[dominant] / (k_ms[dominant] / 1000.0) / 1e9
    # a workload whose flops per algorithmic byte exceed the VALU / HBM ridge (the
    # multi-token prefill) is priced against the fp32 VALU peak instead
    flops = units // calls * FLOP_PER_SEQ_HEAD_STEP                                   # per launch
    alu_bound = flops / nbytes[dominant] > VALU_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    achieved_tflops = flops / (k_ms[dominant] / 1000.0) / 1e12
    mixer_bytes = calls * (nbytes["one"] if single else nbytes["conv"] + nbytes["step_norm"])
    mixer_gbps = mixer_bytes / (ms_per_step / 1000.0) / 1e9
    two_gbps = nbytes["step_norm"] / (two_k["step_norm"] / 1000.0) / 1e9
    three_step_gbps = nbytes["step"] / (three_k["step"] / 1000.0) / 1e9
    one_gbps = nbytes["one"] / (one_k["one"] / 1000.0) / 1e9 if single else None
    if single:
        log(f"one launch: {one_k['one'] * 1000:.1f}us kernel; {one_ms * 1000:.1f} us/step; {one_gbps:.0f} GB/s")
    log("two calls: " + ", ".join(f"{k}={v * 1000:.1f}us" for k, v in two_k.items()) +
        f"; {two_ms * 1000:.1f} us/step; recurrence+norm kernel {two_gbps:.0f} GB/s")
    log(f"ab projection: {ab_us:.1f} us for {wl.B * wl.T} rows ({ab_bytes / ab_us / 1e3:.0f} GB/s)")
    log("three calls: " + ", ".join(f"{k}={v * 1000:.1f}us" for k, v in three_k.items()) +
        f"; {three_ms * 1000:.1f} us/step; recurrence kernel {three_step_gbps:.0f} GB/s; d2d copy {copy_gbps:.0f} GB/s")
    traffic = read_traffic() if args.config == "b256" else None

    configs = None if args.no_configs else config_blocks(G, W, stream, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        log(f"oracle: {cpu['value']:.0f} {cpu['unit']} on {cpu['cores']} threads")

    out = {
        "metric": "GDN decode seq-head-steps/s and achieved HBM GB/s vs peak at B=256",
        "value": value,
        "unit": "seq-head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "n_slots": wl.n_slots,
                   "h_k": g.h_k, "h_v": g.h_v, "S": g.s, "d_conv": g.d_conv,
                   "state_bytes": int(wl.n_slots * g.h_v * g.s * g.s * 4), "parallelism": "none"},
        "path": (f"gdn_decode_fused, {calls} sequential calls of one token per step" if seq else
                 "gdn_decode_fused (conv, recurrence and gated RMSNorm in one launch, y only)" if single else
                 "gdn_conv_silu_norm + gdn_decode_step_norm (gated RMSNorm fused, y only)"),
        "hbm_gbps_mixer": mixer_gbps,
        "hbm_frac_mixer": mixer_gbps / HBM_PEAK_GBPS,
        "kernel_us": {k: v * 1000.0 for k, v in k_ms.items()},
        "two_call_path": {"ms_per_step": two_ms, "kernel_us": {k: v * 1000.0 for k, v in two_k.items()},
                          "value": units / (two_ms / 1000.0), "recurrence_kernel_gbps": two_gbps,
                          "algorithmic_bytes_per_launch": {"conv": nbytes["conv"], "step_norm": nbytes["step_norm"]}},
        "three_call_path": {"ms_per_step": three_ms, "kernel_us": {k: v * 1000.0 for k, v in three_k.items()},
                            "value": units / (three_ms / 1000.0),
                            "recurrence_kernel_gbps": three_step_gbps},
        "d2d_copy_gbps_same_size": copy_gbps,
        "ab_projection": {"us": ab_us, "algorithmic_bytes": int(ab_bytes), "gbps": ab_bytes / ab_us / 1e3,
                          "rows": wl.B * wl.T, "n_embd": W.N_EMBD},
        "projections": proj,
        "roofline": {"kernel": (f"decode_fused_par_kernel<{g.h_v // g.h_k}>" if single and g.h_v // g.h_k <= 3 else
                                "decode_fused_kernel" if single else "decode_multi_kernel<fused norm>"),
                     "bound": "alu" if alu_bound else "hbm",
                     "achieved": achieved_tflops if alu_bound else achieved,
                     "peak": VALU_PEAK_TFLOPS if alu_bound else HBM_PEAK_GBPS,
                     "unit": "TFLOP/s" if alu_bound else "GB/s",
                     "frac": achieved_tflops / VALU_PEAK_TFLOPS if alu_bound else achieved / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes[dominant],
                     "algorithmic_flops_per_launch": flops,
                     "hbm_gbps": achieved,
                     "event_samples": n_samples,
                     "event_timing": ("one event pair around all timed launches" if single else
                                      "events around the kernels of every sampled step")},
        "gpu_clocks_during_timing": clocks.get("step_one" if single else "step_fused"),
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
