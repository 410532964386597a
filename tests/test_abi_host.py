"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/gdn.h declares, and reject
bad arguments with the documented codes before touching the device.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def L():
    from gated_deltanet_mixer_gdn_amd import gdn
    if not os.path.exists(gdn.LIB_PATH):
        from gated_deltanet_mixer_gdn_amd import _build
        _build.build()
    return gdn.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("gdn_state_pool_create", "gdn_conv_silu_norm", "gdn_decode_step", "gdn_gated_rmsnorm",
              "gdn_state_pool_zero", "gdn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from gated_deltanet_mixer_gdn_amd import gdn
    for name in declared_functions():
        assert hasattr(L, name), f"{name} is declared in gdn.h but not exported"
    assert sorted(gdn.EXPORTS) == declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(gdn_[a-z0-9_]+)$", out, flags=re.M))
    assert exported == set(declared_functions())


def test_package_reexports_every_binding():
    """Every public function and class of the binding module is reachable from the
    package, where the tests and callers look for it."""
    import inspect
    import gated_deltanet_mixer_gdn_amd as G
    from gated_deltanet_mixer_gdn_amd import gdn
    public = [name for name, obj in vars(gdn).items()
              if not name.startswith("_") and (inspect.isfunction(obj) or inspect.isclass(obj))
              and obj.__module__ == gdn.__name__]
    assert public and [name for name in public if not hasattr(G, name)] == []


def test_library_is_built_for_gfx950_only(tmp_path):
    from gated_deltanet_mixer_gdn_amd import gdn
    fb = tmp_path / "fatbin.bin"
    subprocess.check_call(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", gdn.LIB_PATH, str(fb)])
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          "--input=" + str(fb)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets and all(t.endswith("gfx950") for t in targets), targets


def _kernel_disassembly(tmp_path):
    """The gfx950 disassembly of every code object in the built library (the fat binary
    section holds one bundle per source file)."""
    from gated_deltanet_mixer_gdn_amd import gdn
    fb = tmp_path / "fatbin.bin"
    subprocess.check_call(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", gdn.LIB_PATH, str(fb)])
    data = fb.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    assert starts, "no offload bundle in the library"
    text = []
    for n, s in enumerate(starts):
        part = tmp_path / f"bundle{n}.bin"
        part.write_bytes(data[s:starts[n + 1] if n + 1 < len(starts) else len(data)])
        co = tmp_path / f"bundle{n}.co"
        subprocess.check_call(["/opt/rocm/llvm/bin/clang-offload-bundler", "--unbundle", "--type=o",
                               "--input=" + str(part), "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                               "--output=" + str(co)])
        text.append(subprocess.run(["/opt/rocm/llvm/bin/llvm-objdump", "-d", str(co)], capture_output=True,
                                   text=True, check=True).stdout)
    return "\n".join(text)


def test_kernels_make_no_generic_or_scratch_memory_access(tmp_path):
    """Every memory access of the kernels is a global, buffer or LDS instruction: a flat
    (generic) access means an address lost its address space (an LDS pointer cast through
    an integer once turned LDS slots into flat accesses to unmapped low addresses), and a
    scratch access means registers spilled.  Checked on the built gfx950 code."""
    dis = _kernel_disassembly(tmp_path)
    kernels = re.findall(r"<(_ZN3gdn\w+)>:", dis)
    assert any("decode_multi_kernel" in k for k in kernels) and any("conv_silu_norm_kernel" in k for k in kernels)
    bad = [ln.strip() for ln in dis.splitlines() if re.match(r"\s*(flat|scratch)_\w+", ln)]
    assert not bad, bad[:5]


def test_abi_version(L):
    assert L.gdn_abi_version() == 7


def _geom(h_k=16, h_v=48, s=128, d_conv=4):
    from gated_deltanet_mixer_gdn_amd.gdn import gdn_geom
    return gdn_geom(h_k, h_v, s, d_conv, 0, 0)


def test_pool_bytes(L):
    g = _geom()
    n = L.gdn_state_pool_bytes(ctypes.byref(g), 3)
    state = 3 * 48 * 128 * 128 * 4
    conv = 3 * 10240 * 3 * 4
    r = lambda x: (x + 255) // 256 * 256
    assert n == 256 + r(state) + r(conv)
    assert L.gdn_state_pool_bytes(ctypes.byref(g), 0) == 0
    assert b"n_slots" in L.gdn_last_error()
    assert L.gdn_state_pool_bytes(None, 3) == 0
    bad = _geom(s=64)
    assert L.gdn_state_pool_bytes(ctypes.byref(bad), 3) == 0
    assert b"built for" in L.gdn_last_error()


def test_pool_bytes_that_would_wrap_are_refused(L):
    """A pool whose byte count passes the address space (a wide geometry times 2^31
    slots) is refused, and so is creating it, instead of wrapping to a small size."""
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG
    wide = _geom(h_k=1, h_v=1 << 22)              # 2^38 bytes of state per slot
    assert L.gdn_state_pool_bytes(ctypes.byref(wide), 1) == 256 + (1 << 38) + (2 + (1 << 22)) * 128 * 3 * 4
    assert L.gdn_state_pool_bytes(ctypes.byref(wide), 1 << 31) == 0
    assert b"address space" in L.gdn_last_error()
    h = ctypes.c_void_p()
    assert L.gdn_state_pool_create(ctypes.byref(wide), 1 << 31, 4096, 1 << 40, ctypes.byref(h)) == GDN_ERR_ARG
    assert b"address space" in L.gdn_last_error() and h.value is None
    # the largest pool of the pages' geometry still has a size
    g = _geom()
    assert L.gdn_state_pool_bytes(ctypes.byref(g), 1 << 31) > (1 << 31) * 48 * 128 * 128 * 4


def _slots_rc(L, slots, n_slots):
    import numpy as np
    a = np.ascontiguousarray(slots, dtype=np.int32)
    return L.gdn_check_slots(a.ctypes.data if a.size else None, int(a.size), n_slots)


def test_check_slots_clean_lists(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_OK
    import numpy as np
    assert _slots_rc(L, [], 4) == GDN_OK
    assert _slots_rc(L, [3, 0, 2, 1], 4) == GDN_OK
    perm = np.random.default_rng(3).choice(2048, 1024, replace=False)
    assert _slots_rc(L, perm, 2048) == GDN_OK
    assert L.gdn_last_error() == b""


def test_check_slots_out_of_range(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG
    assert _slots_rc(L, [0, 4, 1], 4) == GDN_ERR_ARG
    assert L.gdn_last_error() == b"gdn_check_slots: slots[1]=4 is outside the pool's 4 slots"
    assert _slots_rc(L, [0, 1, -1, 9], 4) == GDN_ERR_ARG
    assert b"slots[2]=-1" in L.gdn_last_error()
    assert L.gdn_check_slots(None, 3, 4) == GDN_ERR_ARG
    assert b"host_slots is null" in L.gdn_last_error()
    assert L.gdn_check_slots(None, -1, 4) == GDN_ERR_ARG
    assert _slots_rc(L, [0], 0) == GDN_ERR_ARG


def test_check_slots_duplicates(L):
    """The first entry that repeats an earlier one is named, with that earlier position,
    whatever order the repeats come in."""
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG
    assert _slots_rc(L, [5, 2, 7, 2], 8) == GDN_ERR_ARG
    assert L.gdn_last_error() == b"gdn_check_slots: slots[3]=2 repeats slots[1]: slots within a call must be unique"
    assert _slots_rc(L, [1, 6, 6, 1, 6], 8) == GDN_ERR_ARG
    assert b"slots[2]=6 repeats slots[1]" in L.gdn_last_error()
    assert _slots_rc(L, [0, 0], 1) == GDN_ERR_ARG
    assert b"slots[1]=0 repeats slots[0]" in L.gdn_last_error()


def test_binding_check_slots_and_debug_switch():
    """The binding's gdn_check_slots raises GdnError on a bad list; the debug switch
    turns the host check of every mixer call on and off."""
    import numpy as np
    import gated_deltanet_mixer_gdn_amd as G
    from gated_deltanet_mixer_gdn_amd import gdn
    G.gdn_check_slots(np.array([2, 0, 1], np.int32), 3)
    with pytest.raises(G.GdnError) as e:
        G.gdn_check_slots([2, 0, 2], 3)
    assert e.value.code == G.GDN_ERR_ARG and "repeats" in str(e.value)
    was = gdn._check_slots_on
    try:
        G.set_slot_checks(True)
        assert gdn._check_slots_on
        G.set_slot_checks(False)
        assert not gdn._check_slots_on
    finally:
        G.set_slot_checks(was)


def test_pool_create_argument_errors(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_ERR_UNSUPPORTED
    g = _geom()
    h = ctypes.c_void_p()
    need = L.gdn_state_pool_bytes(ctypes.byref(g), 2)
    assert L.gdn_state_pool_create(ctypes.byref(g), 2, 4096, need, None) == GDN_ERR_ARG
    assert L.gdn_state_pool_create(ctypes.byref(g), 2, None, need, ctypes.byref(h)) == GDN_ERR_ARG
    assert b"dev_base is null" in L.gdn_last_error()
    assert L.gdn_state_pool_create(ctypes.byref(g), 2, 4096 + 16, need, ctypes.byref(h)) == GDN_ERR_ARG
    assert b"256-byte" in L.gdn_last_error()
    assert L.gdn_state_pool_create(ctypes.byref(g), 2, 4096, need - 1, ctypes.byref(h)) == GDN_ERR_ARG
    assert L.gdn_state_pool_create(ctypes.byref(g), -1, 4096, need, ctypes.byref(h)) == GDN_ERR_ARG
    odd = _geom(h_k=16, h_v=40)
    assert L.gdn_state_pool_create(ctypes.byref(odd), 2, 4096, need, ctypes.byref(h)) == GDN_ERR_ARG
    assert b"multiple" in L.gdn_last_error()
    wide = _geom(d_conv=5)
    assert L.gdn_state_pool_create(ctypes.byref(wide), 2, 4096, need, ctypes.byref(h)) == GDN_ERR_UNSUPPORTED
    assert h.value is None


def test_calls_on_null_pool_are_rejected(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG
    assert L.gdn_conv_silu_norm(None, None, None, 1, 1, 16, 16, 1e-6, 16, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_conv_silu_norm: pool is null")
    assert L.gdn_decode_step(None, None, None, 1, 1, 16, 16, 16, 16, 16, 16, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_decode_step: pool is null")
    assert L.gdn_state_pool_zero(None, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_state_pool_state(None) is None
    assert L.gdn_state_pool_slots(None) == 0
    L.gdn_state_pool_destroy(None)


def test_rmsnorm_argument_errors(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_OK
    assert L.gdn_gated_rmsnorm(16, 16, 16, 1e-6, 4, 64, 0, 16, None) == GDN_ERR_UNSUPPORTED
    assert L.gdn_gated_rmsnorm(16, 16, 16, 1e-6, -1, 128, 0, 16, None) == GDN_ERR_ARG
    assert L.gdn_gated_rmsnorm(16, 16, 16, float("nan"), 4, 128, 0, 16, None) == GDN_ERR_ARG
    assert L.gdn_gated_rmsnorm(16, 16, 16, -1.0, 4, 128, 0, 16, None) == GDN_ERR_ARG
    assert L.gdn_gated_rmsnorm(None, 16, 16, 1e-6, 4, 128, 0, 16, None) == GDN_ERR_ARG
    assert b"o is null" in L.gdn_last_error()
    assert L.gdn_gated_rmsnorm(16, 16, 20, 1e-6, 4, 128, 0, 16, None) == GDN_ERR_ARG
    assert b"w is not 16-byte aligned" in L.gdn_last_error()
    # z and y overlapping is refused; rows = 0 is a no-op that touches nothing
    assert L.gdn_gated_rmsnorm(4096, 1 << 20, 16, 1e-6, 4, 128, 0, 1 << 20, None) == GDN_ERR_ARG
    assert L.gdn_gated_rmsnorm(None, None, None, 1e-6, 0, 128, 0, None, None) == GDN_OK
    assert L.gdn_last_error() == b""
    assert L.gdn_gated_rmsnorm(16, 16, 16, 1e-6, 4, 128, 2, 16, None) == GDN_ERR_ARG
    assert b"gate_silu" in L.gdn_last_error()


def test_geometry_option_flags(L):
    """The two model options are 0 or 1; anything else is refused before any work."""
    import ctypes
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, gdn_geom
    for flags in ((2, 0), (0, -1)):
        g = gdn_geom(16, 48, 128, 4, *flags)
        assert L.gdn_state_pool_bytes(ctypes.byref(g), 4) == 0
        p = ctypes.c_void_p()
        assert L.gdn_state_pool_create(ctypes.byref(g), 4, 256, 1 << 30, ctypes.byref(p)) == GDN_ERR_ARG
        assert b"must be 0 or 1" in L.gdn_last_error()
    g = gdn_geom(16, 48, 128, 4, 1, 1)
    assert L.gdn_state_pool_bytes(ctypes.byref(g), 4) == L.gdn_state_pool_bytes(ctypes.byref(_geom()), 4) > 0


def test_last_error_is_thread_local(L):
    import threading
    L.gdn_gated_rmsnorm(16, 16, 16, 1e-6, 4, 64, 0, 16, None)
    seen = []
    t = threading.Thread(target=lambda: seen.append(L.gdn_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert b"s=64" in L.gdn_last_error()


def test_binding_refuses_cpu_tensors():
    import torch
    from gated_deltanet_mixer_gdn_amd import gdn
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        gdn.gdn_gated_rmsnorm(x, x, torch.zeros(128), 1e-6, x)


def test_product_path_does_not_reference_the_oracle():
    """The HIP path and the oracle share no code; neither imports the other."""
    pkg = os.path.join(ROOT, "gated_deltanet_mixer_gdn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower().replace("oracle-free", ""), f
                assert "gdn_workloads" not in src, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert "gated_deltanet_mixer_gdn_amd" not in src and "gdn.h" not in src, f


def test_import_without_gpu_does_not_load_library():
    code = ("import gated_deltanet_mixer_gdn_amd.gdn as g, sys; "
            "assert g._lib is None; print('ok')")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert out.returncode == 0 and "ok" in out.stdout, out.stderr


def test_new_entry_points_reject_null_pool(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_OK
    assert L.gdn_decode_step_norm(None, None, None, 1, 1, 16, 16, 16, 16, 16, 16, 16, 1e-6, None, 16, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_decode_step_norm: pool is null")
    assert L.gdn_decode_step_norm(None, None, None, 1, 1, 16, 16, 16, 16, 16, 16, 16, 1e-6, None, None, None) == GDN_ERR_ARG
    assert b"y is null" in L.gdn_last_error()
    assert L.gdn_decode_fused(None, None, 1, 16, 16, 16, 16, 16, 16, 16, 16, 1e-6, 16, None, None, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_decode_fused: pool is null")
    assert L.gdn_verify_window(None, None, None, 1, 2, 16, 16, 16, 16, 16, 16, 16, 16, 1e-6, 16, 16, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_verify_window: pool is null")
    assert L.gdn_verify_window(None, None, None, 1, 2, 16, 16, 16, 16, 16, 16, 16, 16, 1e-6, None, 16, None) == GDN_ERR_ARG
    assert b"h is null" in L.gdn_last_error()
    assert L.gdn_commit(None, None, None, 1, 2, 16, 16, 16, 16, 16, 16, None) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_commit: pool is null")
    args = [None, None, 1, None, 2, 16, 16, 16, 16, None, 3, 16, 16, 16, 16, 16, 16, 16, 16, 1e-6, 16, 16, None]
    assert L.gdn_commit_window(*args) == GDN_ERR_ARG
    assert L.gdn_last_error().startswith(b"gdn_commit_window: pool is null")
    for k in (6, 20, 21):                             # h0, h1, y1
        bad = list(args)
        bad[k] = None
        assert L.gdn_commit_window(*bad) == GDN_ERR_ARG
        assert b"is null" in L.gdn_last_error()
    assert L.gdn_commit_window(*(args[:2] + [0] + args[3:])) == GDN_ERR_ARG   # B = 0 still checks the pool


def test_ab_project_argument_errors(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_OK
    assert L.gdn_ab_project(16, 16, 16, -1, 2560, 48, 16, 16, None) == GDN_ERR_ARG
    assert L.gdn_ab_project(16, 16, 16, 4, 2562, 48, 16, 16, None) == GDN_ERR_UNSUPPORTED
    assert L.gdn_ab_project(16, 16, 16, 4, 0, 48, 16, 16, None) == GDN_ERR_ARG
    assert L.gdn_ab_project(None, 16, 16, 4, 2560, 48, 16, 16, None) == GDN_ERR_ARG
    assert b"x is null" in L.gdn_last_error()
    assert L.gdn_ab_project(16, 12, 16, 4, 2560, 48, 16, 16, None) == GDN_ERR_ARG
    assert b"w_alpha" in L.gdn_last_error()
    assert L.gdn_ab_project(16, 16, 16, 4, 2560, 48, 1 << 20, 1 << 20, None) == GDN_ERR_ARG
    assert b"overlaps" in L.gdn_last_error()
    assert L.gdn_ab_project(None, None, None, 0, 2560, 48, None, None, None) == GDN_OK


def test_projection_argument_errors(L):
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_OK
    assert L.gdn_split_bf16_bytes(70, 2560) == 96 * 2560 * 4
    assert L.gdn_split_bf16_bytes(1, 8) == 32 * 64 * 4
    assert L.gdn_split_bf16_bytes(-1, 64) == -1 and L.gdn_split_bf16_bytes(4, 12) == -1
    assert L.gdn_pack_bf16_bytes(100, 136) == 128 * 192 * 2
    assert L.gdn_pack_bf16_bytes(0, 64) == -1 and L.gdn_pack_bf16_bytes(4, 0) == -1
    assert L.gdn_split_bf16_bytes(1, (1 << 24) + 8) == -1 and L.gdn_pack_bf16_bytes(1, (1 << 24) + 8) == -1
    assert L.gdn_project_bf16(16, 16, 4, (1 << 24) + 8, 32, 1 << 20, None, 0, None) == GDN_ERR_ARG
    assert b"at most" in L.gdn_last_error()
    assert L.gdn_split_bf16(16, -1, 64, 16, None) == GDN_ERR_ARG
    assert L.gdn_split_bf16(16, 4, 60, 16, None) == GDN_ERR_ARG
    assert b"multiple of 8" in L.gdn_last_error()
    assert L.gdn_split_bf16(None, 4, 64, 1 << 20, None) == GDN_ERR_ARG
    assert L.gdn_split_bf16(1 << 20, 4, 64, (1 << 20) + 512, None) == GDN_ERR_ARG
    assert b"xs overlaps x" in L.gdn_last_error()
    assert L.gdn_split_bf16(16, 4, 64, 8, None) == GDN_ERR_ARG       # misaligned xs
    assert L.gdn_split_bf16(None, 0, 64, None, None) == GDN_OK
    assert L.gdn_pack_bf16(16, 0, 64, 1 << 20, None) == GDN_ERR_ARG
    assert L.gdn_pack_bf16(24, 4, 64, 1 << 20, None) == GDN_ERR_ARG
    assert L.gdn_pack_bf16(1 << 20, 32, 64, (1 << 20) + 64, None) == GDN_ERR_ARG
    assert b"wp overlaps w" in L.gdn_last_error()
    assert L.gdn_project_bf16(16, 16, -1, 64, 32, 16, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_project_bf16(16, 16, 4, 12, 32, 1 << 20, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_project_bf16(16, 16, 4, 64, 0, 1 << 20, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_project_bf16(16, 24, 4, 64, 32, 1 << 20, None, 0, None) == GDN_ERR_ARG
    assert b"wp is not 16-byte aligned" in L.gdn_last_error()
    assert L.gdn_project_bf16(1 << 20, 1 << 24, 4, 64, 32, (1 << 20) + 64, None, 0, None) == GDN_ERR_ARG
    assert b"output overlaps xs" in L.gdn_last_error()
    assert L.gdn_project_bf16(1 << 24, 1 << 20, 4, 64, 32, (1 << 20) + 64, None, 0, None) == GDN_ERR_ARG
    assert b"output overlaps wp" in L.gdn_last_error()
    assert L.gdn_project_bf16(None, None, 0, 64, 32, None, None, 0, None) == GDN_OK
    assert L.gdn_project2_bf16(16, 16, 4, 64, 32, 1 << 20, 0, 1 << 22, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_project2_bf16(16, 16, 4, 64, 0, 1 << 20, 32, 1 << 22, None, 0, None) == GDN_ERR_ARG
    assert L.gdn_project2_bf16(16, 16, 4, 64, 32, 1 << 20, 32, (1 << 20) + 256, None, 0, None) == GDN_ERR_ARG
    assert b"out1 overlaps out2" in L.gdn_last_error()
    assert L.gdn_project2_bf16(16, 16, 4, 64, 32, 1 << 20, 32, 2, None, 0, None) == GDN_ERR_ARG
    assert b"out2 is not 4-byte aligned" in L.gdn_last_error()
    assert L.gdn_project2_bf16(None, None, 0, 64, 32, None, 16, None, None, 0, None) == GDN_OK


def test_projection_workspace(L):
    """The workspace is 0 bytes unless a long k range meets few output tiles; a launch
    that needs one refuses a missing, short, misaligned or overlapping workspace before
    anything runs (every call below fails its checks)."""
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_OK
    W = L.gdn_project_workspace_bytes
    assert W(256, 2560, 16384) == 0 and W(1, 2560, 2560) == 0 and W(0, 6144, 2560) == 0
    # 1 row, out projection: 80 tiles of 32 x 32, k split 3 ways, one 4 KiB block each
    assert W(1, 6144, 2560) == 80 * 3 * 4096 == W(32, 6144, 2560)
    # 100 rows, 1000 columns: 4 x 16 tiles of 32 x 64 split 4 ways, 8 KiB blocks
    assert W(100, 6144, 1000) == 4 * 16 * 4 * 8192
    assert W(256, 6144, 2560) == 0 and W(96, 6144, 2560) == 0
    assert W(-1, 64, 32) == -1 and W(4, 12, 32) == -1 and W(4, 64, 0) == -1 and W(4, (1 << 24) + 8, 32) == -1
    xs, wp, out, ws = 1 << 30, 2 << 30, 3 << 30, 4 << 30
    need = W(1, 6144, 2560)
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, None, 0, None) == GDN_ERR_ARG
    assert b"the launch needs %d" % need in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, ws, need - 16, None) == GDN_ERR_ARG
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, None, need, None) == GDN_ERR_ARG
    assert b"workspace is null" in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, ws + 8, need, None) == GDN_ERR_ARG
    assert b"workspace is not 16-byte aligned" in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, xs + 4096, need, None) == GDN_ERR_ARG
    assert b"workspace overlaps xs" in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, wp - 4096, need, None) == GDN_ERR_ARG
    assert b"workspace overlaps wp" in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, out - 16, need, None) == GDN_ERR_ARG
    assert b"workspace overlaps out" in L.gdn_last_error()
    assert L.gdn_project2_bf16(xs, wp, 1, 6144, 2000, out, 560, out + 8192, out + 8192 + 16, need, None) == GDN_ERR_ARG
    assert b"workspace overlaps out2" in L.gdn_last_error()
    assert L.gdn_project_bf16(xs, wp, 1, 6144, 2560, out, ws, -1, None) == GDN_ERR_ARG
    assert b"negative" in L.gdn_last_error()
    assert L.gdn_project_bf16(None, None, 0, 6144, 2560, None, None, 0, None) == GDN_OK


def test_projection_multi_argument_errors(L):
    """Bad output counts, column counts, null or overlapping outputs are refused before
    anything runs (every call below fails its checks)."""
    import ctypes
    from gated_deltanet_mixer_gdn_amd.gdn import GDN_ERR_ARG, GDN_OK
    xs, wp, o = 1 << 30, 2 << 30, 3 << 30
    cols = lambda *c: (ctypes.c_int32 * len(c))(*c)
    outs = lambda *p: (ctypes.c_void_p * len(p))(*p)
    M = L.gdn_project_multi_bf16
    assert M(xs, wp, 4, 64, 0, cols(1), outs(o), None, 0, None) == GDN_ERR_ARG
    assert b"n_out=0" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 5, cols(1, 1, 1, 1, 1), outs(o, o, o, o, o), None, 0, None) == GDN_ERR_ARG
    assert M(xs, wp, 4, 64, 2, None, outs(o, o + 4096), None, 0, None) == GDN_ERR_ARG
    assert b"cols is null" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 2, cols(8, 8), None, None, 0, None) == GDN_ERR_ARG
    assert b"outs is null" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 3, cols(8, 0, 8), outs(o, o + 4096, o + 8192), None, 0, None) == GDN_ERR_ARG
    assert b"outs[1] has 0 columns" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 3, cols(8, 8, 8), outs(o, None, o + 8192), None, 0, None) == GDN_ERR_ARG
    assert b"outs[1] is null" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 4, cols(8, 8, 8, 8), outs(o, o + 4096, o + 8192, o + 8192 + 64), None, 0, None) \
        == GDN_ERR_ARG
    assert b"outs[2] overlaps outs[3]" in L.gdn_last_error()
    assert M(xs, wp, 4, 64, 4, cols(8, 8, 8, 8), outs(o, o + 4096, o + 8192, xs + 64), None, 0, None) == GDN_ERR_ARG
    assert b"an output overlaps xs" in L.gdn_last_error()
    assert M(None, None, 0, 64, 2, cols(8, 8), outs(None, None), None, 0, None) == GDN_OK
