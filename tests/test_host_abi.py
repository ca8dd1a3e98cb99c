"""Host-side tests of the C-ABI library (no GPU needed, nothing is launched).

The library must load, export every function include/moe.h declares, and
reject invalid arguments before enqueueing anything.
"""
import ctypes
import os
import re

import numpy as np

import pytest

import oracle as O
import workloads as W

M = pytest.importorskip("expert_router_gemm_softmax_amd")
B = M.binding


def _declared_functions(repo_root):
    text = open(os.path.join(repo_root, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(",
                                 text, flags=re.M)))


def test_library_exports_every_declared_function(repo_root):
    names = _declared_functions(repo_root)
    assert len(names) >= 15, names
    lib = ctypes.CDLL(M.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each one
    assert set(names) <= set(B._SIGS), set(names) - set(B._SIGS)


def test_library_exports_only_the_c_entry_points(repo_root):
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", M.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = sorted({ln.split()[-1] for ln in out.splitlines()
                    if len(ln.split()) == 3 and ln.split()[1] in ("T", "W")})
    declared = set(_declared_functions(repo_root))
    extra = [f for f in funcs if f not in declared and not f.startswith("_init")
             and not f.startswith("_fini")]
    assert not extra, extra


def test_library_is_in_tree_and_for_gfx950(repo_root):
    assert os.path.dirname(M.LIB_PATH) == os.path.join(repo_root,
                                                        "expert_router_gemm_softmax_amd")
    blob = open(M.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


@pytest.mark.parametrize("T,k,E,cf", [(64, 1, 4, 1.25), (4096, 2, 8, 1.25),
                                      (32768, 8, 128, 1.0), (80, 1, 8, 1.1),
                                      (81, 1, 8, 1.1), (1000, 3, 7, 0.3),
                                      (10, 2, 4, 0.0), (12345, 4, 96, 2.5)])
def test_capacity_helper_matches_oracle(T, k, E, cf):
    assert M.moe_capacity(T, k, E, cf) == O.capacity(T, k, E, cf)


def test_capacity_helper_is_exact_at_large_sizes_and_decimal_boundaries():
    """The factor is read as its shortest round-trip decimal, like the
    oracle's Fraction(str(cf)), and the ceiling is taken exactly: no slack
    that grows with T*k/E, and no binary rounding of decimals such as 0.1."""
    cases = [(2 ** 30, 1, 3, 1.0), (1000, 1, 2, 1.0000000005), (1000, 1, 2, 1.0000000000000002),
             (10, 1, 1, 0.1), (30, 1, 1, 0.1), (3, 1, 10, 0.1), (7, 3, 21, 1.0),
             (2 ** 31 - 1, 1, 256, 1.1), (2 ** 31 - 1, 1, 255, 0.9999999999999999),
             (1, 1, 1, 1e-300), (5, 1, 1, 5e-324), (10 ** 6, 32, 7, 2.3333333333333335),
             (4096, 2, 8, 1.25), (32768, 8, 128, 1.0), (2 ** 40, 1, 1000, 0.001)]
    rng = np.random.default_rng(0)
    for _ in range(400):
        digits = int(rng.integers(1, 8))
        cf = float(f"{rng.integers(1, 10 ** digits)}e{-int(rng.integers(0, digits + 2))}")
        cases.append((int(rng.integers(1, 1 << 22)), int(rng.integers(1, 33)),
                      int(rng.integers(1, 257)), cf))
        # T k / E an exact multiple of 1 / cf's decimal: the value is an integer
        E = int(rng.integers(1, 257))
        cases.append((E * 10 ** 3, 1, E, float(f"{rng.integers(1, 999)}e-3")))
    for T, k, E, cf in cases:
        want = O.capacity(T, k, E, cf)
        want = min(want, T * k)   # the helper saturates at T*k (drops nothing either way)
        assert M.moe_capacity(T, k, E, cf) == want, (T, k, E, cf)
    assert M.moe_capacity(2 ** 30, 1, 3, 1.0) == 357913942
    assert M.moe_capacity(1000, 1, 2, 1.0000000005) == 501
    assert M.moe_capacity(2 ** 62, 4, 1, 0.5) == M.MOE_NO_CAPACITY  # T*k overflows int64


def test_capacity_negative_factor_means_no_limit():
    assert M.moe_capacity(100, 2, 4, -1.0) == M.MOE_NO_CAPACITY


def test_capacity_of_non_finite_or_huge_factors():
    # NaN and +inf mean no limit; a factor whose C would pass T*k saturates at
    # T*k, which drops nothing, exactly like the unsaturated value
    assert M.moe_capacity(100, 2, 4, float("nan")) == M.MOE_NO_CAPACITY
    assert M.moe_capacity(100, 2, 4, float("inf")) == M.MOE_NO_CAPACITY
    assert M.moe_capacity(100, 2, 4, 1e300) == 200
    assert M.moe_capacity(100, 2, 4, 4.0) == O.capacity(100, 2, 4, 4.0) == 200
    # the saturated C (T*k = 8) and the unsaturated one (18) both keep all
    idx = [[0, 1], [0, 2], [0, 1], [3, 0]]
    for C in (M.moe_capacity(4, 2, 4, 9.0), O.capacity(4, 2, 4, 9.0)):
        counts, offsets, row_of, _ = O.assign(np.array(idx, dtype=np.int32), 4, C)
        assert offsets[-1] == 8 and (row_of >= 0).all()


def test_rows_max_with_a_huge_capacity_does_not_overflow():
    c = M.make_cfg(4096, 1024, 256, 8, 4096, "bf16", capacity=2**62)
    assert M.moe_rows_max(c) == 4096 * 8
    ws = M.moe_workspace_bytes(c)
    assert 0 < ws < 2**40
    c2 = M.make_cfg(4096, 1024, 256, 8, 4096, "bf16", capacity=4096 * 8)
    assert M.moe_workspace_bytes(c2) == ws


def test_rows_max_and_workspace():
    c = M.make_cfg(4096, 1024, 8, 2, 4096, "bf16", capacity=1280)
    assert M.moe_rows_max(c) == 8192
    c = M.make_cfg(32768, 4096, 128, 8, 1536, "bf16", capacity=2048)
    assert M.moe_rows_max(c) == 128 * 2048
    c = M.make_cfg(100, 32, 4, 2, 64, "f32", capacity=None)
    assert M.moe_rows_max(c) == 200
    assert M.moe_workspace_bytes(c) > 0
    c0 = M.make_cfg(0, 32, 4, 2, 64, "bf16", capacity=None)
    assert M.moe_rows_max(c0) == 0 and M.moe_workspace_bytes(c0) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), B.MOE_ERR_ARG), (dict(k=33, E=64), B.MOE_ERR_ARG),
    (dict(E=1, k=2), B.MOE_ERR_ARG), (dict(E=257), B.MOE_ERR_ARG),
    (dict(d=0), B.MOE_ERR_ARG), (dict(f=0), B.MOE_ERR_ARG),
    (dict(T=-1), B.MOE_ERR_ARG), (dict(capacity=-5), B.MOE_ERR_ARG),
    (dict(d=12), B.MOE_ERR_ALIGN), (dict(f=20), B.MOE_ERR_ALIGN),
])
def test_invalid_cfg_is_rejected(kw, status):
    base = dict(T=16, d=64, E=8, k=2, f=64, dtype="bf16", capacity=None)
    base.update(kw)
    cap = base.pop("capacity")
    c = M.make_cfg(**base, capacity=None)
    if cap is not None:
        c.capacity = cap
    assert M.moe_check_cfg(c) == status
    assert M.moe_rows_max(c) == -1 and M.moe_workspace_bytes(c) == 0


def test_bad_dtype_and_flags():
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16")
    c.dtype = 7
    assert M.moe_check_cfg(c) == B.MOE_ERR_DTYPE
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16")
    for bad in (16, 32, 1 << 31):
        c.flags = bad
        assert M.moe_check_cfg(c) == B.MOE_ERR_ARG
    for ok in (B.MOE_FLAG_RECOMPUTE, B.MOE_FLAG_RENORM, B.MOE_FLAG_SLOT_PRIORITY,
               B.MOE_FLAG_DROP_IDENTITY, 15):
        c.flags = ok
        assert M.moe_check_cfg(c) == B.MOE_OK
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16", recompute=True, renorm=True, priority="slot")
    assert c.flags == 7
    with pytest.raises(ValueError):
        M.make_cfg(16, 64, 8, 2, 64, "bf16", priority="expert")


def test_slot_priority_sizes_the_permute_workspace_for_k_t_virtual_tokens():
    tok = M.make_cfg(100000, 64, 64, 8, 64, "bf16")
    slot = M.make_cfg(100000, 64, 64, 8, 64, "bf16", priority="slot")
    # per-block expert counts: ceil(k T / 256) blocks instead of ceil(T / 256)
    extra = (-(-8 * 100000 // 256) - (-(-100000 // 256))) * 64 * 4
    grow = M.moe_workspace_bytes(slot) - M.moe_workspace_bytes(tok)
    assert extra <= grow <= extra + 256
    c = M.make_cfg(16, 12, 8, 2, 64, "f32")   # 48-byte rows: aligned for fp32
    assert M.moe_check_cfg(c) == B.MOE_OK


# Fake device addresses: validation only inspects them, never dereferences.
_A = 1 << 20


def _call_route(cfg, **over):
    args = dict(x=_A, Wr=_A, b=None, probs=_A, idx=_A, gate=_A, ws=_A,
                ws_bytes=M.moe_workspace_bytes(cfg))
    args.update(over)
    return B.lib.moe_route(ctypes.byref(cfg), args["x"], args["Wr"], args["b"],
                           args["probs"], args["idx"], args["gate"], args["ws"],
                           args["ws_bytes"], None)


def test_entry_points_reject_bad_arguments_before_launch():
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16")
    assert _call_route(c, x=None) == B.MOE_ERR_ARG
    assert _call_route(c, probs=None) == B.MOE_ERR_ARG
    assert _call_route(c, x=_A + 2) == B.MOE_ERR_ALIGN
    assert _call_route(c, ws_bytes=10) == B.MOE_ERR_WORKSPACE
    assert _call_route(c, ws=None) == B.MOE_ERR_ARG
    bad = M.make_cfg(16, 64, 8, 2, 64, "bf16")
    bad.k = 9
    assert _call_route(bad) == B.MOE_ERR_ARG
    assert B.lib.moe_combine(ctypes.byref(c), None, _A, _A, None, _A, None) == B.MOE_ERR_ARG
    assert B.lib.moe_permute(ctypes.byref(c), _A, _A, _A, _A, _A, _A, _A, _A, 0,
                             None) == B.MOE_ERR_WORKSPACE
    assert B.lib.moe_layer_fwd(ctypes.byref(c), None, _A, _A, None, _A, 1 << 30,
                               None) == B.MOE_ERR_ARG
    # a probe with an unknown kernel id, or events missing, is rejected
    probe = B.MoeProbe(kernel_id=99, capacity=1, count=0)
    c.probe = ctypes.addressof(probe)
    assert B.lib.moe_check_cfg(ctypes.byref(c)) == B.MOE_ERR_ARG
    probe.kernel_id = B.KERNELS["GEMM_DH"]
    assert B.lib.moe_check_cfg(ctypes.byref(c)) == B.MOE_ERR_ARG  # begin/end NULL
    probe.capacity = 0
    assert B.lib.moe_check_cfg(ctypes.byref(c)) == B.MOE_OK


def test_noalloc_permute_validates_before_anything_else():
    # argument checks and the scratch-size check need no GPU
    c = M.make_cfg(1000, 64, 16, 2, 64, "bf16", capacity=None)
    f = B.lib.moe_permute_noalloc
    assert f(ctypes.byref(c), None, _A, _A, _A, _A, _A, _A, None) == B.MOE_ERR_ARG
    assert f(ctypes.byref(c), _A + 2, _A, _A, _A, _A, _A, _A, None) == B.MOE_ERR_ALIGN
    big = M.make_cfg(2 ** 22, 64, 256, 2, 64, "bf16", capacity=None)
    assert f(ctypes.byref(big), _A, _A, _A, _A, _A, _A, _A, None) == B.MOE_ERR_WORKSPACE
    assert b"4194304 available" in B.lib.moe_last_error()


def test_cfg_copies_field_by_field():
    import copy
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16", capacity=5, aux_coeff=0.5)
    probe = B.MoeProbe(kernel_id=1, capacity=0, count=0)
    c.probe = ctypes.addressof(probe)
    c2 = copy.copy(c)
    c2.aux_coeff = 1.0
    assert c.aux_coeff == 0.5 and c2.capacity == 5 and c2.probe == c.probe


def test_status_strings():
    for st in range(-7, 1):
        assert M.status_str(st) and M.status_str(st) != "unknown status"
    assert M.status_str(-99) == "unknown status"


def test_cfg_struct_layout_matches_header():
    # int64 T; 5 x int32; int64 capacity (8-aligned); float; uint32; float
    # aux_coeff -> 52 bytes, padded to 56 for the probe pointer
    assert ctypes.sizeof(B.MoeCfg) == 64
    assert B.MoeCfg.capacity.offset == 32 and B.MoeCfg.flags.offset == 44
    assert B.MoeCfg.aux_coeff.offset == 48 and B.MoeCfg.probe.offset == 56
    assert ctypes.sizeof(B.MoeProbe) == 32 and B.MoeProbe.begin.offset == 16
    # MoeCtx: eleven tensors, then the optional diagnostics output
    assert B.MoeCtx.aux.offset == 11 * ctypes.sizeof(ctypes.c_void_p)


def test_recompute_mode_moves_a_and_h_into_the_workspace():
    base = M.make_cfg(1000, 64, 8, 2, 96, "bf16", capacity=300)
    rec = M.make_cfg(1000, 64, 8, 2, 96, "bf16", capacity=300, recompute=True)
    Rmax = M.moe_rows_max(base)
    grow = M.moe_workspace_bytes(rec) - M.moe_workspace_bytes(base)
    # two [Rmax, f] bf16 regions, each rounded up to 256 bytes
    assert 2 * Rmax * 96 * 2 <= grow <= 2 * Rmax * 96 * 2 + 512
    ws = M.moe_workspace_bytes(rec)
    # A and H may be NULL under the flag (validation then stops at ws_bytes)
    ffn = lambda cfg, A, H: B.lib.moe_grouped_ffn(ctypes.byref(cfg), _A, _A, _A, _A, A, H,
                                                  _A, _A, 10, None)
    assert ffn(base, None, None) == B.MOE_ERR_ARG
    assert ffn(rec, None, None) == B.MOE_ERR_WORKSPACE
    bwd = lambda cfg: B.lib.moe_grouped_ffn_bwd(ctypes.byref(cfg), _A, _A, _A, _A, None, None,
                                                _A, _A, _A, _A, _A, 10, None)
    assert bwd(base) == B.MOE_ERR_ARG
    assert bwd(rec) == B.MOE_ERR_WORKSPACE
    assert ws > 0


def test_identity_fallback_entry_points_need_its_extra_inputs():
    plain = M.make_cfg(16, 64, 8, 2, 64, "bf16")
    fb = M.make_cfg(16, 64, 8, 2, 64, "bf16", fallback="identity")
    assert fb.flags == B.MOE_FLAG_DROP_IDENTITY and M.moe_check_cfg(fb) == B.MOE_OK
    with pytest.raises(ValueError):
        M.make_cfg(16, 64, 8, 2, 64, "bf16", fallback="zero")
    # combine: x only under the flag (a NULL out stops a valid call first)
    comb = lambda cfg, x: B.lib.moe_combine(ctypes.byref(cfg), _A, _A, _A, x, None, None)
    assert comb(plain, None) == B.MOE_ERR_ARG and comb(fb, None) == B.MOE_ERR_ARG
    assert B.lib.moe_combine(ctypes.byref(fb), _A, _A, _A, _A + 2, _A, None) == B.MOE_ERR_ALIGN
    cb = lambda cfg, x: B.lib.moe_combine_bwd(ctypes.byref(cfg), _A, _A, _A, _A, x, _A, None,
                                              None)
    assert cb(plain, None) == B.MOE_ERR_ARG   # dgate NULL
    assert cb(fb, _A + 2) == B.MOE_ERR_ALIGN
    ub = lambda cfg, g, dO: B.lib.moe_unpermute_bwd(ctypes.byref(cfg), _A, _A, g, dO, None,
                                                    None)
    assert ub(fb, None, _A) == B.MOE_ERR_ARG and ub(fb, _A, None) == B.MOE_ERR_ARG
    assert ub(plain, None, None) == B.MOE_ERR_ARG  # dXe NULL
    # the router backward takes the finished unpermute-sum: no fallback inputs
    rb = lambda cfg, dxe: B.lib.moe_route_bwd(
        ctypes.byref(cfg), _A, _A, _A, _A, _A, None, _A, dxe, _A, _A, None, _A, 10, None)
    assert rb(fb, None) == B.MOE_ERR_ARG and rb(plain, None) == B.MOE_ERR_ARG
    assert rb(fb, _A + 4) == B.MOE_ERR_ALIGN
    assert rb(fb, _A) == B.MOE_ERR_WORKSPACE
    assert rb(plain, _A) == B.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("coeff", [-0.01, float("nan"), float("inf")])
def test_invalid_balancing_coefficient_is_rejected(coeff):
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16", aux_coeff=coeff)
    assert M.moe_check_cfg(c) == B.MOE_ERR_ARG
    assert M.moe_workspace_bytes(c) == 0


def test_balancing_entry_points_validate_arguments():
    c = M.make_cfg(16, 64, 8, 2, 64, "bf16", aux_coeff=0.01)
    assert M.moe_check_cfg(c) == B.MOE_OK
    ws = M.moe_workspace_bytes(c)
    aux = B.lib.moe_router_aux
    assert aux(ctypes.byref(c), None, _A, _A, _A, _A, ws, None) == B.MOE_ERR_ARG
    assert aux(ctypes.byref(c), _A, None, _A, _A, _A, ws, None) == B.MOE_ERR_ARG
    assert aux(ctypes.byref(c), _A, _A, None, _A, _A, ws, None) == B.MOE_ERR_ARG
    assert aux(ctypes.byref(c), _A, _A, _A, None, _A, ws, None) == B.MOE_ERR_ARG
    assert aux(ctypes.byref(c), _A, _A, _A, _A + 2, _A, ws, None) == B.MOE_ERR_ALIGN
    assert aux(ctypes.byref(c), _A, _A, _A, _A, _A, 10, None) == B.MOE_ERR_WORKSPACE
    # the router backward needs counts only when the loss is on
    rb = lambda cfg, counts: B.lib.moe_route_bwd(
        ctypes.byref(cfg), _A, _A, _A, _A, _A, counts, _A, _A, _A, _A, None, _A, 10, None)
    assert rb(c, None) == B.MOE_ERR_ARG
    assert rb(c, _A) == B.MOE_ERR_WORKSPACE
    c.aux_coeff = 0.0
    assert rb(c, None) == B.MOE_ERR_WORKSPACE


def test_binding_has_no_oracle_dependency(repo_root):
    pkg = os.path.join(repo_root, "expert_router_gemm_softmax_amd")
    for root, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(root, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn


def test_workload_shapes_are_the_named_configs():
    assert (W.get("C1").T, W.get("C1").d, W.get("C1").E, W.get("C1").k, W.get("C1").f) == \
        (4096, 1024, 8, 2, 4096)
    assert W.get("C4").cf == 1.0 and W.get("C2").cf is None


def test_one_hip_runtime_in_the_process(repo_root):
    """libmoe.so must share torch's HIP runtime (pointers and streams come
    from it), whatever the import order."""
    import subprocess
    import sys
    for order in ("import expert_router_gemm_softmax_amd, torch",
                  "import torch, expert_router_gemm_softmax_amd"):
        code = order + ("; print(len({l.split()[-1] for l in open('/proc/self/maps') "
                        "if 'libamdhip64' in l}))")
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           cwd=repo_root, timeout=300)
        assert r.returncode == 0, r.stderr[-500:]
        assert r.stdout.strip() == "1", (order, r.stdout)


def test_plain_c_program_uses_the_c_abi(repo_root, tmp_path):
    """include/moe.h compiles as C99 and a C program linked against libmoe.so
    runs the host-side entry points (no GPU, no Python in the program)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_host"
    lib_dir = os.path.join(repo_root, "expert_router_gemm_softmax_amd")
    cmd = [cc, "-std=c99", "-Wall", "-Werror", "-pedantic",
           "-I", os.path.join(repo_root, "include"),
           os.path.join(repo_root, "tests", "c_abi", "abi_host.c"),
           "-L", lib_dir, "-lmoe", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "all host checks passed" in r.stdout


def test_binding_refuses_host_tensors():
    # checked before any library call, so no GPU is needed
    import torch
    assert B._ptr(None) is None and B._ptr(1024) == 1024
    with pytest.raises(ValueError, match="GPU memory only"):
        B._ptr(torch.zeros(4, 4))
    c = M.make_cfg(64, 64, 4, 2, 64, "bf16")
    with pytest.raises(ValueError, match="GPU memory only"):
        M.moe_combine(c, torch.zeros(128, 64), None, None, None)
