"""Host-side checks of libapmoe: it loads, exports every entry point the header
declares, validates arguments before touching the GPU, and its host planner
agrees bit-exactly with the planner oracle.  No GPU compute is called."""
import ctypes
import subprocess

import numpy as np
import pytest

import synth
from any_precision_quantized_amd import _lib
from oracle import planner as planner_ref


def test_library_exports_header_symbols():
    lib = _lib._lib()
    names = _lib.header_symbols()
    assert len(names) == 30, names
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in nm.splitlines() if line.strip()}
    assert set(names) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", _lib.HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_strerror():
    for code in (0, -1, -2, -3, -4, -99):
        assert isinstance(_lib.strerror(code), str) and _lib.strerror(code)


def test_validation_before_launch():
    lib = _lib._lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    # route: k > E, bad scale, null pointers
    big = 1 << 20
    assert lib.apmoe_route(fake, 4, 64, fake, None, 1.0, 8, 9, fake, fake, None, fake, big, None) == _lib.EINVAL
    assert lib.apmoe_route(fake, 4, 64, fake, None, 0.0, 8, 2, fake, fake, None, fake, big, None) == _lib.EINVAL
    assert lib.apmoe_route(None, 4, 64, fake, None, 1.0, 8, 2, fake, fake, None, fake, big, None) == _lib.EINVAL
    assert lib.apmoe_route(fake, 4, 64, fake, None, 1.0, 300, 2, fake, fake, None, fake, big, None) == _lib.EINVAL
    assert lib.apmoe_route(fake, 4, 48, fake, None, 1.0, 8, 2, fake, fake, None, fake, big, None) == _lib.EINVAL   # H % 32
    assert lib.apmoe_route(ctypes.c_void_p(0x1002), 4, 64, fake, None, 1.0, 8, 2, fake, fake, None, fake, big,
                           None) == _lib.EINVAL   # x not 16-byte aligned
    # partial logits of several expert tiles are staged in the workspace
    assert lib.apmoe_route(fake, 4096, 4096, fake, None, 1.0, 256, 2, fake, fake, None, fake,
                           4096 * 256 * 8 - 1, None) == _lib.ENOSPACE
    assert lib.apmoe_route(fake, 4096, 4096, fake, None, 1.0, 256, 2, fake, fake, None, None, big, None) == _lib.ENOSPACE
    assert lib.apmoe_route(None, 0, 64, None, None, 1.0, 8, 2, None, None, None, None, 0, None) == _lib.OK   # T = 0
    assert _lib.workspace_bytes(4096, 2, 256, 4096, 64) >= 4096 * 256 * 8   # staged router logits
    # route statistics
    assert lib.apmoe_route_stats(fake, 4, 64, fake, fake, 9, 8, fake, fake, fake, big, None) == _lib.EINVAL   # k > E
    assert lib.apmoe_route_stats(fake, 4, 48, fake, fake, 2, 8, fake, fake, fake, big, None) == _lib.EINVAL   # H % 32
    assert lib.apmoe_route_stats(fake, 4, 64, fake, fake, 2, 8, None, fake, fake, big, None) == _lib.EINVAL
    assert lib.apmoe_route_stats(fake, 4, 64, fake, fake, 2, 8, fake, fake, fake, 15, None) == _lib.ENOSPACE
    assert lib.apmoe_route_stats(fake, 4, 64, fake, fake, 2, 8, fake, fake, None, big, None) == _lib.ENOSPACE
    # online planner: no stages, a stage bitwidth that is not a level
    lv = np.array([6, 5, 4, 3], np.int8)
    hm = np.zeros((2, 4))
    nb = np.array([[600, 500, 400, 300]] * 2, dtype=np.uint64)
    fl = np.array([3, 3], np.int8)
    now = np.array([6, 6], np.int8)
    out = np.zeros(2, np.int8)
    stage = ctypes.c_int(0)
    for sb, n in ((np.array([4], np.int8), 0), (np.array([7], np.int8), 1)):
        assert lib.apmoe_plan_online(2, 4, lv.ctypes.data, hm.ctypes.data, nb.ctypes.data, fl.ctypes.data, n,
                                     sb.ctypes.data, 2000, 0, 0, now.ctypes.data, out.ctypes.data,
                                     ctypes.byref(stage)) == _lib.EINVAL
    # permute
    assert lib.apmoe_permute(fake, 4, 0, 8, 0, fake, fake, fake, fake, None, None, None, None, None, 0, None) == _lib.EINVAL
    assert lib.apmoe_permute(None, 4, 2, 8, 0, fake, fake, fake, fake, None, None, None, None, None, 0, None) == _lib.EINVAL
    assert lib.apmoe_permute(fake, 4, 2, 8, -1, fake, fake, fake, fake, None, None, None, None, None, 0, None) == _lib.EINVAL
    assert lib.apmoe_permute(fake, 4, 2, 250, 7, fake, fake, fake, fake, None, None, None, None, None, 0, None) == _lib.EINVAL   # E + n > 256
    assert lib.apmoe_permute(None, 0, 2, 8, 0, None, None, None, None, None, None, None, None, None, 0, None) == _lib.OK
    # permute with routing statistics: wnorm, topk_w and x_norms are required,
    # and the workspace must hold S * 8 bytes (S = T * (k + n_shared) = 4 * 3)
    pm = lib.apmoe_permute
    assert pm(fake, 4, 2, 8, 1, fake, fake, fake, fake, fake, fake, fake, None, fake, big, None) == _lib.EINVAL
    assert pm(fake, 4, 2, 8, 1, fake, fake, fake, fake, None, fake, fake, fake, fake, big, None) == _lib.EINVAL
    assert pm(fake, 4, 2, 8, 1, fake, fake, fake, fake, fake, fake, fake, fake, fake, 4 * 3 * 8 - 1, None) == _lib.ENOSPACE
    # gemm: bad stage, H or I not a multiple of 32, mfma_min_tokens < 1
    g = lib.apmoe_bitplane_lut_gemm
    assert g(7, fake, fake, 8, fake, fake, 2, fake, fake, 4, 64, 64, 16, None, 0, None) == _lib.EINVAL
    assert g(0, fake, fake, 8, fake, fake, 2, fake, fake, 4, 65, 64, 16, None, 0, None) == _lib.EINVAL
    assert g(1, fake, fake, 8, fake, fake, 2, fake, fake, 4, 64, 48, 16, None, 0, None) == _lib.EINVAL
    assert g(0, fake, fake, 8, fake, fake, 2, fake, fake, 4, 64, 64, 0, None, 0, None) == _lib.EINVAL
    assert g(0, fake, fake, 8, fake, None, 2, fake, fake, 4, 64, 64, 16, None, 0, None) == _lib.EINVAL
    assert g(0, None, None, 8, None, None, 2, None, None, 0, 64, 64, 16, None, 0, None) == _lib.OK
    # buffers past the kernels' 32-bit byte offsets are refused before any launch:
    # x of T * H * 2 = 2 GiB (gate/up), A of T * k * I * 2 = 2 GiB (down), a
    # 2 GiB fp16 matrix; one element less passes validation up to the workspace check
    assert g(0, fake, fake, 8, fake, fake, 2, fake, fake, 1 << 18, 4096, 64, 16, fake, big, None) == _lib.EINVAL
    assert g(1, fake, fake, 8, fake, fake, 2, fake, fake, 1 << 16, 64, 8192, 16, fake, big, None) == _lib.EINVAL
    assert g(1, fake, fake, 8, fake, fake, 2, fake, fake, 4, 32768, 32768, 16, fake, big, None) == _lib.EINVAL
    # (over 32 experts, whose router stages partial logits, so the workspace is not empty)
    assert g(0, fake, fake, 32, fake, fake, 2, fake, fake, (1 << 18) - 1, 4096, 64, 16, fake, 0, None) == _lib.ENOSPACE
    # the allocation-free stage refuses shapes whose split-K partials exceed its
    # static scratch before touching the GPU: 16384 tokens over 4 experts of 64
    # rows, K = 14336 split in 4: 4 * 16384 * 2 * 64 * 4 bytes = 32 MiB > 16 MiB
    na = lib.apmoe_bitplane_lut_gemm_noalloc
    assert na(0, fake, fake, 4, fake, fake, 1, fake, fake, 16384, 14336, 64, 1 << 30, None) == _lib.ENOSPACE
    assert na(7, fake, fake, 8, fake, fake, 2, fake, fake, 4, 64, 64, 16, None) == _lib.EINVAL
    assert na(0, None, None, 8, None, None, 2, None, None, 0, 64, 64, 16, None) == _lib.OK
    # combine
    assert lib.apmoe_combine(fake, fake, fake, 4, 2, 0, 48, None, fake, None) == _lib.EINVAL
    assert lib.apmoe_combine(None, fake, fake, 4, 2, 0, 64, None, fake, None) == _lib.EINVAL
    assert lib.apmoe_combine(fake, fake, fake, 4, 2, -1, 64, None, fake, None) == _lib.EINVAL
    # pack: rows not a multiple of 16, cols not a multiple of 32, overlap
    assert lib.apmoe_pack_planes(fake, 24, 64, ctypes.c_void_p(0x100000), None) == _lib.EINVAL
    assert lib.apmoe_pack_planes(fake, 32, 48, ctypes.c_void_p(0x100000), None) == _lib.EINVAL
    assert lib.apmoe_pack_planes(fake, 32, 64, fake, None) == _lib.EINVAL
    assert _lib.packed_plane_words(32, 704) == 6 * 32 * 4 * 6
    # commit: invalid bitwidth rejected on the host
    bad = (ctypes.c_int8 * 3)(6, 7, 3)
    assert lib.apmoe_commit_bits(bad, 3, fake, None) == _lib.EBITS
    assert lib.apmoe_commit_bits(bad, 0, fake, None) == _lib.EINVAL


@pytest.mark.parametrize("seed", range(20))
def test_host_planner_matches_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    levels = [16, 6, 5, 4, 3] if seed % 2 else [6, 5, 4, 3]
    E = int(rng.integers(1, 40))
    L = len(levels)
    size = rng.integers(1000, 10**7, size=E)
    nb = np.array([[int(s * b / 16) + 31 for b in levels] for s in size], dtype=np.uint64)
    harm = np.cumsum(rng.random((E, L)), axis=1) * rng.random((E, 1))
    harm -= harm[:, :1]
    if seed % 3 == 0:
        harm = np.round(harm, 1)          # many exact ties in cost
    floors = np.array([rng.choice(levels[1:]) for _ in range(E)], dtype=np.int8)
    lo = planner_ref.plan_total(levels, nb, floors)
    hi = planner_ref.plan_total(levels, nb, [levels[0]] * E)
    for budget in list(np.linspace(lo, hi, 9).astype(np.int64)) + [lo - 1]:
        st_ref, bits_ref = planner_ref.plan_bitwidths(levels, harm, nb, floors, int(budget))
        st, bits = _lib.plan_bitwidths(levels, harm, nb, floors, int(budget))
        assert st == st_ref
        assert np.array_equal(bits, bits_ref)


def test_host_planner_zipf_plan():
    cfg = synth.get("qwen_decode")
    p = synth.gen.zipf_prior(cfg.E, cfg.zipf_s)
    plan = synth.planner_inputs(cfg, p)
    args = (plan["levels"], plan["harm"], plan["bytes"], plan["floors"], plan["budget"])
    st, bits = _lib.plan_bitwidths(*args)
    st_ref, bits_ref = planner_ref.plan_bitwidths(*args)
    assert st == st_ref == 0
    assert np.array_equal(bits, bits_ref)


def test_host_planner_rejects_bad_inputs():
    st, _ = _lib.plan_bitwidths([6, 7, 4], np.zeros((2, 3)), np.array([[3, 2, 1]] * 2), [4, 4], 10)
    assert st == _lib.EBITS
    st, _ = _lib.plan_bitwidths([6, 5, 4], np.zeros((2, 3)), np.array([[3, 3, 1]] * 2), [4, 4], 10)
    assert st == _lib.EINVAL
    st, _ = _lib.plan_bitwidths([6, 5, 4], np.zeros((2, 3)), np.array([[3, 2, 1]] * 2), [3, 4], 10)
    assert st == _lib.EINVAL


def test_workspace_covers_routers_over_fewer_experts():
    """One workspace serves the router over the routed experts and the expert
    stages over routed + always-on experts: the size never shrinks as E grows,
    and the router's counters sit past the GEMM's bytes."""
    for T in (1, 16, 64, 256, 8192):
        for H in (256, 2048, 2816, 4096):
            prev = 0
            for E in range(1, 257):
                n = _lib.workspace_bytes(T, 2, E, H, 1408)
                assert n >= prev, (T, H, E)
                prev = n
