"""CPU tests of the C ABI boundary: the library loads, exports every entry point
include/fa.h declares, and rejects invalid arguments before launching anything.
No test here reaches a kernel launch (there is no GPU on this host)."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def L():
    # Most tests here pass fake device pointers that validation must reject; on a host with a
    # GPU a case that validation let through would launch on them, so they run only without one.
    import torch
    if torch.cuda.is_available():
        pytest.skip("boundary validation tests use fake device pointers; run them on a host without a GPU")
    from exact_attention_102_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from exact_attention_102_amd import build
        build.build()
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), "libfa.so does not export " + n


def test_status_strings_and_version(L):
    from exact_attention_102_amd import fa_status_string, fa_version
    assert fa_status_string(0) == "FA_OK"
    for s in range(1, 5):
        assert fa_status_string(s).startswith("FA_ERR_")
    assert "gfx950" in fa_version()


def test_config_tables(L):
    from exact_attention_102_amd import fa_config_name, fa_default_config, fa_num_configs
    for p in range(4):
        for d in (64, 128, 256, 288, 384):
            n = fa_num_configs(p, d)
            assert n >= 1
            names = [fa_config_name(p, d, False, i) for i in range(n)]
            assert all(("d%d" % d) in s for s in names)
            assert 0 <= fa_default_config(p, d) < n
            with pytest.raises(IndexError):
                fa_config_name(p, d, False, n)
        assert fa_num_configs(p, 100) == 0
        assert fa_default_config(p, 100) == -1


P = 0x7f0000000000            # fake, 16-byte aligned, never dereferenced (validation fails first)
MB = 1 << 20


def fwd(L, q=P, k=P + 64 * MB, v=P + 128 * MB, B=1, H=1, N=128, d=64, causal=0, scale=0.125,
        o=P + 192 * MB, lse=P + 256 * MB):
    return L.fa_fwd(ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), B, H, N, d, causal, scale,
                    ctypes.c_void_p(o), ctypes.c_void_p(lse), None)


def test_fwd_rejects_bad_arguments(L):
    from exact_attention_102_amd import FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED
    assert fwd(L, q=0) == FA_ERR_INVALID_ARG
    assert fwd(L, o=0) == FA_ERR_INVALID_ARG
    assert fwd(L, lse=0) == FA_ERR_INVALID_ARG
    assert fwd(L, q=P + 8) == FA_ERR_INVALID_ARG          # misaligned
    assert fwd(L, B=0) == FA_ERR_INVALID_ARG
    assert fwd(L, H=-1) == FA_ERR_INVALID_ARG
    assert fwd(L, N=0) == FA_ERR_INVALID_ARG
    assert fwd(L, d=100) == FA_ERR_UNSUPPORTED
    assert fwd(L, d=0) == FA_ERR_UNSUPPORTED
    assert fwd(L, scale=0.0) == FA_ERR_INVALID_ARG
    assert fwd(L, scale=-1.0) == FA_ERR_INVALID_ARG
    assert fwd(L, scale=float("nan")) == FA_ERR_INVALID_ARG
    assert fwd(L, scale=float("inf")) == FA_ERR_INVALID_ARG
    assert fwd(L, o=P) == FA_ERR_INVALID_ARG               # output aliases q
    assert fwd(L, lse=P + 192 * MB + 64) == FA_ERR_INVALID_ARG   # lse inside o
    assert fwd(L, B=65536, H=65536) == FA_ERR_INVALID_ARG  # row count beyond 32-bit
    assert L.fa_fwd_ex(ctypes.c_void_p(P), ctypes.c_void_p(P + 64 * MB), ctypes.c_void_p(P + 128 * MB), 1, 1, 128,
                       64, 0, ctypes.c_float(0.125), ctypes.c_void_p(P + 192 * MB), ctypes.c_void_p(P + 256 * MB),
                       None, 99) == FA_ERR_UNSUPPORTED     # unknown tile configuration


def bwd(L, variant=1, ws=P + 900 * MB, ws_bytes=1 << 20, dq=P + 600 * MB, d=64, N=128, scale=0.125):
    args = [ctypes.c_void_p(P + i * 64 * MB) for i in range(6)]   # q k v o lse dout
    return L.fa_bwd(*args, 1, 1, N, d, 0, scale, variant, ctypes.c_void_p(dq), ctypes.c_void_p(P + 700 * MB),
                    ctypes.c_void_p(P + 800 * MB), ctypes.c_void_p(ws), ws_bytes, None)


def test_bwd_rejects_bad_arguments(L):
    from exact_attention_102_amd import FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE
    assert L.fa_bwd_workspace_size(1, 1, 128, 64, 1) == 512
    assert L.fa_bwd_workspace_size(2, 3, 1000, 128, 0) == 24064
    assert L.fa_bwd_workspace_size(1, 1, 0, 64, 1) == 0
    assert bwd(L, variant=7) == FA_ERR_UNSUPPORTED
    assert bwd(L, ws=0) == FA_ERR_WORKSPACE
    assert bwd(L, ws_bytes=100) == FA_ERR_WORKSPACE
    assert bwd(L, dq=P) == FA_ERR_INVALID_ARG              # dq aliases q
    assert bwd(L, dq=P + 700 * MB) == FA_ERR_INVALID_ARG   # dq aliases dk
    assert bwd(L, ws=P + 800 * MB) == FA_ERR_INVALID_ARG   # workspace aliases dv
    assert bwd(L, d=160) == FA_ERR_UNSUPPORTED
    assert bwd(L, scale=float("nan")) == FA_ERR_INVALID_ARG
    assert L.fa_bwd_preprocess(None, ctypes.c_void_p(P), 1, 1, 8, 64, ctypes.c_void_p(P + MB), None, 0,
                               None) == FA_ERR_INVALID_ARG
    assert L.fa_bwd_preprocess(ctypes.c_void_p(P), ctypes.c_void_p(P + MB), 1, 1, 8, 64, ctypes.c_void_p(P + 2 * MB),
                               None, 1, None) == FA_ERR_INVALID_ARG   # zero_dq without dq
    # the fused dQ stage: o is required, and the delta it writes may alias neither o nor dq
    ptrs = [ctypes.c_void_p(P + i * MB) for i in range(4)]   # q k v dout
    lse = ctypes.c_void_p(P + 4 * MB)

    def dqd(o, delta, dq):
        return L.fa_bwd_dq_delta(*ptrs[:3], o, ptrs[3], lse, 1, 1, 8, 64, 0, 0.125, delta, dq, None, -1)
    o, delta, dq = ctypes.c_void_p(P + 5 * MB), ctypes.c_void_p(P + 6 * MB), ctypes.c_void_p(P + 7 * MB)
    assert dqd(None, delta, dq) == FA_ERR_INVALID_ARG
    assert dqd(o, o, dq) == FA_ERR_INVALID_ARG               # delta aliases o
    assert dqd(o, dq, dq) == FA_ERR_INVALID_ARG              # delta aliases dq
    assert dqd(o, delta, o) == FA_ERR_INVALID_ARG            # dq aliases o
    assert dqd(o, delta, ctypes.c_void_p(P)) == FA_ERR_INVALID_ARG   # dq aliases q


def test_heads_of_2gib_or_more_rejected(L):
    """One head of a bf16 input must stay below 2^31 bytes (N * d * 2): the tile copies
    address a head through one 32-bit buffer range and zero-fill the padded columns of
    d = 96 / 192 through an offset of 2^31, which must fall outside that range."""
    from exact_attention_102_amd import FA_ERR_INVALID_ARG
    for d in (64, 96, 128, 192, 256, 288, 384):
        n_limit = -(-(1 << 31) // (2 * d))       # smallest N with N * d * 2 >= 2^31
        assert fwd(L, N=n_limit, d=d) == FA_ERR_INVALID_ARG
        assert bwd(L, N=n_limit, d=d, ws_bytes=1 << 40) == FA_ERR_INVALID_ARG
        assert L.fa_bwd_workspace_size(1, 1, n_limit, d, 1) == 0
        assert L.fa_bwd_workspace_size(1, 1, n_limit - 1, d, 1) > 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from exact_attention_102_amd import binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


# ----------------------------------------------------------------------------- host-side accounting
def test_flop_accounting_matches_the_pages():
    from exact_attention_102_amd.flops import attention_flops, mfa_op_counts, pairs
    g = json.load(open(os.path.join(GOLDEN, "mfa_op_counts.json")))
    for d in (64, 128, 256):
        for N in (1, 128, 2048):
            c = mfa_op_counts(N, d, dispatches=g["dispatches_per_trial"])
            for k, (a, b) in g["per_pair"].items():
                assert c[k] == (a * d + b) * N * N * g["dispatches_per_trial"]
    r = json.load(open(os.path.join(GOLDEN, "gemm_ratio.json")))
    f = attention_flops(4, 16, 2048, 128, False)
    assert f["fwd"] == 2 * r["gemms"]["forward"] * 128 * f["pairs"]
    assert f["bwd_effective"] == 2 * r["gemms"]["backward_5gemm"] * 128 * f["pairs"]
    assert f["bwd_7gemm_issued"] == 2 * r["gemms"]["backward_7gemm"] * 128 * f["pairs"]
    assert f["bwd_7gemm_issued"] / f["bwd_effective"] == pytest.approx(r["ratio_7_over_5"])
    assert r["h100_5gemm_bwd_tflops"] * r["ratio_7_over_5"] == pytest.approx(r["h100_7gemm_breakeven_tflops"])
    assert pairs(2048, False, 4, 16) == 4 * 16 * 2048 * 2048
    assert pairs(5, True) == 15 and pairs(1, True) == 1
    assert pairs(2048, True) == sum(i + 1 for i in range(2048))


def test_block_size_rule_toy_example():
    from exact_attention_102_amd.flops import block_size_rule
    g = json.load(open(os.path.join(GOLDEN, "block_size_rule.json")))
    assert block_size_rule(g["M"], g["d"]) == g["block"]
    # 160 KiB of LDS in bf16 elements: 81920 -> d=64: 320, d=128: 160, d=256: 80
    assert [block_size_rule(81920, d) for d in (64, 128, 256)] == [320, 160, 80]


def test_d_spectrum_matches_the_page():
    from exact_attention_102_amd.flops import d_spectrum
    g = json.load(open(os.path.join(GOLDEN, "d_spectrum.json")))
    assert d_spectrum() == g["values"]
    assert len(g["values"]) == 42


def test_report_tile_counts_match_brute_force():
    """Tile accounting of the per-configuration report: loaded tiles per head for the query-major passes
    (forward, dQ) and the key-major dK/dV pass, against an explicit walk over the tile grid."""
    import itertools

    from exact_attention_102_amd.report import tile_shape, tiles

    assert tile_shape("fwd d128 Br32x4 Bc64 occ2") == (128, 64)
    assert tile_shape("dkdv+atomic-dq d64 Bk32x8 Bq64 kv_regs deferred") == (256, 64)

    def walk(N, rows, cols, causal, keys_major):
        nr, nc = -(-N // rows), -(-N // cols)
        seen = 0
        for r, c in itertools.product(range(nr), range(nc)):
            if keys_major:  # key block r meets query tile c unless every query precedes every key
                seen += (not causal) or min(N, (c + 1) * cols) - 1 >= r * rows
            else:  # query block r meets key tile c unless every key follows every query
                seen += (not causal) or c * cols <= min(N, (r + 1) * rows) - 1
        return seen, nr * nc

    for N, rows, cols, causal, km in itertools.product([1, 33, 300, 2048], [64, 128, 256], [32, 64], [False, True],
                                                      [False, True]):
        assert tiles(N, rows, cols, causal, km) == walk(N, rows, cols, causal, km)


def test_general_entries_validate_before_launching(L):
    """Any head dim 1..384 and strided views: sizes of the padded workspace and the error paths (no
    call here reaches a launch)."""
    from exact_attention_102_amd import FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE
    from exact_attention_102_amd.binding import FaStrides

    def a256(x):
        return (x + 255) // 256 * 256

    B, H, N = 2, 3, 77
    for d, dp in ((1, 64), (40, 64), (64, 64), (65, 96), (96, 96), (127, 128), (160, 192), (192, 192), (256, 256),
                  (257, 288), (300, 320), (352, 352), (384, 384)):
        el = B * H * N * dp
        assert L.fa_fwd_general_workspace_size(B, H, N, d) == 3 * a256(2 * el) + a256(4 * el)
        assert L.fa_bwd_general_workspace_size(B, H, N, d, 1) == 4 * a256(2 * el) + 4 * a256(4 * el) + a256(4 * B * H * N)
    assert L.fa_fwd_general_workspace_size(B, H, N, 0) == 0
    assert L.fa_fwd_general_workspace_size(B, H, N, 385) == 0
    assert L.fa_bwd_general_workspace_size(B, H, N, 96, 5) == 0

    # d = 100 is not a multiple of 8, so these calls take the padded-copy path, the one that
    # needs the workspace; every case below fails validation before anything is launched
    d = 100
    c = FaStrides(H * N * d, N * d, d)            # contiguous
    t = FaStrides(N * H * d, d, H * d)            # a [B, N, H, d] tensor seen as [B, H, N, d]
    ws_need = L.fa_fwd_general_workspace_size(B, H, N, d)

    def gfwd(q=P, qs=t, o=P + 192 * MB, os_=c, lse=P + 256 * MB, ws=P + 512 * MB, wsb=ws_need, d=d, scale=0.1):
        return L.fa_fwd_general(ctypes.c_void_p(q), qs, ctypes.c_void_p(P + 64 * MB), t, ctypes.c_void_p(P + 128 * MB),
                                t, B, H, N, d, 1, scale, ctypes.c_void_p(o), os_, ctypes.c_void_p(lse),
                                ctypes.c_void_p(ws), wsb, None)

    assert gfwd(d=0) == FA_ERR_UNSUPPORTED
    assert gfwd(d=385) == FA_ERR_UNSUPPORTED
    assert gfwd(q=0) == FA_ERR_INVALID_ARG
    assert gfwd(q=P + 1) == FA_ERR_INVALID_ARG                 # bf16 view on an odd byte address
    assert gfwd(lse=P + 256 * MB + 4) == FA_ERR_INVALID_ARG    # lse must be 16-byte aligned
    assert gfwd(qs=FaStrides(-1, d, H * d)) == FA_ERR_INVALID_ARG
    assert gfwd(o=P + 8) == FA_ERR_INVALID_ARG                 # o overlaps q
    assert gfwd(scale=float("nan")) == FA_ERR_INVALID_ARG
    assert gfwd(ws=0) == FA_ERR_WORKSPACE
    assert gfwd(wsb=ws_need - 1) == FA_ERR_WORKSPACE
    assert gfwd(ws=P + 192 * MB + 256) == FA_ERR_INVALID_ARG   # workspace overlaps o

    bneed = L.fa_bwd_general_workspace_size(B, H, N, d, 1)

    def gbwd(variant=1, dq=P + 600 * MB, ws=P + 1024 * MB, wsb=bneed):
        views = []
        for i in range(4):   # q k v o
            views += [ctypes.c_void_p(P + i * 64 * MB), t]
        return L.fa_bwd_general(*views, ctypes.c_void_p(P + 320 * MB), ctypes.c_void_p(P + 384 * MB), t, B, H, N, d,
                                0, 0.1, variant, ctypes.c_void_p(dq), c, ctypes.c_void_p(P + 700 * MB), c,
                                ctypes.c_void_p(P + 800 * MB), c, ctypes.c_void_p(ws), wsb, None)

    assert gbwd(variant=3) == FA_ERR_UNSUPPORTED
    assert gbwd(ws=0) == FA_ERR_WORKSPACE
    assert gbwd(wsb=bneed - 16) == FA_ERR_WORKSPACE
    assert gbwd(dq=P + 700 * MB) == FA_ERR_INVALID_ARG         # dq overlaps dk
    assert gbwd(dq=P + 64 * MB) == FA_ERR_INVALID_ARG          # dq overlaps k

    # d = 96 with 16-byte aligned rows runs in place (the kernels pad the head dim): the backward
    # then needs only the row-term workspace of the padded size, checked before any launch
    d = 96
    t = FaStrides(N * H * d, d, H * d)
    c = FaStrides(H * N * d, N * d, d)
    inplace_need = L.fa_bwd_workspace_size(B, H, N, 96, 1)
    assert 0 < inplace_need < L.fa_bwd_general_workspace_size(B, H, N, d, 1)
    assert gbwd(ws=0) == FA_ERR_WORKSPACE
    assert gbwd(wsb=inplace_need - 16) == FA_ERR_WORKSPACE
    assert gbwd(ws=P + 700 * MB + 256) == FA_ERR_INVALID_ARG   # workspace overlaps dk
    assert gbwd(dq=P + 64 * MB) == FA_ERR_INVALID_ARG          # dq overlaps k


def test_dropout_entries_validate_and_keep_scale(L):
    """Dropout entry points: the keep scale is the oracle's 2^16 / (2^16 - floor(p 2^16)); p outside
    [0, 1), bad sizes and bad pointers are rejected before any launch."""
    from oracle import keep_scale

    from exact_attention_102_amd import FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE
    from exact_attention_102_amd.binding import FaDropout
    for p in (0.0, 1e-9, 0.1, 0.25, 0.5, 0.9, 1 - 2 ** -20):
        assert L.fa_dropout_keep_scale(p) == keep_scale(p)
    for p in (-0.5, 1.0, 2.0, float("nan"), float("inf")):
        assert L.fa_dropout_keep_scale(p) == -1.0

    B, H, N, d = 2, 3, 100, 64

    def dfwd(p=0.1, d=d, q=P, o=P + 64 * MB):
        return L.fa_fwd_dropout(ctypes.c_void_p(q), ctypes.c_void_p(P + 16 * MB), ctypes.c_void_p(P + 32 * MB), B, H,
                                N, d, 0, 0.125, FaDropout(p, 1234, 5), ctypes.c_void_p(o),
                                ctypes.c_void_p(P + 128 * MB), None)

    assert dfwd(p=-0.1) == FA_ERR_INVALID_ARG
    assert dfwd(p=1.0) == FA_ERR_INVALID_ARG
    assert dfwd(p=float("nan")) == FA_ERR_INVALID_ARG
    assert dfwd(d=100) == FA_ERR_UNSUPPORTED
    assert dfwd(d=320) == FA_ERR_UNSUPPORTED           # no dropout kernels above 256
    assert dfwd(q=0) == FA_ERR_INVALID_ARG
    assert dfwd(o=P + 8) == FA_ERR_INVALID_ARG         # o overlaps q
    need = L.fa_bwd_workspace_size(B, H, N, d, 1)

    def dbwd(p=0.1, variant=1, ws=P + 1024 * MB, wsb=need):
        ins = [ctypes.c_void_p(P + i * 16 * MB) for i in range(6)]
        return L.fa_bwd_dropout(*ins, B, H, N, d, 1, 0.125, FaDropout(p, 99, 0), variant,
                                ctypes.c_void_p(P + 256 * MB), ctypes.c_void_p(P + 320 * MB),
                                ctypes.c_void_p(P + 384 * MB), ctypes.c_void_p(ws), wsb, None)

    assert dbwd(p=1.5) == FA_ERR_INVALID_ARG
    assert dbwd(variant=7) == FA_ERR_UNSUPPORTED
    assert dbwd(ws=0) == FA_ERR_WORKSPACE
    assert dbwd(wsb=need - 16) == FA_ERR_WORKSPACE

    # general (strided, any d) dropout entries validate the same way (d = 100: the padded-copy path,
    # so the workspace checks apply and nothing is launched)
    from exact_attention_102_amd.binding import FaStrides
    dg = 100
    t = FaStrides(N * H * dg, dg, H * dg)
    gneed = L.fa_fwd_general_workspace_size(B, H, N, dg)

    def gfwd(p=0.1, d=dg, wsb=gneed):
        return L.fa_fwd_general_dropout(ctypes.c_void_p(P), t, ctypes.c_void_p(P + 64 * MB), t,
                                        ctypes.c_void_p(P + 128 * MB), t, B, H, N, d, 0, 0.1, FaDropout(p, 1, 0),
                                        ctypes.c_void_p(P + 192 * MB), t, ctypes.c_void_p(P + 256 * MB),
                                        ctypes.c_void_p(P + 512 * MB), wsb, None)

    assert gfwd(p=1.0) == FA_ERR_INVALID_ARG
    assert gfwd(d=300) == FA_ERR_UNSUPPORTED           # no dropout kernels above 256
    assert gfwd(wsb=gneed - 1) == FA_ERR_WORKSPACE
    bneed = L.fa_bwd_general_workspace_size(B, H, N, dg, 1)

    def gbwd(p=0.1, wsb=bneed):
        views = []
        for i in range(4):
            views += [ctypes.c_void_p(P + i * 64 * MB), t]
        return L.fa_bwd_general_dropout(*views, ctypes.c_void_p(P + 320 * MB), ctypes.c_void_p(P + 384 * MB), t, B, H,
                                        N, dg, 0, 0.1, FaDropout(p, 1, 0), 1, ctypes.c_void_p(P + 600 * MB), t,
                                        ctypes.c_void_p(P + 700 * MB), t, ctypes.c_void_p(P + 800 * MB), t,
                                        ctypes.c_void_p(P + 1024 * MB), wsb, None)

    assert gbwd(p=-1.0) == FA_ERR_INVALID_ARG
    assert gbwd(wsb=bneed - 16) == FA_ERR_WORKSPACE


def test_traffic_classifies_kernel_names():
    """The counter summary keys kernels by pass and mask from their template arguments."""
    from exact_attention_102_amd.traffic import classify
    assert classify("void fa::fwd_kernel<128, 128, 64, 4, 2, true, false>(fa::FwdArgs)") == ("fwd", "causal")
    assert classify("void fa::fwd_kernel<64, 64, 64, 8, 2, false, false>(fa::FwdArgs)") == ("fwd", "full")
    assert classify("void fa::dq_kernel<128, 128, 64, 8, 2, false, false>(fa::BwdArgs)") == ("dq", "full")
    assert classify("void fa::dkdv_kernel<128, 128, 64, 4, true, true, false, false, false>(fa::BwdArgs)") == \
        ("dkdv_atomic", "causal")
    assert classify("void fa::dkdv_kernel<128, 128, 64, 4, false, false, true, false, false>(fa::BwdArgs)") == \
        ("dkdv", "full")
    assert classify("void fa::fwd_kernel<128, 128, 64, 4, 2, false, true>(fa::FwdArgs)") is None   # dropout
    assert classify("void fa::preprocess_kernel<128>(fa::PreArgs)") == ("preprocess", None)


def test_bench_atomic_add_count():
    """Atomic adds of the fused dQ: N/BK per dq element without the mask; with the causal mask key
    tile kt starts at query row kt*BK (BK a multiple of BQ), so it adds to N - kt*BK rows."""
    import bench
    B, H, N, d, bk, bq = 2, 3, 1024, 64, 256, 64
    assert bench.atomic_adds_per_launch(B, H, N, d, False, bk, bq) == B * H * N * d * (N // bk)
    rows = sum(N - kt * bk for kt in range(N // bk))
    assert bench.atomic_adds_per_launch(B, H, N, d, True, bk, bq) == B * H * rows * d
    # ragged: padded rows past N are not added
    assert bench.atomic_adds_per_launch(1, 1, 100, 8, False, 64, 32) == 100 * 8 * 2
