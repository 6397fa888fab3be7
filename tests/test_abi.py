"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
every argument check returns its status before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

from bit_quantized_weight_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4w.h")

OK, INVALID, SHAPE, ALIGN, WS = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.lib_path()):
        pytest.fail("libq4w.so is not built (run __graft_entry__.build())")
    return binding.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["q4_pack", "q4_gemv_skinny", "q4_gemv_skinny_ws_bytes", "a8_quantize_act",
              "a8w4_gemm_prefill", "a8w4_ws_bytes", "a8w4_debug_block_acc",
              "a8w4_prepare_act", "a8w4_gemm_prepared",
              "q4_gemv_batched_ws_bytes", "q4_gemv_batched_plan", "q4_gemv_batched_run",
              "q4_gemv_skinny_noalloc",
              "q4w_status_str", "q4w_last_hip_error"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in q4w.h but not exported"


def test_status_strings(L):
    assert L.q4w_status_str(0) == b"OK"
    assert L.q4w_status_str(-4) == b"WORKSPACE"
    assert L.q4w_status_str(123) == b"UNKNOWN"


# Fake "device" addresses: aligned or not.  Every call below must be rejected
# (or be a no-op) on the host, so these are never dereferenced.
A = 1 << 20          # 16- and 256-byte aligned
U = (1 << 20) + 2    # 2-byte aligned only
NUL = None


def p(v):
    return ctypes.c_void_p(v)


def test_pack_checks(L):
    assert L.q4_pack(p(A), -1, 64, p(A), p(A), NUL) == INVALID
    assert L.q4_pack(p(A), 4, 48, p(A), p(A), NUL) == SHAPE
    assert L.q4_pack(p(A), 0, 64, p(A), p(A), NUL) == OK     # empty: no-op
    assert L.q4_pack(p(A), 4, 0, p(A), p(A), NUL) == OK
    assert L.q4_pack(NUL, 4, 64, p(A), p(A), NUL) == INVALID
    assert L.q4_pack(p(U), 4, 64, p(A), p(A), NUL) == ALIGN
    assert L.q4_pack(p(A), 4, 64, p(U), p(A), NUL) == ALIGN
    assert L.q4_pack(p(A), 4, 64, p(A), p(A + 1), NUL) == ALIGN


def test_gemv_checks(L):
    g = L.q4_gemv_skinny
    assert g(p(A), p(A), p(A), p(A), 0, 64, 64, 0, NUL, 0, NUL) == SHAPE    # M < 1
    assert g(p(A), p(A), p(A), p(A), 17, 64, 64, 0, NUL, 0, NUL) == SHAPE   # M > 16
    assert g(p(A), p(A), p(A), p(A), 1, 64, 48, 0, NUL, 0, NUL) == SHAPE    # K % 32
    assert g(p(A), p(A), p(A), p(A), 1, 64, (1 << 24) + 32, 0, NUL, 0, NUL) == SHAPE
    assert g(p(A), p(A), p(A), p(A), 1, -1, 64, 0, NUL, 0, NUL) == INVALID
    assert g(p(A), p(A), p(A), p(A), 1, 64, 64, -1, NUL, 0, NUL) == INVALID  # split_k < 0
    assert g(p(A), p(A), p(A), p(A), 1, 64, 64, 65, NUL, 0, NUL) == INVALID  # split_k > 64
    assert g(p(A), p(A), p(A), p(A), 1, 0, 64, 0, NUL, 0, NUL) == OK        # N == 0: no-op
    assert g(p(A), p(A), p(A), NUL, 1, 64, 64, 0, NUL, 0, NUL) == INVALID   # y null
    assert g(NUL, p(A), p(A), p(A), 1, 64, 64, 0, NUL, 0, NUL) == INVALID
    assert g(p(U), p(A), p(A), p(A), 1, 64, 64, 0, NUL, 0, NUL) == ALIGN
    assert g(p(A), p(U), p(A), p(A), 1, 64, 64, 0, NUL, 0, NUL) == ALIGN
    assert g(p(A), p(A), p(A), p(A + 2), 1, 64, 64, 0, NUL, 0, NUL) == ALIGN
    # a shape that needs split-K partials rejects a missing or short workspace
    ws = L.q4_gemv_skinny_ws_bytes(4, 5120, 17408, 0)
    assert ws > 0
    assert g(p(A), p(A), p(A), p(A), 4, 5120, 17408, 0, NUL, 0, NUL) == WS
    assert g(p(A), p(A), p(A), p(A), 4, 5120, 17408, 0, p(A), ws - 1, NUL) == WS
    assert g(p(A), p(A), p(A), p(A), 4, 5120, 17408, 0, p(A + 16), ws, NUL) == ALIGN


def test_gemv_noalloc_checks(L):
    """The allocation-free entry point makes the same checks as q4_gemv_skinny
    and rejects a plan larger than its static scratch, all before any HIP
    call."""
    g = L.q4_gemv_skinny_noalloc
    assert g(p(A), p(A), p(A), p(A), 0, 64, 64, 0, NUL) == SHAPE
    assert g(p(A), p(A), p(A), p(A), 17, 64, 64, 0, NUL) == SHAPE
    assert g(p(A), p(A), p(A), p(A), 1, 64, 48, 0, NUL) == SHAPE
    assert g(p(A), p(A), p(A), p(A), 1, 64, 64, 65, NUL) == INVALID
    assert g(p(A), p(A), p(A), p(A), 1, 0, 64, 0, NUL) == OK          # N == 0: no-op
    assert g(p(A), p(A), p(A), NUL, 1, 64, 64, 0, NUL) == INVALID
    assert g(p(U), p(A), p(A), p(A), 1, 64, 64, 0, NUL) == ALIGN
    assert g(p(A), p(A), p(A), p(A + 2), 1, 64, 64, 0, NUL) == ALIGN
    # the gate and up projections as one (N = 34816) at M = 16 need more
    # split-K scratch than the static array holds
    big = L.q4_gemv_skinny_ws_bytes(16, 34816, 5120, 0)
    assert big > binding.NOALLOC_SCRATCH_BYTES
    assert g(p(A), p(A), p(A), p(A), 16, 34816, 5120, 0, NUL) == WS
    for m in range(1, 17):
        for k, n in ((5120, 7168), (5120, 5120), (5120, 17408), (17408, 5120)):
            assert L.q4_gemv_skinny_ws_bytes(m, n, k, 0) <= binding.NOALLOC_SCRATCH_BYTES, (m, k, n)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define Q4W_NOALLOC_SCRATCH_BYTES \((.*)\)", text)
    assert m and eval(m.group(1).replace("u", "")) == binding.NOALLOC_SCRATCH_BYTES


def test_gemv_ws_sizes(L):
    f = L.q4_gemv_skinny_ws_bytes
    assert f(0, 64, 64, 0) == 0 and f(17, 64, 64, 0) == 0 and f(1, 64, 48, 0) == 0
    assert f(16, 5120, 17408, 0) > 0               # verify widths up to 16
    assert f(1, 512, 256, 1) == 0                  # one slice: no partials
    # explicit split: S slices x M x N fp32 partials plus the counter region
    s = f(2, 1000, 1024, 4)
    assert s >= 4 * 2 * 1000 * 4
    assert s % 256 == 0 or s > 0


def test_gemv_split_policy(L):
    """The library's split choice, read through the workspace size (the 256 KiB
    counter region plus S x M x N fp32 partials, none when S = 1)."""
    f = L.q4_gemv_skinny_ws_bytes
    region = 256 * 1024

    def slices(m, n, k):
        b = f(m, n, k, 0)
        if b == 0:
            return 1
        assert (b - region) % (m * n * 4) == 0, (m, n, k, b)
        return (b - region) // (m * n * 4)

    # VALU kernel (M <= 3): one slice when a row fits the largest slice
    # (12 steps of 32 blocks at M = 1, 11 at M = 2 (LDS), 5 at M = 3); the
    # 4x4x4 kernel (M = 4): 10 steps of 16 blocks, else slices of 4 at most ...
    assert slices(1, 17408, 5120) == 1        # decode gate/up
    assert slices(1, 7168, 5120) == 1         # qkv
    assert slices(1, 5120, 5120) == 1         # out
    assert slices(2, 17408, 5120) == 1
    assert slices(1, 4100, 12256) == 1        # 12 steps
    assert slices(2, 4100, 11232) == 1        # 11 steps
    assert slices(2, 4100, 12256) == 3        # 12 steps: slices of 4
    assert slices(3, 4100, 5088) == 1         # 5 steps
    assert slices(3, 4100, 6112) == 3         # 191 blocks: past one slice, M = 3 takes the 4x4x4 kernel
    # ... else slices of 6 steps at M = 1, 4 above (within the ring: no refill)
    assert slices(1, 5120, 17408) == 3        # verify down: 17 steps of 32 blocks
    assert slices(2, 5120, 17408) == 5
    assert slices(3, 5120, 17408) == 9        # the 4x4x4 kernel, as at M = 4
    assert slices(4, 5120, 17408) == 9        # 34 steps of 16 blocks: slices of 4
    assert slices(4, 4100, 11232) == 6        # 22 steps
    assert slices(4, 4100, 5120) == 1         # 10 steps: one slice
    # forced slice counts are raised until a slice fits the deepest copy:
    # 10 steps with one A operand, 6 with two (M = 5..7)
    assert f(4, 1000, 17376, 2) == region + 4 * 4 * 1000 * 4
    assert f(6, 1000, 17376, 2) == region + 6 * 6 * 1000 * 4
    # ... and more slices only below 256 workgroups (16 rows each)
    assert slices(1, 512, 8192) == 8          # 32 row tiles, 8 steps
    # the 4x4x4 kernel at M = 5..7 (two A operands): slices of at most 4
    # steps on 32-row tiles, from 5 steps on
    for m in (5, 6, 7):
        assert slices(m, 5120, 17408) == 9, m
        assert slices(m, 5120, 5120) == 3, m   # 10 steps: 4 + 4 + 2
        assert slices(m, 4100, 2048) == 1, m   # 4 steps: one slice
    assert slices(5, 512, 5120) == 10          # 16 row tiles: one-step slices toward 256 workgroups
    # 16x16x32 kernel (M >= 8): slices of at most 8 steps of 4 blocks, at
    # every width up to 16 (two activation staging items per thread past M = 8)
    for m in (8, 9, 13, 16):
        assert slices(m, 5120, 17408) == 17, m
    # ... and no more than that at or above 256 workgroups (64 rows each)
    assert slices(8, 5120, 5120) == 5          # 80 row tiles x 5 = 400 workgroups
    assert slices(8, 7168, 5120) == 5
    assert slices(8, 17408, 5120) == 5
    assert slices(8, 512, 5120) == 20          # 8 row tiles: 32 wanted, 2-step slices give 20


def test_act_quant_checks(L):
    q = L.a8_quantize_act
    assert q(p(A), -1, 64, p(A), p(A), NUL) == INVALID
    assert q(p(A), 4, 96, p(A), p(A), NUL) == SHAPE
    assert q(p(A), 0, 64, p(A), p(A), NUL) == OK
    assert q(NUL, 4, 64, p(A), p(A), NUL) == INVALID
    assert q(p(U), 4, 64, p(A), p(A), NUL) == ALIGN
    assert q(p(A), 4, 64, p(A), p(A + 2), NUL) == ALIGN


def test_a8_workspace_sizes(L):
    """A8 workspace: quantized activations of M rounded up to 128 rows
    (int8 [Mp, K], then fp32 scales [Mp, K/64], each 256-byte aligned), plus,
    from 256 padded rows on, the GEMM's region for shared tiles: 512 arrival
    counters (2 KiB) and two fp32 128 x 128 partial tiles per workgroup."""
    f = L.a8w4_ws_bytes

    def act(mp, k):
        def a256(v):
            return (v + 255) // 256 * 256
        return a256(mp * k) + a256(mp * (k // 64) * 4)

    region = 2048 + 2 * 512 * 128 * 128 * 4
    assert f(1, 64) == act(128, 64)
    assert f(128, 5120) == act(128, 5120)
    assert f(129, 5120) == act(256, 5120) + region
    assert f(2048, 17408) == act(2048, 17408) + region


def test_a8_checks(L):
    gm = L.a8w4_gemm_prefill
    ws = L.a8w4_ws_bytes(64, 128)
    assert ws >= 128 * 128
    assert gm(p(A), p(A), p(A), p(A), 64, 32, 96, p(A), ws, NUL) == SHAPE      # K % 64
    assert gm(p(A), p(A), p(A), p(A), -1, 32, 128, p(A), ws, NUL) == INVALID
    assert gm(p(A), p(A), p(A), p(A), 0, 32, 128, p(A), ws, NUL) == OK          # M == 0
    assert gm(p(A), p(A), p(A), p(A), 64, 0, 128, p(A), ws, NUL) == OK          # N == 0
    assert gm(p(A), p(A), p(A), NUL, 64, 32, 128, p(A), ws, NUL) == INVALID
    assert gm(p(A), p(A), NUL, p(A), 64, 32, 128, p(A), ws, NUL) == INVALID
    assert gm(p(A), p(A), p(A), p(A), 64, 32, 128, NUL, 0, NUL) == WS
    assert gm(p(A), p(A), p(A), p(A), 64, 32, 128, p(A), ws - 1, NUL) == WS
    assert gm(p(A), p(A), p(A), p(A), 64, 32, 128, p(A + 16), ws, NUL) == ALIGN
    assert gm(p(U), p(A), p(A), p(A), 64, 32, 128, p(A), ws, NUL) == ALIGN
    pr = L.a8w4_prepare_act
    assert pr(p(A), 64, 96, p(A), ws, NUL) == SHAPE
    assert pr(p(A), 0, 128, p(A), ws, NUL) == OK
    assert pr(NUL, 64, 128, p(A), ws, NUL) == INVALID
    assert pr(p(A), 64, 128, p(A), ws - 1, NUL) == WS
    assert pr(p(U), 64, 128, p(A), ws, NUL) == ALIGN
    gp = L.a8w4_gemm_prepared
    assert gp(p(A), p(A), p(A), p(A), 64, 32, 96, ws, NUL) == SHAPE
    assert gp(p(A), p(A), p(A), p(A), 64, 32, 128, ws - 1, NUL) == WS
    assert gp(NUL, p(A), p(A), p(A), 64, 32, 128, ws, NUL) == INVALID
    assert gp(p(A), p(A), NUL, p(A), 64, 32, 128, ws, NUL) == INVALID
    dbg = L.a8w4_debug_block_acc
    assert dbg(p(A), p(A), p(A), 64, 32, 96, p(A), ws, NUL) == SHAPE
    # K = 2^24 would take the 128-row tile's 32-bit buffer range to 2^31: refused
    # by every A8 entry point; 2^24 - 64 passes the shape rules (and then needs
    # its workspace)
    big = 1 << 24
    assert gm(p(A), p(A), p(A), p(A), 64, 32, big, p(A), ws, NUL) == SHAPE
    assert pr(p(A), 64, big, p(A), ws, NUL) == SHAPE
    assert gp(p(A), p(A), p(A), p(A), 64, 32, big, ws, NUL) == SHAPE
    assert dbg(p(A), p(A), p(A), 64, 32, big, p(A), ws, NUL) == SHAPE
    assert gm(p(A), p(A), p(A), p(A), 64, 32, big - 64, p(A), ws, NUL) == WS
    assert pr(p(A), 64, big - 64, p(A), ws, NUL) == WS
    assert dbg(p(A), p(A), p(A), 64, 32, 128, NUL, 0, NUL) == WS
    assert dbg(p(A), NUL, p(A), 64, 32, 128, p(A), ws, NUL) == INVALID


def test_binding_loads_lazily_and_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises instead of falling back."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def _descs(entries):
    arr = (binding.GemvDesc * len(entries))()
    for d, (x, c, s, y, n, k) in zip(arr, entries):
        d.x, d.codes, d.scales, d.y, d.N, d.K = x, c, s, y, n, k
    return arr


def test_batched_checks(L):
    """Every argument check of the batched entry points returns before any HIP
    call (a valid batch would upload its table, so none is planned here)."""
    good = (A, A, A, A, 5120, 17408)
    ws_bytes = L.q4_gemv_batched_ws_bytes
    plan = binding.BatchedPlan()
    pl = ctypes.byref(plan)
    one = _descs([good])
    assert ws_bytes(5, one, 1) > 0
    assert ws_bytes(5, one, 0) == 0 and ws_bytes(0, one, 1) == 0 and ws_bytes(17, one, 1) == 0
    assert ws_bytes(16, one, 1) > 0
    assert ws_bytes(5, None, 1) == 0
    assert ws_bytes(5, _descs([(A, A, A, A, 64, 48)]), 1) == 0       # K % 32
    assert ws_bytes(5, _descs([(A, A, A, A, 0, 64)]), 1) == 0        # N == 0
    # two matmuls need at least the sum of their split-K workspaces
    two = _descs([good, (A, A, A, A, 7168, 5120)])
    assert ws_bytes(5, two, 2) >= ws_bytes(5, one, 1)
    bp = L.q4_gemv_batched_plan
    need = ws_bytes(5, one, 1)
    assert bp(5, one, 1, p(A), need, None) == INVALID                # no plan struct
    assert bp(5, None, 1, p(A), need, pl) == INVALID
    assert bp(5, one, 0, p(A), need, pl) == INVALID
    assert bp(0, one, 1, p(A), need, pl) == SHAPE
    assert bp(17, one, 1, p(A), need, pl) == SHAPE
    assert bp(5, _descs([(A, A, A, A, -1, 64)]), 1, p(A), need, pl) == INVALID
    assert bp(5, _descs([(A, A, A, A, 64, 0)]), 1, p(A), need, pl) == INVALID
    assert bp(5, _descs([(A, A, A, A, 64, 96 + 16)]), 1, p(A), need, pl) == SHAPE
    assert bp(5, _descs([(A, A, A, A, 1 << 20, 64)]), 1, p(A), need, pl) == SHAPE   # N > 2^19
    assert bp(5, _descs([(0, A, A, A, 64, 64)]), 1, p(A), need, pl) == INVALID     # null x
    assert bp(5, _descs([(U, A, A, A, 64, 64)]), 1, p(A), need, pl) == ALIGN       # x not 16-aligned
    assert bp(5, _descs([(A, U, A, A, 64, 64)]), 1, p(A), need, pl) == ALIGN
    assert bp(5, _descs([(A, A, A + 1, A, 64, 64)]), 1, p(A), need, pl) == ALIGN
    assert bp(5, _descs([(A, A, A, U, 64, 64)]), 1, p(A), need, pl) == ALIGN       # y not 4-aligned
    assert bp(5, one, 1, None, need, pl) == WS
    assert bp(5, one, 1, p(A), need - 1, pl) == WS
    assert bp(5, one, 1, p(A + 16), need, pl) == ALIGN
    run = L.q4_gemv_batched_run
    assert run(None, NUL) == INVALID
    assert run(ctypes.byref(binding.BatchedPlan()), NUL) == INVALID  # never planned


def test_attn_checks(L):
    """q4_attn_decode: shape, pointer, alignment and workspace checks, and the
    workspace size (S key slices x H_kv x R rows of D fp32 partials, then the
    per-row max and sum)."""
    ws = L.q4_attn_decode_ws_bytes
    # T = 262144, M = 5, 20 query heads over 4 K/V heads: 64 slices x 4 x 25 rows
    assert ws(5, 20, 4, 256, 262144) == 64 * 4 * 25 * 256 * 4 + 64 * 4 * 25 * 2 * 4
    # T = 100: 4 tiles of 32 keys -> one slice
    assert ws(1, 20, 4, 256, 100) == 4 * 5 * 256 * 4 + 4 * 5 * 2 * 4
    assert ws(0, 20, 4, 256, 100) == 0 and ws(1, 20, 4, 128, 100) == 0 and ws(1, 20, 3, 256, 100) == 0
    assert ws(5, 40, 4, 256, 100) == 0           # R = 50 > 32
    assert ws(5, 20, 4, 256, 4) == 0             # T < M
    assert ws(1, 4, 4, 256, (1 << 22) - 1) > 0 and ws(1, 4, 4, 256, 1 << 22) == 0   # 32-bit cache offsets
    need = ws(5, 20, 4, 256, 1000)
    f = L.q4_attn_decode
    args = lambda **kw: [p(kw.get("q", A)), p(kw.get("kc", A)), p(kw.get("ks", A)), p(kw.get("vc", A)),
                         p(kw.get("vs", A)), p(kw.get("o", A)), kw.get("m", 5), kw.get("hq", 20), 4, 256,
                         kw.get("t", 1000), p(kw.get("ws", A)), kw.get("wsb", need), NUL]
    assert f(*args(m=0)) == INVALID
    assert f(*args(t=-1)) == INVALID
    assert f(*args(hq=21)) == SHAPE
    assert f(*args(t=4)) == SHAPE
    assert f(*args(q=0)) == INVALID and f(*args(vs=0)) == INVALID and f(*args(o=0)) == INVALID
    assert f(*args(q=U)) == ALIGN and f(*args(kc=A + 8)) == ALIGN and f(*args(vc=A + 8)) == ALIGN
    assert f(*args(ks=A + 4)) == ALIGN and f(*args(vs=A + 4)) == ALIGN and f(*args(o=A + 1)) == ALIGN
    assert f(*args(ws=0)) == WS and f(*args(wsb=need - 1)) == WS
    assert f(*args(ws=A + 16)) == ALIGN


def test_stream_read_checks(L):
    f = L.q4w_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(p(A), 1024, NUL, 256, 512, NUL) == INVALID
    assert f(NUL, 1024, p(A), 256, 512, NUL) == INVALID
    assert f(p(A), 1024, p(A), 0, 512, NUL) == INVALID and f(p(A), 1024, p(A), 65537, 512, NUL) == INVALID
    assert f(p(A), 1024, p(A), 256, 32, NUL) == INVALID and f(p(A), 1024, p(A), 256, 96 + 16, NUL) == INVALID
    assert f(p(A), 1024, p(A), 256, 2048, NUL) == INVALID
    assert f(p(A), 1000, p(A), 256, 512, NUL) == SHAPE
    assert f(p(A + 8), 1024, p(A), 256, 512, NUL) == ALIGN and f(p(A), 1024, p(A + 2), 256, 512, NUL) == ALIGN
