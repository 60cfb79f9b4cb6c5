"""The C ABI library on the host: it loads, exports every symbol the headers under
include/ declare, and rejects bad arguments before anything reaches a GPU (no compute
calls here)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_46_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

FAKE = 1 << 40          # a 16-byte aligned address that is never dereferenced
MIS = FAKE + 8          # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe.so is not built: run python -m mixture_experts_layer_46_amd.build")
    return _lib.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_shape_struct_layout_matches_header():
    # int64 T; int32 H, E, k, F, dtype, ffn; uint32 flags; int32 capacity -> 40 bytes
    assert ctypes.sizeof(_lib.MoeShape) == 40
    assert _lib.MoeShape.capacity.offset == 36


def _shape(**kw):
    d = dict(T=16, H=64, E=8, k=2, F=128, dtype=_lib.MOE_BF16, ffn=_lib.MOE_FFN_SWIGLU, flags=0, capacity=0)
    d.update(kw)
    return _lib.MoeShape(**d)


def _ws(lib, s):
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), 2), (dict(H=0), 2), (dict(E=0), 2), (dict(k=0), 2), (dict(F=-8), 2),
    (dict(k=9, E=8), 2), (dict(E=257, k=2), 3), (dict(E=64, k=9), 3), (dict(H=60), 3),
    (dict(F=100), 3), (dict(dtype=7), 3), (dict(ffn=5), 3), (dict(flags=0x10), 3),
    (dict(capacity=-1), 2), (dict(T=1 << 31, k=1), 2), (dict(T=1 << 30, k=2), 2),
    # 32-bit byte offsets of the grouped GEMM with the out-of-range marker at 2^31: an
    # expert matrix (plus 128 rows) or x of 2 GiB or more
    (dict(H=65536, F=32768), 3), (dict(H=8, F=1 << 24), 3), (dict(T=300000, H=8192), 3),
    (dict(H=16384, F=65536), 3), (dict(T=131072, H=8192), 3),
    (dict(H=8, F=(1 << 30) // 136 // 8 * 8 + 8), 3),
    # the bf16 gate's weight planes (3 x E x H rounded up to 32, bf16) of 2 GiB or more
    (dict(T=300, H=1398088, E=256), 3),
])
def test_bad_shapes_are_rejected(lib, kw, code):
    s = _shape(**kw)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == code
    assert lib.moe_last_error().decode() != ""
    rc = lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == code


def test_null_and_alignment_checks(lib):
    s = _shape()
    ws = _ws(lib, s)
    ok = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws]
    names = ["x", "w_gate", "bias", "w_in", "w_up", "w_out", "out", "workspace"]

    def fwd(args):
        return lib.moe_forward(ctypes.byref(s), *args, None)

    for i, name in enumerate(names):
        if name == "bias":
            a = list(ok)
            a[i] = MIS
            assert fwd(a) == 4 and "bias" in lib.moe_last_error().decode()
            continue
        a = list(ok)
        a[i] = None
        want = 5 if name == "workspace" else 1
        assert fwd(a) == want, name
        assert name in lib.moe_last_error().decode()
        a[i] = MIS
        assert fwd(a) == 4, name
    # workspace too small
    a = list(ok)
    a[-1] = ws - 1
    assert fwd(a) == 5
    assert "need" in lib.moe_last_error().decode()
    # w_up must be NULL for the SiLU two-layer FFN
    s2 = _shape(ffn=_lib.MOE_FFN_SILU2)
    assert lib.moe_forward(ctypes.byref(s2), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 2


def test_zero_tokens_is_a_no_op(lib):
    s = _shape(T=0)
    ws = _ws(lib, s)
    assert lib.moe_forward(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 0
    assert lib.moe_route(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == 0
    assert lib.moe_combine(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None) == 0
    assert lib.moe_permute(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == 0


def test_stage_argument_checks(lib):
    s = _shape()
    ws = _ws(lib, s)
    # route from logits: logits required; w_gate may be NULL
    assert lib.moe_route(ctypes.byref(s), None, None, None, None, FAKE, FAKE, None) == 1
    # permute: x and x_perm together
    assert lib.moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == 1
    assert lib.moe_permute(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16, None) == 5
    # grouped ffn: SwiGLU needs w_up
    assert lib.moe_grouped_ffn(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == 1
    # stats: capacity needs offsets
    s3 = _shape(capacity=4)
    assert lib.moe_router_stats(ctypes.byref(s3), FAKE, None, FAKE, None, FAKE, None) == 1


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.moe_status_str(code).decode().startswith(name)


def test_workspace_grows_with_the_layer(lib):
    a = _ws(lib, _shape())                              # 4 rows per expert: 16-row tiles
    b = _ws(lib, _shape(T=1024))                        # 256 rows per expert: large tiles
    c = _ws(lib, _shape(T=1024, dtype=_lib.MOE_F32))
    d = _ws(lib, _shape(dtype=_lib.MOE_F32))
    assert 0 < a < b and 0 < d < c
    # the large-tile bf16 GEMM carries the split buffers of its last round: 256 slots of
    # up to 256 x 256 fp32 accumulators (the 16-row tiles and fp32 layers have none)
    assert b - a > 256 * 256 * 256 * 4
    assert c - d < 256 * 256 * 256 * 4


def test_largest_accepted_shapes(lib):
    # just below the 2 GiB limits: (H + 128) * F * 2 bytes and T * H * 2 bytes
    ok = _shape(H=8, F=(1 << 30) // 136 // 8 * 8)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(ok), ctypes.byref(n)) == 0
    ok2 = _shape(T=(1 << 30) // 8192 - 1, H=8192)
    assert lib.moe_workspace_size(ctypes.byref(ok2), ctypes.byref(n)) == 0
    # the gate's weight planes just below 2 GiB (3 * 256 * 1398080 * 2 bytes), and above it
    # for fp32 x, whose gate reads W_g directly
    ok3 = _shape(T=300, H=1398080, E=256)
    assert lib.moe_workspace_size(ctypes.byref(ok3), ctypes.byref(n)) == 0
    ok4 = _shape(T=300, H=1398088, E=256, dtype=_lib.MOE_F32)
    assert lib.moe_workspace_size(ctypes.byref(ok4), ctypes.byref(n)) == 0


def test_capacity_rows(lib):
    # the library's C = max(1, ceil(cf * T * k / E)) ([Principles §4.3], pairs as the total)
    assert _lib.capacity_rows(None, 8192, 2, 64) == 0
    assert _lib.capacity_rows(1.0, 8192, 2, 64) == 256
    assert _lib.capacity_rows(1.25, 8192, 2, 64) == 320
    assert _lib.capacity_rows(0.75, 30, 2, 4) == 12            # ceil(11.25)
    assert _lib.capacity_rows(1e-9, 1, 1, 256) == 1
    rows = ctypes.c_int32(-5)
    assert lib.moe_capacity_rows(0.0, 8, 2, 4, ctypes.byref(rows)) == 2
    assert lib.moe_capacity_rows(float("nan"), 8, 2, 4, ctypes.byref(rows)) == 2
    assert lib.moe_capacity_rows(1.0, 8, 0, 4, ctypes.byref(rows)) == 2
    assert lib.moe_capacity_rows(1.0, 8, 2, 4, None) == 1
    assert lib.moe_capacity_rows(1.0, 8, 2, 4, ctypes.byref(rows)) == 0 and rows.value == 4


def test_workspace_layout(lib):
    for kw in (dict(), dict(T=1024), dict(T=1024, dtype=_lib.MOE_F32), dict(T=0)):
        s = _shape(**kw)
        lay = _lib.workspace_layout(_lib.Shape(**{f: getattr(s, f) for f, _ in _lib.MoeShape._fields_}))
        assert lay["total"] == _ws(lib, s)
        P, E = s.T * s.k, s.E
        es = 4 if s.dtype == _lib.MOE_F32 else 2
        spans = [("logit_parts", lay["logit_splits"] * s.T * E * 4), ("topk_idx", P * 4), ("topk_w", P * 4),
                 ("counts", E * 4), ("offsets", (E + 1) * 4), ("sorted_token", P * 4),
                 ("row_of_pair", P * 4), ("h", P * s.F * es), ("y", P * s.H * es)]
        assert lay["logit_splits"] >= 1
        ends = sorted((lay[n], lay[n] + b, n) for n, b in spans)
        for (a0, a1, na), (b0, b1, nb) in zip(ends, ends[1:]):
            assert a1 <= b0, (na, nb)                       # no overlap
        assert all(lay[n] % 256 == 0 for n, _ in spans)
        assert ends[-1][1] <= lay["total"]
    assert lib.moe_workspace_layout(ctypes.byref(_shape()), None) == 1
    assert lib.moe_workspace_layout(ctypes.byref(_shape(E=0)), ctypes.byref(_lib.MoeWorkspaceParts())) == 2


def test_forward_timed_argument_checks(lib):
    s = _shape()
    ws = _ws(lib, s)
    args = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws]
    bad = (ctypes.c_void_p * 6)(*([FAKE] * 5 + [None]))
    assert lib.moe_forward_timed(ctypes.byref(s), *args, bad, None) == 1          # NULL entry
    assert b"events[5]" in lib.moe_last_error()
    s0 = _shape(T=0)
    arr = (ctypes.c_void_p * 6)(*([FAKE] * 6))
    assert lib.moe_forward_timed(ctypes.byref(s0), *args[:-1], _ws(lib, s0), arr, None) == 0
    assert lib.moe_forward_timed(ctypes.byref(s0), *args[:-1], _ws(lib, s0), None, None) == 0


def test_peak_entry_points_argument_checks(lib):
    khz = ctypes.c_int(0)
    assert lib.moe_peak_mfma_bf16(256, 10, None, FAKE, ctypes.byref(khz), None) == 1
    assert lib.moe_peak_mfma_bf16(0, 10, FAKE, FAKE, None, None) == 2
    assert lib.moe_peak_mfma_bf16(256, 0, FAKE, FAKE, None, None) == 2
    assert lib.moe_peak_mfma_bf16(256, 10, MIS, FAKE, None, None) == 4
    assert lib.moe_peak_hbm_read(None, 1 << 20, 256, FAKE, None) == 1
    assert lib.moe_peak_hbm_read(FAKE, (1 << 20) + 4, 256, FAKE, None) == 2
    assert lib.moe_peak_hbm_read(FAKE, 0, 256, FAKE, None) == 2
    assert lib.moe_peak_hbm_read(FAKE, 1 << 20, 70000, FAKE, None) == 2
    assert lib.moe_peak_hbm_read(MIS, 1 << 20, 256, FAKE, None) == 4
    assert lib.moe_peak_hbm_copy(FAKE, None, 1 << 20, 256, None) == 1
    assert lib.moe_peak_hbm_copy(FAKE, FAKE + (1 << 19), 1 << 20, 256, None) == 2   # overlap
    assert b"overlap" in lib.moe_last_error()


def test_forward_noalloc_argument_checks(lib):
    # refused on the host before any device work: too large for the static scratch,
    # NULL or misaligned pointers, a bad shape; T == 0 is a no-op
    big = _shape(T=8192, H=4096, E=64, k=2, F=16384, ffn=_lib.MOE_FFN_SILU2)
    assert lib.moe_forward_noalloc(ctypes.byref(big), FAKE, FAKE, None, FAKE, None, FAKE, FAKE, None) == 5
    assert b"static scratch" in lib.moe_last_error()
    s = _shape()
    assert _ws(lib, s) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(s), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.moe_forward_noalloc(ctypes.byref(s), FAKE, FAKE, MIS, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert lib.moe_forward_noalloc(ctypes.byref(_shape(E=0)), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert lib.moe_forward_noalloc(ctypes.byref(_shape(T=0)), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == 0
