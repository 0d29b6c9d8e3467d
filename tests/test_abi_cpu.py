"""CPU tests of the C ABI: the library loads, exports every entry point that
include/gla.h declares, and its host-side validation rejects bad arguments with the
documented status before touching the GPU (every case here is invalid, so no HIP
call and no kernel launch happens)."""
import ctypes
import os
import re

import pytest

from causal_gated_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")
TEST_HEADER = os.path.join(ROOT, "include", "gla_testing.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from causal_gated_linear_amd import build
        build.build()
    return _lib.load()


def _declared(*headers):
    text = "".join(open(h).read() for h in (headers or (HEADER,)))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(["gla_state_alloc", "gla_state_free", "gla_prefill_workspace_bytes",
                                  "gla_prefill_chunked", "gla_decode_step", "gla_strerror",
                                  "gla_last_error_detail", "gla_prefill_chunked_norm",
                                  "gla_decode_step_norm", "gla_delta_workspace_bytes",
                                  "gla_prefill_delta", "gla_decode_step_delta", "gla_gate_project",
                                  "gla_prefill_outer", "gla_decode_step_outer",
                                  "gla_prefill_chunked_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(_lib.LIB_PATH)
    both = _declared(HEADER, TEST_HEADER)
    assert _declared(TEST_HEADER) == ["gla_testing_set_plan"]
    for name in both:
        assert hasattr(raw, name), name
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == both


def test_testing_plan_hook(lib):
    """gla_testing_set_plan validates its values, and the workspace query follows the
    forced segment count (then returns to the automatic plan)."""
    for bad in [(8, 0, 0), (0, -1, 0), (0, 0, 128), (48, 0, 0)]:
        assert lib.gla_testing_set_plan(*bad) == _lib.GLA_ERR_UNSUPPORTED
    args = (1, 2, 64 * 20, 128, 128, 64, _lib.GLA_BF16)
    assert lib.gla_prefill_workspace_bytes(*args) == 0          # 2 heads of 20 chunks: one segment
    try:
        assert lib.gla_testing_set_plan(0, 3, 0) == _lib.GLA_OK
        assert lib.gla_prefill_workspace_bytes(*args) > 0
    finally:
        assert lib.gla_testing_set_plan(0, 0, 0) == _lib.GLA_OK
    assert lib.gla_prefill_workspace_bytes(*args) == 0


def test_strerror_covers_every_status(lib):
    for st in range(0, -9, -1):
        s = lib.gla_strerror(st).decode()
        assert s and s != "unknown status"
    assert lib.gla_strerror(-99).decode() == "unknown status"


# fake, 16-byte aligned device addresses: validation must reject every call below
# before any of them is dereferenced or passed to HIP
A = 0x10000000
MB = 1 << 20


def _prefill(lib, **kw):
    args = dict(q=A, k=A + 16 * MB, v=A + 32 * MB, g=A + 48 * MB, gate=1, s0=None, o=A + 96 * MB,
                s_final=A + 128 * MB, B=1, H=2, L=64, d_k=64, d_v=64, chunk=64, dtype=1, phi=0,
                ws=None, ws_bytes=0)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_prefill_chunked(P(args["q"]), P(args["k"]), P(args["v"]), P(args["g"]), args["gate"],
                                   P(args["s0"]), P(args["o"]), P(args["s_final"]), args["B"],
                                   args["H"], args["L"], args["d_k"], args["d_v"], args["chunk"],
                                   args["dtype"], args["phi"], P(args["ws"]), args["ws_bytes"], None)


PREFILL_BAD = {
    "B_zero": (dict(B=0), _lib.GLA_ERR_SHAPE),
    "H_negative": (dict(H=-3), _lib.GLA_ERR_SHAPE),
    "L_negative": (dict(L=-1), _lib.GLA_ERR_SHAPE),
    "d_k_48": (dict(d_k=48), _lib.GLA_ERR_UNSUPPORTED),
    "d_v_256": (dict(d_v=256), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_128_at_d_k_128": (dict(chunk=128, d_k=128), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_256": (dict(chunk=256), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_8": (dict(chunk=8), _lib.GLA_ERR_UNSUPPORTED),
    "L_past_32bit_head_offsets": (dict(L=4194304, d_k=128, d_v=128), _lib.GLA_ERR_SHAPE),
    "segmented_without_workspace": (dict(B=1, H=2, L=64 * 65), _lib.GLA_ERR_WORKSPACE),
    "segmented_short_workspace": (dict(B=1, H=2, L=64 * 65, ws=A + 400 * MB, ws_bytes=4096), _lib.GLA_ERR_WORKSPACE),
    "dtype_7": (dict(dtype=7), _lib.GLA_ERR_UNSUPPORTED),
    "gate_5": (dict(gate=5), _lib.GLA_ERR_UNSUPPORTED),
    "phi_3": (dict(phi=3), _lib.GLA_ERR_UNSUPPORTED),
    "gate_none_with_g": (dict(gate=0), _lib.GLA_ERR_UNSUPPORTED),
    "keydim_without_g": (dict(g=None), _lib.GLA_ERR_NULL),
    "q_null": (dict(q=None), _lib.GLA_ERR_NULL),
    "o_null": (dict(o=None), _lib.GLA_ERR_NULL),
    "q_misaligned": (dict(q=A + 8), _lib.GLA_ERR_ALIGN),
    "s_final_misaligned": (dict(s_final=A + 128 * MB + 4), _lib.GLA_ERR_ALIGN),
    "keydim_g_misaligned": (dict(g=A + 48 * MB + 4), _lib.GLA_ERR_ALIGN),
    "scalar_g_misaligned": (dict(gate=2, g=A + 48 * MB + 2), _lib.GLA_ERR_ALIGN),
    "o_overlaps_v": (dict(o=A + 32 * MB + 4096), _lib.GLA_ERR_ALIAS),
    "o_overlaps_g": (dict(o=A + 48 * MB), _lib.GLA_ERR_ALIAS),
    "o_overlaps_s_final": (dict(s_final=A + 96 * MB + 64), _lib.GLA_ERR_ALIAS),
    "s_final_overlaps_q": (dict(s_final=A + 1024), _lib.GLA_ERR_ALIAS),
    "s_final_partially_overlaps_s0": (dict(s0=A + 200 * MB, s_final=A + 200 * MB + 256), _lib.GLA_ERR_ALIAS),
    # a segmented plan (workspace in use) whose workspace overlaps an input
    "workspace_overlaps_s0": (dict(L=64 * 65, s0=A + 400 * MB + 4096, ws=A + 400 * MB, ws_bytes=64 * MB),
                              _lib.GLA_ERR_ALIAS),
    "workspace_overlaps_k": (dict(L=64 * 65, ws=A + 16 * MB + 4096, ws_bytes=64 * MB), _lib.GLA_ERR_ALIAS),
}


@pytest.mark.parametrize("case", sorted(PREFILL_BAD))
def test_prefill_rejects(lib, case):
    kw, want = PREFILL_BAD[case]
    assert _prefill(lib, **kw) == want
    assert lib.gla_last_error_detail().decode() != ""


def _decode(lib, **kw):
    args = dict(q=A, k=A + MB, v=A + 2 * MB, g=A + 3 * MB, gate=1, state=A + 16 * MB, o=A + 64 * MB,
                B=2, H=4, d_k=128, d_v=128, dtype=1, phi=0)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_decode_step(P(args["q"]), P(args["k"]), P(args["v"]), P(args["g"]), args["gate"],
                               P(args["state"]), P(args["o"]), args["B"], args["H"], args["d_k"],
                               args["d_v"], args["dtype"], args["phi"], None)


DECODE_BAD = {
    "state_null": (dict(state=None), _lib.GLA_ERR_NULL),
    "v_null": (dict(v=None), _lib.GLA_ERR_NULL),
    "B_zero": (dict(B=0), _lib.GLA_ERR_SHAPE),
    "d_v_8": (dict(d_v=8), _lib.GLA_ERR_UNSUPPORTED),
    "scalar_without_g": (dict(gate=2, g=None), _lib.GLA_ERR_NULL),
    "o_overlaps_state": (dict(o=A + 16 * MB + 512), _lib.GLA_ERR_ALIAS),
    "state_overlaps_k": (dict(state=A + MB), _lib.GLA_ERR_ALIAS),
    "o_misaligned": (dict(o=A + 64 * MB + 2), _lib.GLA_ERR_ALIGN),
    "scalar_g_misaligned": (dict(gate=2, g=A + 3 * MB + 1), _lib.GLA_ERR_ALIGN),
}


@pytest.mark.parametrize("case", sorted(DECODE_BAD))
def test_decode_rejects(lib, case):
    kw, want = DECODE_BAD[case]
    assert _decode(lib, **kw) == want


def test_empty_prefill_may_omit_inputs(lib):
    """With L == 0 the inputs (and g) may be NULL; the call is still validated (here it
    fails on the chunk size, so nothing is launched)."""
    assert _prefill(lib, L=0, q=None, k=None, v=None, o=None, g=None, chunk=8) == _lib.GLA_ERR_UNSUPPORTED
    assert _prefill(lib, L=1, g=None) == _lib.GLA_ERR_NULL


def test_chunk_128_accepted_for_small_key_dims(lib):
    """Chunks of 128 rows pass validation for d_k <= 64 (in the plain, allocation-free
    and normalised prefills) and fail only on the deliberately misaligned s_final;
    at d_k = 128 they are rejected."""
    for dk in (16, 32, 64):
        for dv in (16, 64, 128):
            assert _prefill(lib, chunk=128, d_k=dk, d_v=dv, s_final=A + 128 * MB + 4) == _lib.GLA_ERR_ALIGN
            assert _prefill_norm(lib, chunk=128, d_k=dk, d_v=dv, s_final=A + 128 * MB + 4) == _lib.GLA_ERR_ALIGN
    assert _prefill(lib, chunk=128, d_k=128, d_v=64) == _lib.GLA_ERR_UNSUPPORTED
    assert "128" in lib.gla_last_error_detail().decode()
    assert _prefill_norm(lib, chunk=128, d_k=128) == _lib.GLA_ERR_UNSUPPORTED
    # few long sequences at chunk 128 are segmented like any other chunk size
    assert lib.gla_prefill_workspace_bytes(1, 2, 128 * 70, 64, 64, 128, 1) > 0
    assert lib.gla_prefill_workspace_bytes(1, 2, 128 * 70, 128, 64, 128, 1) == 0


def test_state_alloc_rejects(lib):
    assert lib.gla_state_alloc(1, 1, 16, 16, None, None) == _lib.GLA_ERR_NULL
    p = ctypes.c_void_p(1234)
    assert lib.gla_state_alloc(0, 1, 16, 16, ctypes.byref(p), None) == _lib.GLA_ERR_SHAPE
    assert lib.gla_state_alloc(1, 1, 24, 16, ctypes.byref(p), None) == _lib.GLA_ERR_UNSUPPORTED
    assert p.value == 1234                      # untouched on error
    assert lib.gla_state_free(None, None) == _lib.GLA_OK


def test_workspace_for_few_long_sequences(lib):
    """Few long sequences are split into segments, which need a workspace: the fp32
    states from zero [B*H][pieces][d_k][d_v] of the pieces of all segments but the last,
    their gate totals [B*H][pieces][d_k], and room for a copy of s0 [B*H][d_k][d_v]
    (taken when the state is updated in place).  The state-only pass splits each such
    segment into equal pieces until up to three of its workgroups share a CU."""
    n = lib.gla_prefill_workspace_bytes(1, 32, 32768, 128, 128, 64, 1)
    rnd = lambda x: (x + 255) // 256 * 256
    # 4 segments of 8192 tokens; 32 heads x 2 value tiles x 3 segments = 192 workgroups
    # in the state-only pass, so 4 pieces per segment (768); then room for a copy of s0
    assert n == rnd(32 * 12 * 128 * 128 * 4) + rnd(32 * 12 * 128 * 4) + rnd(32 * 128 * 128 * 4)
    assert lib.gla_prefill_workspace_bytes(8, 16, 4096, 128, 128, 64, 1) == 0   # enough heads
    assert lib.gla_prefill_workspace_bytes(1, 2, 64 * 31, 64, 64, 64, 1) == 0   # too short
    # 32 to 63 chunks on too few heads for even the narrowest tile: short segments
    assert lib.gla_prefill_workspace_bytes(1, 2, 64 * 63, 64, 64, 64, 1) > 0
    assert lib.gla_prefill_workspace_bytes(4, 8, 2048, 64, 64, 64, 1) > 0
    assert lib.gla_prefill_workspace_bytes(8, 16, 2048, 64, 64, 64, 1) == 0   # enough heads


def test_workspace_query_is_host_only(lib):
    assert lib.gla_prefill_workspace_bytes(8, 16, 4096, 128, 128, 64, 1) >= 0
    assert lib.gla_prefill_workspace_bytes(-1, 16, 4096, 128, 128, 64, 1) == 0


def test_python_binding_checks_shapes():
    """The binding checks shapes and dtypes itself (the ABI cannot see buffer sizes)."""
    import torch
    from causal_gated_linear_amd import api
    q = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        api.prefill(q, q, q)                                   # host tensors
    q = torch.zeros(1, 1, 16, 16, device="meta")
    with pytest.raises(ValueError):
        api.prefill(q, q, torch.zeros(1, 1, 8, 16))            # L mismatch
    with pytest.raises(ValueError):
        api.prefill(q, q.to(torch.bfloat16), q)                # dtype mismatch
    with pytest.raises(ValueError):
        api.prefill(q, q, q, log_gate=torch.zeros(1, 1, 16), gate="keydim")   # gate shape
    with pytest.raises(ValueError):
        api.prefill(q.transpose(2, 3), q, q)                   # non-contiguous


# the normalised entry points share the validation above and add the z arguments
def _prefill_norm(lib, **kw):
    args = dict(q=A, k=A + 16 * MB, v=A + 32 * MB, g=A + 48 * MB, gate=1, s0=None, z0=None, o=A + 96 * MB,
                s_final=A + 128 * MB, z_final=A + 160 * MB, B=1, H=2, L=64, d_k=64, d_v=64, chunk=64,
                dtype=1, phi=0)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_prefill_chunked_norm(P(args["q"]), P(args["k"]), P(args["v"]), P(args["g"]), args["gate"],
                                        P(args["s0"]), P(args["z0"]), P(args["o"]), P(args["s_final"]),
                                        P(args["z_final"]), args["B"], args["H"], args["L"], args["d_k"],
                                        args["d_v"], args["chunk"], args["dtype"], args["phi"], None)


PREFILL_NORM_BAD = {
    "d_k_48": (dict(d_k=48), _lib.GLA_ERR_UNSUPPORTED),
    "z0_misaligned": (dict(z0=A + 200 * MB + 4), _lib.GLA_ERR_ALIGN),
    "z_final_misaligned": (dict(z_final=A + 160 * MB + 8), _lib.GLA_ERR_ALIGN),
    "o_overlaps_z_final": (dict(z_final=A + 96 * MB + 256), _lib.GLA_ERR_ALIAS),
    "z_final_overlaps_k": (dict(z_final=A + 16 * MB + 64), _lib.GLA_ERR_ALIAS),
    "z_final_partially_overlaps_z0": (dict(z0=A + 200 * MB, z_final=A + 200 * MB + 16), _lib.GLA_ERR_ALIAS),
    "z_final_equals_z0": (dict(z0=A + 200 * MB, z_final=A + 200 * MB), _lib.GLA_ERR_ALIAS),
    "s_final_overlaps_z0": (dict(z0=A + 128 * MB + 32), _lib.GLA_ERR_ALIAS),
}


@pytest.mark.parametrize("case", sorted(PREFILL_NORM_BAD))
def test_prefill_norm_rejects(lib, case):
    kw, want = PREFILL_NORM_BAD[case]
    assert _prefill_norm(lib, **kw) == want
    assert lib.gla_last_error_detail().decode() != ""


def test_prefill_norm_needs_no_workspace_even_when_segmentable(lib):
    """Sizes that the plain prefill would split into segments (and so need a
    workspace) run unsegmented in the normalised form; validation must pass that
    point and fail only on the deliberately bad alignment below."""
    assert lib.gla_prefill_workspace_bytes(1, 2, 64 * 65, 64, 64, 64, 1) > 0
    assert _prefill_norm(lib, L=64 * 65, o=A + 96 * MB + 2) == _lib.GLA_ERR_ALIGN


def test_decode_norm_requires_z(lib):
    P = ctypes.c_void_p
    st = lib.gla_decode_step_norm(P(A), P(A + MB), P(A + 2 * MB), P(A + 3 * MB), 1, P(A + 16 * MB), None,
                                  P(A + 64 * MB), 2, 4, 128, 128, 1, 0, None)
    assert st == _lib.GLA_ERR_NULL


def test_decode_norm_rejects_z_overlapping_state(lib):
    P = ctypes.c_void_p
    st = lib.gla_decode_step_norm(P(A), P(A + MB), P(A + 2 * MB), P(A + 3 * MB), 1, P(A + 16 * MB),
                                  P(A + 16 * MB + 1024), P(A + 64 * MB), 2, 4, 128, 128, 1, 0, None)
    assert st == _lib.GLA_ERR_ALIAS


# the delta rule: no gate or feature map; beta and a workspace always
def _prefill_delta(lib, **kw):
    args = dict(q=A, k=A + 16 * MB, v=A + 32 * MB, beta=A + 48 * MB, s0=None, o=A + 96 * MB,
                s_final=A + 128 * MB, B=1, H=2, L=64, d_k=64, d_v=64, chunk=64, dtype=1,
                ws=A + 256 * MB, ws_bytes=1 * MB)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_prefill_delta(P(args["q"]), P(args["k"]), P(args["v"]), P(args["beta"]), P(args["s0"]),
                                 P(args["o"]), P(args["s_final"]), args["B"], args["H"], args["L"],
                                 args["d_k"], args["d_v"], args["chunk"], args["dtype"], P(args["ws"]),
                                 args["ws_bytes"], None)


PREFILL_DELTA_BAD = {
    "B_zero": (dict(B=0), _lib.GLA_ERR_SHAPE),
    "L_negative": (dict(L=-5), _lib.GLA_ERR_SHAPE),
    "d_k_48": (dict(d_k=48), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_128": (dict(chunk=128), _lib.GLA_ERR_UNSUPPORTED),
    "dtype_2": (dict(dtype=2), _lib.GLA_ERR_UNSUPPORTED),
    "beta_null": (dict(beta=None), _lib.GLA_ERR_NULL),
    "o_null": (dict(o=None), _lib.GLA_ERR_NULL),
    "beta_misaligned": (dict(beta=A + 48 * MB + 2), _lib.GLA_ERR_ALIGN),
    "q_misaligned": (dict(q=A + 8), _lib.GLA_ERR_ALIGN),
    "workspace_missing": (dict(ws=None, ws_bytes=0), _lib.GLA_ERR_WORKSPACE),
    "workspace_short": (dict(ws_bytes=64 * 128 * 2 * 2 - 2), _lib.GLA_ERR_WORKSPACE),
    "L_past_32bit_head_offsets": (dict(L=4194304, d_k=128, d_v=128), _lib.GLA_ERR_SHAPE),
    "o_overlaps_beta": (dict(o=A + 48 * MB + 64), _lib.GLA_ERR_ALIAS),
    "o_overlaps_workspace": (dict(o=A + 256 * MB + 4096), _lib.GLA_ERR_ALIAS),
    "workspace_overlaps_k": (dict(ws=A + 16 * MB + 1024), _lib.GLA_ERR_ALIAS),
    "s_final_overlaps_v": (dict(s_final=A + 32 * MB + 16), _lib.GLA_ERR_ALIAS),
    "s_final_partially_overlaps_s0": (dict(s0=A + 200 * MB, s_final=A + 200 * MB + 256), _lib.GLA_ERR_ALIAS),
}


@pytest.mark.parametrize("case", sorted(PREFILL_DELTA_BAD))
def test_prefill_delta_rejects(lib, case):
    kw, want = PREFILL_DELTA_BAD[case]
    assert _prefill_delta(lib, **kw) == want
    assert lib.gla_last_error_detail().decode() != ""


def test_delta_workspace_bytes(lib):
    """Chunks of 64: -W rows [B*H][padded L][d_k] and U~ [B*H][padded L][d_v], in the
    input dtype.  Chunks of 16 or 32 run fused and need none."""
    assert lib.gla_delta_workspace_bytes(8, 16, 4096, 128, 128, 64, 1) == 8 * 16 * 4096 * 256 * 2
    assert lib.gla_delta_workspace_bytes(1, 2, 100, 64, 32, 64, 0) == 2 * 128 * 96 * 4
    assert lib.gla_delta_workspace_bytes(8, 16, 4096, 128, 128, 32, 1) == 0
    assert lib.gla_delta_workspace_bytes(8, 16, 4096, 128, 128, 16, 0) == 0
    assert lib.gla_delta_workspace_bytes(1, 2, 0, 64, 32, 32, 0) == 0
    assert lib.gla_delta_workspace_bytes(1, 2, 100, 48, 32, 32, 0) == 0


def _decode_delta(lib, **kw):
    args = dict(q=A, k=A + MB, v=A + 2 * MB, beta=A + 3 * MB, state=A + 16 * MB, o=A + 64 * MB,
                B=2, H=4, d_k=128, d_v=128, dtype=1)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_decode_step_delta(P(args["q"]), P(args["k"]), P(args["v"]), P(args["beta"]),
                                     P(args["state"]), P(args["o"]), args["B"], args["H"], args["d_k"],
                                     args["d_v"], args["dtype"], None)


DECODE_DELTA_BAD = {
    "beta_null": (dict(beta=None), _lib.GLA_ERR_NULL),
    "state_null": (dict(state=None), _lib.GLA_ERR_NULL),
    "H_zero": (dict(H=0), _lib.GLA_ERR_SHAPE),
    "d_k_8": (dict(d_k=8), _lib.GLA_ERR_UNSUPPORTED),
    "beta_misaligned": (dict(beta=A + 3 * MB + 1), _lib.GLA_ERR_ALIGN),
    "o_overlaps_state": (dict(o=A + 16 * MB + 512), _lib.GLA_ERR_ALIAS),
    "state_overlaps_beta": (dict(state=A + 3 * MB), _lib.GLA_ERR_ALIAS),
}


@pytest.mark.parametrize("case", sorted(DECODE_DELTA_BAD))
def test_decode_delta_rejects(lib, case):
    kw, want = DECODE_DELTA_BAD[case]
    assert _decode_delta(lib, **kw) == want


def _gate(lib, **kw):
    args = dict(x=A, wd=A + 64 * MB, wu=A + 65 * MB, g=A + 128 * MB, B=2, L=64, dm=256, r=16, H=2, dk=64,
                tau=1.0, dtype=1)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_gate_project(P(args["x"]), P(args["wd"]), P(args["wu"]), P(args["g"]), args["B"], args["L"],
                                args["dm"], args["r"], args["H"], args["dk"], args["tau"], args["dtype"], None)


GATE_BAD = {
    "B_zero": (dict(B=0), _lib.GLA_ERR_SHAPE),
    "L_negative": (dict(L=-1), _lib.GLA_ERR_SHAPE),
    "d_model_48": (dict(dm=48), _lib.GLA_ERR_UNSUPPORTED),
    "rank_8": (dict(r=8), _lib.GLA_ERR_UNSUPPORTED),
    "d_k_24": (dict(dk=24), _lib.GLA_ERR_UNSUPPORTED),
    "tau_zero": (dict(tau=0.0), _lib.GLA_ERR_SHAPE),
    "tau_nan": (dict(tau=float("nan")), _lib.GLA_ERR_SHAPE),
    "x_null": (dict(x=None), _lib.GLA_ERR_NULL),
    "g_misaligned": (dict(g=A + 128 * MB + 4), _lib.GLA_ERR_ALIGN),
    "g_overlaps_w_up": (dict(g=A + 65 * MB + 16), _lib.GLA_ERR_ALIAS),
    "g_overlaps_x": (dict(g=A + 4096), _lib.GLA_ERR_ALIAS),
    "dtype_3": (dict(dtype=3), _lib.GLA_ERR_UNSUPPORTED),
}


@pytest.mark.parametrize("case", sorted(GATE_BAD))
def test_gate_project_rejects(lib, case):
    kw, want = GATE_BAD[case]
    assert _gate(lib, **kw) == want
    assert lib.gla_last_error_detail().decode() != ""


def _prefill_outer(lib, **kw):
    args = dict(q=A, k=A + 16 * MB, v=A + 32 * MB, g=A + 48 * MB, gv=A + 64 * MB, s0=None, o=A + 96 * MB,
                s_final=A + 128 * MB, B=1, H=2, L=64, d_k=64, d_v=64, chunk=64, dtype=1, phi=0)
    args.update(kw)
    P = ctypes.c_void_p
    return lib.gla_prefill_outer(P(args["q"]), P(args["k"]), P(args["v"]), P(args["g"]), P(args["gv"]),
                                 P(args["s0"]), P(args["o"]), P(args["s_final"]), args["B"], args["H"], args["L"],
                                 args["d_k"], args["d_v"], args["chunk"], args["dtype"], args["phi"], None)


PREFILL_OUTER_BAD = {
    "g_null": (dict(g=None), _lib.GLA_ERR_NULL),
    "gv_null": (dict(gv=None), _lib.GLA_ERR_NULL),
    "gv_misaligned": (dict(gv=A + 64 * MB + 4), _lib.GLA_ERR_ALIGN),
    "d_v_8": (dict(d_v=8), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_48": (dict(chunk=48), _lib.GLA_ERR_UNSUPPORTED),
    "chunk_128": (dict(chunk=128), _lib.GLA_ERR_UNSUPPORTED),
    "phi_7": (dict(phi=7), _lib.GLA_ERR_UNSUPPORTED),
    "o_overlaps_gv": (dict(o=A + 64 * MB + 512), _lib.GLA_ERR_ALIAS),
    "s_final_overlaps_gv": (dict(s_final=A + 64 * MB + 1024), _lib.GLA_ERR_ALIAS),
    "s_final_partially_overlaps_s0": (dict(s0=A + 200 * MB, s_final=A + 200 * MB + 256), _lib.GLA_ERR_ALIAS),
    "L_past_32bit_head_offsets": (dict(L=4194304, d_k=128, d_v=128), _lib.GLA_ERR_SHAPE),
}


@pytest.mark.parametrize("case", sorted(PREFILL_OUTER_BAD))
def test_prefill_outer_rejects(lib, case):
    kw, want = PREFILL_OUTER_BAD[case]
    assert _prefill_outer(lib, **kw) == want
    assert lib.gla_last_error_detail().decode() != ""


def test_decode_outer_rejects(lib):
    P = ctypes.c_void_p
    call = lambda gv, state: lib.gla_decode_step_outer(P(A), P(A + MB), P(A + 2 * MB), P(A + 3 * MB), P(gv),
                                                       P(state), P(A + 64 * MB), 2, 4, 128, 128, 1, 0, None)
    assert call(None, A + 16 * MB) == _lib.GLA_ERR_NULL
    assert call(A + 4 * MB + 8, A + 16 * MB) == _lib.GLA_ERR_ALIGN
    assert call(A + 4 * MB, A + 4 * MB + 256) == _lib.GLA_ERR_ALIAS      # state overlaps gv


def test_prefill_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """The allocation-free prefill holds 32 MiB of scratch, which covers every size the
    automatic plan segments (at most 768 state-pass pieces of one value tile's state,
    24 MiB at d_k = 128 and 64-column tiles).  A
    plan forced through the test hook to more segments needs more and is rejected on
    the host, before any HIP call."""
    P = ctypes.c_void_p
    B, H, L = 1, 16, 64 * 2000
    assert lib.gla_prefill_workspace_bytes(B, H, L, 128, 128, 64, _lib.GLA_BF16) <= 32 << 20
    try:
        assert lib.gla_testing_set_plan(0, 64, 0) == _lib.GLA_OK      # 16 heads x 64 segments
        assert lib.gla_prefill_workspace_bytes(B, H, L, 128, 128, 64, _lib.GLA_BF16) > 32 << 20
        st = lib.gla_prefill_chunked_noalloc(P(A), P(A + 256 * MB), P(A + 512 * MB), P(A + 768 * MB), 1, None,
                                             P(A + 1280 * MB), None, B, H, L, 128, 128, 64, _lib.GLA_BF16, 0,
                                             None)
        detail = lib.gla_last_error_detail().decode()
    finally:
        lib.gla_testing_set_plan(0, 0, 0)
    assert st == _lib.GLA_ERR_WORKSPACE
    assert "scratch" in detail


def test_prefill_noalloc_scratch_covers_every_automatic_plan(lib):
    """The largest automatic segmented workspace over head counts and lengths (d = 128,
    the widest state) stays within the 32 MiB of scratch."""
    worst = max(lib.gla_prefill_workspace_bytes(1, bh, 64 * 4096, 128, 128, chunk, dt)
                for bh in range(1, 300) for chunk in (16, 32, 64) for dt in (_lib.GLA_BF16, _lib.GLA_F32))
    assert 0 < worst <= 32 << 20
    worst128 = max(lib.gla_prefill_workspace_bytes(1, bh, 128 * 2048, 64, dv, 128, dt)
                   for bh in range(1, 300) for dv in (64, 128) for dt in (_lib.GLA_BF16, _lib.GLA_F32))
    assert 0 < worst128 <= 32 << 20
