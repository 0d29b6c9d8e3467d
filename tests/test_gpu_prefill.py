"""GPU parity of gla_prefill_chunked (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs once and gives the same bits to both sides.  The
metric is the normwise relative error per (batch, head), max|x - ref| / max|ref|,
bounded by 2e-2 for bf16 inputs and 1e-4 for fp32 inputs; outputs and final states
are both compared.  Small cases cover all heads at sizes that span several chunks
and a ragged tail; the full workload sizes are checked on every head (the decode workload's
prefill on one head of each of its 256 sequences).
"""
import numpy as np
import pytest
import torch

from causal_gated_linear_amd import api, inputs
from oracle import oracle
from tests import util

pytestmark = pytest.mark.gpu
DEV = "cuda"
W = inputs.WORKLOADS


def _to(d, dev):
    return {k: (None if v is None else v.to(dev)) for k, v in d.items()}


def _run_gpu(w, inp, s0=None, chunk=None, **kw):
    o, s = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=inp["g"], gate=w.gate,
                       initial_state=s0, chunk=chunk or w.chunk, feature_map=w.feature_map, **kw)
    torch.cuda.synchronize()
    return o, s


def _check_all_heads(w, B, H, L, seed, chunk=None, with_s0=False):
    inp = inputs.draw(w, B=B, H=H, L=L, seed=seed)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=seed + 1, scale=0.5) if with_s0 else None
    o, s = _run_gpu(w, _to(inp, DEV), s0=None if s0 is None else s0.to(DEV), chunk=chunk)
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate,
                            feature_map=w.feature_map, s0=s0)
    tol = util.TOL[w.dtype]
    eo = util.assert_close(o, ro, tol, "%s o" % w.name)
    es = util.assert_close(s, rs, tol, "%s s_final" % w.name)
    print("%s B=%d H=%d L=%d chunk=%s s0=%s: err o %.2e s %.2e" % (w.name, B, H, L, chunk or w.chunk,
                                                                 with_s0, eo, es))
    return o, s


SMALL = {
    # name: (workload, B, H, L)  -- several chunks plus a ragged tail
    "fp32_single_head_full": ("fp32_single_head", 1, 1, 256),
    "fp32_single_head_ragged": ("fp32_single_head", 2, 3, 250),
    "linear_elu1_small": ("linear_elu1", 2, 3, 209),
    "gla_prefill_small": ("gla_prefill", 2, 2, 300),
    "scalar_long_small": ("scalar_long", 1, 3, 1000),
    "decode_prefill_small": ("decode", 3, 2, 130),
}


@pytest.mark.parametrize("case", sorted(SMALL))
@pytest.mark.parametrize("with_s0", [False, True])
def test_prefill_small(case, with_s0):
    name, B, H, L = SMALL[case]
    _check_all_heads(W[name], B, H, L, seed=100 + len(case), with_s0=with_s0)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("name", ["fp32_single_head", "gla_prefill", "scalar_long", "linear_elu1"])
def test_prefill_chunk_sizes(name, chunk):
    """Any chunk size gives the recurrence's result (chunking is a regrouping)."""
    _check_all_heads(W[name], 1, 2, 3 * chunk + 7, seed=7 + chunk, chunk=chunk, with_s0=True)


@pytest.mark.parametrize("L", [1, 15, 16, 17, 63, 64, 65, 129])
def test_prefill_lengths(L):
    _check_all_heads(W["gla_prefill"], 1, 2, L, seed=300 + L, with_s0=True)
    _check_all_heads(W["fp32_single_head"], 1, 2, L, seed=400 + L, with_s0=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 32), (16, 128), (128, 16)])
@pytest.mark.parametrize("gate", ["keydim", "scalar", None])
def test_prefill_dims(dtype, dk, dv, gate):
    w = inputs.Workload("dims", dtype, 2, 2, 150, dk, dv, 64, gate, None, True, seed=0)
    _check_all_heads(w, 2, 2, 150, seed=dk * 1000 + dv + (0 if gate is None else len(gate)), with_s0=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(32, 64), (128, 128), (64, 16)])
@pytest.mark.parametrize("gate", ["keydim", "scalar"])
def test_prefill_elu1_with_gates(dtype, dk, dv, gate):
    """phi = elu + 1 together with gates (the key-dimension path forms phi(x) e^(+-B)
    with one exponential), against the oracle's phi then gate."""
    w = inputs.Workload("elu1_gated", dtype, 2, 2, 150, dk, dv, 64, gate, "elu1", True, seed=0)
    _check_all_heads(w, 2, 2, 150, seed=7 * dk + dv + len(gate), with_s0=True)


def test_prefill_empty_sequence_copies_state():
    w = W["gla_prefill"]
    s0 = inputs.draw_state(2, 3, 128, 128, seed=5).to(DEV)
    z = torch.empty(2, 3, 0, 128, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(2, 3, 0, 128, dtype=torch.float32, device=DEV)
    o, s = api.prefill(z, z, z, log_gate=g, gate="keydim", initial_state=s0, chunk=w.chunk)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 128) and torch.equal(s, s0)
    o, s = api.prefill(z, z, z, log_gate=g, gate="keydim", chunk=w.chunk)
    torch.cuda.synchronize()
    assert torch.count_nonzero(s).item() == 0


def test_prefill_in_place_state():
    """final_state may be the initial_state buffer (continue in place)."""
    w = W["gla_prefill"]
    inp = _to(inputs.draw(w, B=2, H=2, L=200, seed=11), DEV)
    s0 = inputs.draw_state(2, 2, 128, 128, seed=12).to(DEV)
    o_ref, s_ref = _run_gpu(w, inp, s0=s0.clone())
    buf = s0.clone()
    o, s = _run_gpu(w, inp, s0=buf, final_state=buf)
    assert s.data_ptr() == buf.data_ptr()
    assert torch.equal(o, o_ref) and torch.equal(buf, s_ref)


def test_prefill_gate_none_equals_zero_keydim_gate():
    w = W["gla_prefill"]
    inp = _to(inputs.draw(w, B=1, H=2, L=190, seed=13), DEV)
    o1, s1 = api.prefill(inp["q"], inp["k"], inp["v"], chunk=64)
    o2, s2 = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=torch.zeros_like(inp["g"]), gate="keydim", chunk=64)
    o3, s3 = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=torch.zeros_like(inp["g"][..., 0]).contiguous(),
                         gate="scalar", chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)


def test_prefill_scalar_equals_broadcast_keydim():
    w = W["scalar_long"]
    inp = _to(inputs.draw(w, B=1, H=2, L=333, seed=14), DEV)
    o1, s1 = _run_gpu(w, inp)
    gk = inp["g"][..., None].expand(-1, -1, -1, 128).contiguous()
    o2, s2 = api.prefill(inp["q"], inp["k"], inp["v"], log_gate=gk, gate="keydim", chunk=64)
    torch.cuda.synchronize()
    assert util.head_errors(o1, o2.double().cpu().numpy()).max() < 2e-2
    assert util.head_errors(s1, s2.double().cpu().numpy()).max() < 2e-2


def test_prefill_deterministic():
    w = W["gla_prefill"]
    inp = _to(inputs.draw(w, B=2, H=4, L=500, seed=15), DEV)
    o1, s1 = _run_gpu(w, inp)
    o2, s2 = _run_gpu(w, inp)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_nan_stays_causal_and_in_its_head():
    """A NaN in v at token t of one head reaches every later output of that head, and
    never another head or an earlier chunk.  (Inside t's own chunk, earlier rows may
    also turn NaN: the masked score 0 times NaN is NaN in the chunk product.)"""
    w = W["gla_prefill"]
    inp = _to(inputs.draw(w, B=1, H=2, L=256, seed=16), DEV)
    t_bad = 150
    inp["v"][0, 1, t_bad, 5] = float("nan")
    o, s = _run_gpu(w, inp)
    nan_rows = torch.isnan(o).any(dim=-1)[0]            # [H, L]
    chunk_start = t_bad // w.chunk * w.chunk
    assert not nan_rows[0].any()
    assert not nan_rows[1, :chunk_start].any()
    assert nan_rows[1, t_bad:].all()
    assert torch.isfinite(s[0, 0]).all() and not torch.isfinite(s[0, 1]).all()


# ---- full workload sizes, every head -------------------------------------------------
FULL = ["linear_elu1", "gla_prefill", "scalar_long"]


@pytest.mark.parametrize("name", FULL)
def test_prefill_full_size_all_heads(name):
    """The workloads at their specified sizes, in the launch configuration the
    benchmark times, every head against the oracle."""
    w = W[name]
    inp = inputs.draw(w, device=DEV)                    # seeded on the device, all sizes as specified
    o, s = _run_gpu(w, inp)
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate, feature_map=w.feature_map)
    tol = util.TOL[w.dtype]
    eo = util.assert_close(o, ro, tol, "%s o" % name)
    es = util.assert_close(s, rs, tol, "%s s" % name)
    print("%s full size, all %d heads: err o %.2e s %.2e" % (name, w.B * w.H, eo, es))


def test_prefill_decode_workload_one_head_per_sequence():
    """The decode workload's 512-token prefill (256 sequences x 32 heads): one head of
    every sequence against the oracle (the other heads share the launch)."""
    w = W["decode"]
    inp = inputs.draw(w, device=DEV)
    o, s = _run_gpu(w, inp)
    heads = [(b, (7 * b) % w.H) for b in range(w.B)]
    ro, rs = util.oracle_heads(inp, heads, w.gate, w.feature_map)
    tol = util.TOL[w.dtype]
    util.assert_close(util.pick_heads(o, heads), ro, tol, "decode prefill o")
    util.assert_close(util.pick_heads(s, heads), rs, tol, "decode prefill s")


# Few long sequences run as segments: a state-only pass per segment, a scan over the
# segments, then all segments in parallel ("Attention is recurrent", Prefill: the
# prefix states form a (weighted) scan).  These sizes trigger it: B*H = 2 heads with
# at least 64 chunks; the ragged lengths leave a short last segment.
SEGMENTED = {
    # name: (workload, B, H, L)
    "gla_prefill_seg": ("gla_prefill", 1, 2, 64 * 65 + 37),
    "scalar_seg": ("scalar_long", 1, 2, 64 * 80 + 5),
    "linear_elu1_seg": ("linear_elu1", 2, 1, 64 * 70),
    "fp32_seg": ("fp32_single_head", 1, 2, 16 * 70 + 9),
}


def test_segmented_sizes_use_a_workspace():
    for case, (name, B, H, L) in SEGMENTED.items():
        w = W[name]
        assert api.workspace_bytes(B, H, L, w.d_k, w.d_v, w.chunk, w.dtype) > 0, case
    w = W["gla_prefill"]
    assert api.workspace_bytes(w.B, w.H, w.L, w.d_k, w.d_v, w.chunk, w.dtype) == 0


@pytest.mark.parametrize("case", sorted(SEGMENTED))
@pytest.mark.parametrize("with_s0", [False, True])
def test_prefill_segmented(case, with_s0):
    name, B, H, L = SEGMENTED[case]
    _check_all_heads(W[name], B, H, L, seed=500 + len(case), with_s0=with_s0)


@pytest.mark.parametrize("nseg", [1, 2, 3, 7])
def test_prefill_segment_counts(nseg):
    """Any segmentation gives the recurrence's result (the scan is a regrouping)."""
    with util.plan_override(prefill_segments=nseg):
        _check_all_heads(W["gla_prefill"], 1, 2, 64 * 20 + 3, seed=600 + nseg, with_s0=True)
        _check_all_heads(W["scalar_long"], 1, 2, 64 * 20 + 3, seed=700 + nseg, with_s0=True)


@pytest.mark.parametrize("name", ["gla_prefill", "scalar_long"])
def test_prefill_value_tiles_agree(name):
    """Each value-column tile width (64, 32, 16; the launch picks one from the head
    count) gives the oracle's result, and the same bits: a tile changes only how many
    value columns one workgroup owns, not the arithmetic of any column."""
    w = W[name]
    B, H, L = 1, 2, 64 * 5 + 7
    inp = inputs.draw(w, B=B, H=H, L=L, seed=990 + len(name))
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=991 + len(name), scale=0.5)
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate,
                            feature_map=w.feature_map, s0=s0)
    tol = util.TOL[w.dtype]
    outs = {}
    for tile in ("64", "32", "16"):
        with util.plan_override(prefill_tile=int(tile)):
            o, s = _run_gpu(w, _to(inp, DEV), s0=s0.to(DEV))
        util.assert_close(o, ro, tol, "%s o, value tile %s" % (name, tile))
        util.assert_close(s, rs, tol, "%s s_final, value tile %s" % (name, tile))
        outs[tile] = (o.cpu(), s.cpu())
    for tile in ("32", "16"):
        assert torch.equal(outs[tile][0], outs["64"][0]), "o differs between value tiles %s and 64" % tile
        assert torch.equal(outs[tile][1], outs["64"][1]), "s_final differs between value tiles %s and 64" % tile


@pytest.mark.parametrize("gate", ["keydim", "scalar"])
def test_prefill_segmented_weak_gates_carry_state(gate):
    """Segments with weak gates, so that the state carried across segments matters:
    a mistake in the scan over segments (a dropped or misplaced gate total or segment
    state) would move the later segments' outputs well beyond the tolerance.  With the
    workloads' own gates the carried state has mostly decayed by the next segment."""
    w = W["gla_prefill"] if gate == "keydim" else W["scalar_long"]
    B, H, L = 1, 2, 64 * 21                         # three segments of 7 chunks
    inp = inputs.draw(w, B=B, H=H, L=L, seed=950 + len(gate))
    inp["g"] = inp["g"] * 0.01                      # weak decay, still <= 0
    with util.plan_override(prefill_segments=3):
        o, s = _run_gpu(w, _to(inp, DEV))
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=gate, feature_map=None)
    tol = util.TOL[w.dtype]
    # the last segment restarted from a zero state is far from the whole-sequence result
    t0 = 64 * 14
    tail = {key: t[:, :, t0:].contiguous() for key, t in inp.items()}
    ro_tail, _ = oracle.forward(tail["q"], tail["k"], tail["v"], g=tail["g"], gate=gate, feature_map=None)
    assert util.head_errors(ro_tail, ro[:, :, t0:]).min() > 10 * tol
    eo = util.assert_close(o, ro, tol, "%s weak-gate segmented o" % gate)
    es = util.assert_close(s, rs, tol, "%s weak-gate segmented s_final" % gate)
    print("%s weak gates, 3 segments: err o %.2e s %.2e" % (gate, eo, es))


def test_prefill_segmented_in_place_state():
    """s_final may be s0 on the segmented path too."""
    w = W["gla_prefill"]
    B, H, L = 1, 2, 64 * 66
    inp = inputs.draw(w, B=B, H=H, L=L, seed=801)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=802, scale=0.5)
    st = s0.to(DEV)
    o, s = _run_gpu(w, _to(inp, DEV), s0=st, final_state=st)
    assert s.data_ptr() == st.data_ptr()
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate, s0=s0)
    util.assert_close(o, ro, util.TOL[w.dtype], "o")
    util.assert_close(s, rs, util.TOL[w.dtype], "s_final in place")


def test_prefill_segmented_in_place_state_with_more_workgroups_than_cus():
    """In place on a segmented plan whose full pass has more workgroups (3 heads x 64
    segments x 2 value tiles = 384) than one round of the CUs runs at once: a segment's
    workgroups may start after the last segment's have written s_final, so the full
    pass reads a copy of s0 taken before its launches.  The result equals the
    out-of-place run bit for bit and meets the oracle on every head."""
    w = W["gla_prefill"]
    B, H, L = 1, 3, 64 * 2048
    assert api.workspace_bytes(B, H, L, w.d_k, w.d_v, w.chunk, w.dtype) > 0
    inp = inputs.draw(w, B=B, H=H, L=L, seed=803)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=804, scale=0.5)
    d = _to(inp, DEV)
    o1, s1 = _run_gpu(w, d, s0=s0.to(DEV))
    st = s0.to(DEV)
    o2, s2 = _run_gpu(w, d, s0=st, final_state=st)
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate=w.gate, s0=s0)
    util.assert_close(o2, ro, util.TOL[w.dtype], "o")
    util.assert_close(s2, rs, util.TOL[w.dtype], "s_final in place")


def test_prefill_noalloc_segmented_in_place_state():
    """The allocation-free prefill in place on a segmented plan: the copy of s0 goes to
    the library's scratch array; the result equals the out-of-place run bit for bit."""
    w = W["gla_prefill"]
    B, H, L = 1, 3, 64 * 2048
    assert api.workspace_bytes(B, H, L, w.d_k, w.d_v, w.chunk, w.dtype) > 0
    inp = inputs.draw(w, B=B, H=H, L=L, seed=805)
    s0 = inputs.draw_state(B, H, w.d_k, w.d_v, seed=806, scale=0.5)
    d = _to(inp, DEV)
    o1, s1 = _run_gpu(w, d, s0=s0.to(DEV))
    st = s0.to(DEV)
    o2 = torch.empty_like(o1)
    _, s2 = api.prefill_noalloc(d["q"], d["k"], d["v"], log_gate=d["g"], gate=w.gate, initial_state=st,
                                chunk=w.chunk, out=o2, final_state=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_on_side_stream_with_binding_workspace():
    """A segmented prefill on a side stream, whose workspace the binding allocates:
    the workspace stays reserved for that stream until its work is done, although the
    binding drops it on return (allocations on the current stream in between must not
    receive it)."""
    w = W["gla_prefill"]
    B, H, L = 1, 2, 64 * 66
    inp = inputs.draw(w, B=B, H=H, L=L, seed=812)
    assert api.workspace_bytes(B, H, L, w.d_k, w.d_v, w.chunk, w.dtype) > 0
    d = _to(inp, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pass
    o, s = api.prefill(d["q"], d["k"], d["v"], log_gate=d["g"], gate="keydim", chunk=64, stream=side)
    # the current stream now allocates and fills memory while the side stream may still run
    junk = [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    ro, rs = oracle.forward(inp["q"], inp["k"], inp["v"], g=inp["g"], gate="keydim")
    util.assert_close(o, ro, util.TOL[w.dtype], "side-stream o")
    util.assert_close(s, rs, util.TOL[w.dtype], "side-stream s_final")
