"""GPU parity of rope_bwd, rmsnorm_bwd, rope_rmsnorm_res_bwd, linear_bwd and layer_bwd
(through the C ABI) against the float64 oracle."""

import numpy as np
import pytest
import torch

import synth
import verified_transformer_backward_amd as vtb
from oracle import layer as L
from oracle import specs
from tests.gpu_helpers import TOL, assert_close, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def test_tiny_rope_and_rmsnorm():
    need_gpu()
    say("tiny: RoPE 32 pairs pos 5, RMSNorm n 64")
    t = synth.tiny_inputs()
    dx = vtb.rope_bwd(dev(t["rope_dy"]), pos0=t["rope_pos"], base=t["rope_base"])
    ref = L.rope_backward_rows(t["rope_dy"], [t["rope_pos"]], t["rope_base"])
    assert_close("rope", host(dx), ref, TOL["f32"])
    th = specs.rope_angles([5], 64)[0]
    r0, r1 = specs.rope_backward(t["rope_dy"][0, 0, 0::2], t["rope_dy"][0, 0, 1::2], th)
    assert_close("rope_pairs", host(dx)[0, 0, 0::2], r0, TOL["f32"])
    assert_close("rope_pairs1", host(dx)[0, 0, 1::2], r1, TOL["f32"])
    g = vtb.rmsnorm_bwd(dev(t["rms_x"]), dev(t["rms_gamma"]), dev(t["rms_dy"]), t["rms_eps"])
    ref = specs.rmsnorm_backward(t["rms_x"][0], t["rms_gamma"], t["rms_dy"][0], t["rms_eps"])
    assert_close("rmsnorm", host(g)[0], ref, TOL["f32"])


@pytest.mark.parametrize("layout", [0, 1])
def test_rope_positions_layouts_inplace(layout):
    need_gpu()
    say(f"rope layout {layout}, explicit positions up to 8191, in place")
    rng = np.random.default_rng(3)
    T, H, d = 37, 5, 128
    dy = rng.standard_normal((T, H, d)).astype(np.float32)
    pos = np.sort(rng.integers(0, 8192, T)).astype(np.int32)
    ref = L.rope_backward_rows(dy, pos, 10000.0, layout)
    x = dev(dy)
    vtb.rope_bwd(x, pos=torch.from_numpy(pos).cuda(), layout=layout, dx=x)
    torch.cuda.synchronize()
    assert_close("rope_inplace", host(x), ref, TOL["f32"])


# (T, H, d, layout, pad): the float4 kernel with a padded token stride, and the per-pair
# kernel (head_dim not a multiple of 4, or of 8 for the half-split layout)
@pytest.mark.parametrize("T,H,d,layout,pad", [(29, 20, 128, 0, 4), (29, 4, 64, 1, 12), (11, 3, 6, 0, 0), (11, 3, 12, 1, 2),
                                               (7, 64, 128, 1, 0), (5, 80, 128, 0, 0)])
def test_rope_strided_and_scalar_paths(T, H, d, layout, pad):
    need_gpu()
    say(f"rope T {T} H {H} d {d} layout {layout} token pad {pad}")
    rng = np.random.default_rng(T * 100 + d)
    full = rng.standard_normal((T, H * d + pad)).astype(np.float32)
    dy = full[:, : H * d].reshape(T, H, d)
    ref = L.rope_backward_rows(dy, np.arange(T) + 3, 10000.0, layout)
    buf = dev(full)
    dyv = buf[:, : H * d].view(T, H, d) if pad == 0 else buf.as_strided((T, H, d), (H * d + pad, d, 1))
    dxv = torch.zeros_like(buf).as_strided((T, H, d), (H * d + pad, d, 1))
    vtb.rope_bwd(dyv, pos0=3, layout=layout, dx=dxv)
    torch.cuda.synchronize()
    assert_close("rope", host(dxv), ref, TOL["f32"])


@pytest.mark.parametrize("rows,n", [(3, 64), (17, 2560), (5, 5000), (4, 100)])
def test_rmsnorm_shapes(rows, n):
    need_gpu()
    say(f"rmsnorm rows {rows} n {n}")
    rng = np.random.default_rng(n)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    dy = rng.standard_normal((rows, n)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    out = vtb.rmsnorm_bwd(dev(x), dev(g), dev(dy), 1e-6)
    torch.cuda.synchronize()
    assert_close("rmsnorm", host(out), L.rmsnorm_backward_rows(x, g, dy, 1e-6), TOL["f32"])


FUSED_CASES = [
    # T, H, d, layout, pos0, in place  (the first two take the float4 path, the rest the scalar one)
    (256, 20, 128, 0, 0, False),
    (33, 3, 64, 1, 100, False),
    (8, 32, 128, 1, 8000, True),
    (17, 5, 6, 0, 7, False),
    (40, 2, 12, 1, 3, True),
]


@pytest.mark.parametrize("T,H,d,layout,pos0,inplace", FUSED_CASES)
def test_fused_rope_rmsnorm_residual(T, H, d, layout, pos0, inplace):
    need_gpu()
    say(f"fused rope+rmsnorm+residual T {T} H {H} d {d} layout {layout} pos0 {pos0} in-place {inplace}")
    rng = np.random.default_rng(4 + T + d)
    C = H * d
    dq = rng.standard_normal((T, C)).astype(np.float32)
    x = rng.standard_normal((T, C)).astype(np.float32)
    g = rng.standard_normal((T, C)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, C).astype(np.float32)
    sc = 0.25
    dn = L.rope_backward_rows((sc * dq.astype(np.float64)).reshape(T, H, d), pos0 + np.arange(T), layout=layout)
    ref = g + L.rmsnorm_backward_rows(x, gamma, dn.reshape(T, C), 1e-6)
    gd = dev(g)
    out = vtb.rope_rmsnorm_res_bwd(dev(dq), dev(x), dev(gamma), gd, H, d, dq_scale=sc, pos0=pos0, layout=layout,
                                   dh_in=gd if inplace else None)
    torch.cuda.synchronize()
    assert_close("fused", host(out), ref, TOL["f32"])


# k-step counts (32 deep) of dX / dW: (2, 4), (2, 2), (80, 8), (1, 1), (5, 3), (3, 5): the
# GEMM's two-set pipeline ends on one, two or three steps depending on that count
@pytest.mark.parametrize("T,K,N", [(100, 72, 50), (64, 64, 64), (256, 2560, 2560), (3, 130, 7), (96, 80, 150),
                                   (160, 40, 70)])
def test_linear_shapes(T, K, N):
    need_gpu()
    say(f"linear T {T} K {K} N {N}")
    rng = np.random.default_rng(T + K + N)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    dy = rng.standard_normal((T, N)).astype(np.float32)
    dx, dw = vtb.linear_bwd(dev(x), dev(w), dev(dy))
    torch.cuda.synchronize()
    rx, rw = L.linear_backward(x, w, dy)
    assert_close("linear.dx", host(dx), rx, TOL["f32"])
    assert_close("linear.dw", host(dw), rw, TOL["f32"])
    # run twice: no atomics, bitwise deterministic
    dx2, dw2 = vtb.linear_bwd(dev(x), dev(w), dev(dy))
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)


@pytest.mark.parametrize("want_dx,want_dw", [(True, True), (False, True)])
def test_linear_large_tiles(want_dx, want_dw):
    """T 2048, K = N = 4096: 1536 (both products) or 1024 (dW alone) tiles of 128 x 128, so the
    launch takes the large-tile kernel (k-contiguous dX operands, r-contiguous dW operands
    transposed in registers). Sampled rows of dX and dW, across tile edges, against the
    oracle; a second call bitwise equal."""
    need_gpu()
    T, K, N = 2048, 4096, 4096
    say(f"linear large tiles T {T} K {K} N {N} dx {want_dx} dw {want_dw}")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, K)).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    dy = rng.standard_normal((T, N)).astype(np.float32)
    xd, wd, dyd = dev(x), dev(w), dev(dy)
    dx, dw = vtb.linear_bwd(xd, wd, dyd, want_dx=want_dx, want_dw=want_dw)
    torch.cuda.synchronize()
    x64, w64, dy64 = (a.astype(np.float64) for a in (x, w, dy))
    if want_dx:
        rows = np.array([0, 1, 63, 64, 127, 128, 1000, 1919, 2047])
        assert_close("linear.dx rows", host(dx)[rows], dy64[rows] @ w64.T, TOL["f32"])
    rows = np.array([0, 5, 127, 128, 255, 2049, 3071, 4095])
    assert_close("linear.dw rows", host(dw)[rows], x64[:, rows].T @ dy64, TOL["f32"])
    dx2, dw2 = vtb.linear_bwd(xd, wd, dyd, want_dx=want_dx, want_dw=want_dw)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw2) and (not want_dx or torch.equal(dx, dx2))


def test_linear_repeats_bitwise():
    """30 calls at the layer-chain shape give one bitwise result: a barrier that does not
    wait for another wave's LDS stores shows up here as a few wrong 32 x 16 tiles."""
    need_gpu()
    say("linear T 256 K 2560 N 2560, 30 repeats")
    rng = np.random.default_rng(7)
    x = dev(rng.standard_normal((256, 2560)).astype(np.float32))
    w = dev((rng.standard_normal((2560, 2560)) * 0.02).astype(np.float32))
    dy = dev(rng.standard_normal((256, 2560)).astype(np.float32))
    dx0, dw0 = vtb.linear_bwd(x, w, dy)
    for _ in range(30):
        dx, dw = vtb.linear_bwd(x, w, dy)
        assert torch.equal(dx, dx0) and torch.equal(dw, dw0)
    torch.cuda.synchronize()


_KEYS = {"x": "x", "gamma": "gamma", "W": "w", "o": "o", "q": "q", "K": "k", "V": "v", "P": "P"}


def _saved_to_dev(s):
    """Oracle saved-tensor names -> the binding's layer_bwd keys, uploaded as fp32."""
    return {_KEYS[k]: dev(np.ascontiguousarray(v, dtype=np.float32)) for k, v in s.items()}


def _layer_case(layer, T, H, d):
    p = synth.layer_inputs(layer, T=T, H=H, d=d)
    sc = 1.0 / np.sqrt(d)
    saved = L.layer_saved(p["h"], p["gamma"], p["K"], p["V"], p["W"], H, sc)
    saved32 = {k: v.astype(np.float32) for k, v in saved.items()}
    return saved32, sc


# one token (every product has a single row or a one-deep contraction), a ragged shape, a
# two-tile one; T 512 (the one-kernel dO/dP/dS step at its largest, two full 16-key tiles
# per wave) and T 520 (past it: the split-K sum, dP product and dS rows as three
# launches)
@pytest.mark.parametrize("T,H,d", [(1, 2, 64), (64, 2, 64), (100, 3, 128), (512, 2, 64), (520, 1, 64)])
def test_layer_bwd_small(T, H, d):
    need_gpu()
    say(f"layer_bwd T {T} H {H} d {d}")
    saved, sc = _layer_case(0, T, H, d)
    g = synth.layer_upstream_grad(T=T, H=H, d=d)
    ref = L.layer_backward(saved, g, H, sc)
    sdev = _saved_to_dev(saved)
    got = vtb.layer_bwd(sdev, dev(g), sc)
    torch.cuda.synchronize()
    for n, a, b in zip(("dh_in", "dW", "dK", "dV"), got, ref):
        e = assert_close(f"layer.{n}", host(a), b, TOL["f32"])
        say(f"layer.{n} rel_err={e:.2e}")


def test_layer_chain_30_layers_full_size():
    need_gpu()
    T, H, d, NL = 256, 20, 128, 30
    say("layer chain: 30 layers T256 C2560, building saved tensors with the oracle forward")
    saved, sc = [], 1.0 / np.sqrt(d)
    for l in range(NL):
        s, _ = _layer_case(l, T, H, d)
        saved.append(s)
    g0 = synth.layer_upstream_grad(T=T, H=H, d=d)
    say("layer chain: GPU backward over 30 layers")
    g = dev(g0)
    grads = {}
    for l in reversed(range(NL)):
        sd = _saved_to_dev(saved[l])
        dh_in, dw, dk, dv = vtb.layer_bwd(sd, g, sc)
        if l in (0, NL - 1):
            grads[l] = (host(dw), host(dk), host(dv))
        g = dh_in
    torch.cuda.synchronize()
    say("layer chain: oracle backward over 30 layers")
    gr = g0.astype(np.float64)
    for l in reversed(range(NL)):
        gr, dW, dK, dV = L.layer_backward(saved[l], gr, H, sc, want_dw=l in grads)
        if l in grads:
            for n, a, b in zip(("dW", "dK", "dV"), grads[l], (dW, dK, dV)):
                e = assert_close(f"layer{l}.{n}", a, b, TOL["f32"])
                say(f"layer{l}.{n} rel_err={e:.2e}")
    e = assert_close("chain.g0", host(g), gr, TOL["f32"])
    say(f"chain.g0 rel_err={e:.2e}")


def test_layer_bwd_graph_replays_match_eager():
    # a graph captured over a two-layer chain (dh_in written over dh_out) must replay, again
    # and again with eager work in between, to the eager results bit for bit
    need_gpu()
    T, H, d = 64, 2, 64
    say("layer_bwd graph capture: two layers T64 H2 d64, three replays")
    sc = 1.0 / np.sqrt(d)
    sds = [_saved_to_dev(_layer_case(l, T, H, d)[0]) for l in range(2)]
    g0 = dev(synth.layer_upstream_grad(T=T, H=H, d=d))
    cfg = vtb.make_layer_cfg(T, H, d, sc)
    ws = torch.empty(vtb.layer_bwd_workspace_size(cfg), dtype=torch.uint8, device="cuda:0")
    g = torch.empty_like(g0)
    outs = [(torch.empty_like(sds[l]["w"]), torch.empty_like(sds[l]["k"]), torch.empty_like(sds[l]["v"])) for l in range(2)]

    def chain():
        g.copy_(g0)
        for l in (1, 0):
            dw, dk, dv = outs[l]
            vtb.layer_bwd(sds[l], g, sc, dh_in=g, dw=dw, dk=dk, dv=dv, workspace=ws, stream=torch.cuda.current_stream())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [g.clone()] + [t.clone() for o in outs for t in o]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        chain()
    for rep in range(3):
        g.zero_()
        for o in outs:
            for t in o:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [g] + [t for o in outs for t in o]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"


# bf16 storage: (T, H, d, layout, token pad) on the 8-element vector kernel (rows of up to
# 2048 vectors, both layouts) and on the per-pair kernel (head_dim not a multiple of 8, or
# of 16 for the half-split layout, and rows wider than the vector kernel)
@pytest.mark.parametrize("T,H,d,layout,pad", [(29, 20, 128, 0, 8), (29, 4, 64, 1, 16), (11, 3, 12, 0, 0),
                                               (11, 3, 24, 1, 0), (5, 80, 128, 0, 0), (3, 160, 128, 1, 0)])
def test_rope_bf16(T, H, d, layout, pad):
    need_gpu()
    say(f"rope bf16 T {T} H {H} d {d} layout {layout} token pad {pad}")
    rng = np.random.default_rng(T * 1000 + d + layout)
    full = synth.bf16_round(rng.standard_normal((T, H * d + pad)).astype(np.float32))
    dy = full[:, : H * d].reshape(T, H, d)
    ref = L.rope_backward_rows(dy, np.arange(T) + 7, 10000.0, layout)
    buf = dev(full, "bf16")
    dyv = buf.as_strided((T, H, d), (H * d + pad, d, 1))
    dxv = torch.zeros_like(buf).as_strided((T, H, d), (H * d + pad, d, 1))
    vtb.rope_bwd(dyv, pos0=7, layout=layout, dx=dxv)
    torch.cuda.synchronize()
    assert_close("rope bf16", host(dxv), ref, TOL["bf16"])


def test_rope_bf16_in_place_positions():
    need_gpu()
    say("rope bf16 in place, explicit positions up to 8191")
    rng = np.random.default_rng(11)
    T, H, d = 37, 5, 128
    dy = synth.bf16_round(rng.standard_normal((T, H, d)).astype(np.float32))
    pos = np.sort(rng.integers(0, 8192, T)).astype(np.int32)
    x = dev(dy, "bf16")
    vtb.rope_bwd(x, pos=torch.from_numpy(pos).cuda(), dx=x)
    torch.cuda.synchronize()
    assert_close("rope bf16 in place", host(x), L.rope_backward_rows(dy, pos, 10000.0, 0), TOL["bf16"])


@pytest.mark.parametrize("rows,n", [(3, 64), (17, 2560), (5, 5000), (4, 100)])
def test_rmsnorm_bf16(rows, n):
    need_gpu()
    say(f"rmsnorm bf16 rows {rows} n {n}")
    rng = np.random.default_rng(n + 1)
    x = synth.bf16_round(rng.standard_normal((rows, n)).astype(np.float32))
    dy = synth.bf16_round(rng.standard_normal((rows, n)).astype(np.float32))
    g = rng.uniform(0.5, 1.5, n).astype(np.float32)
    out = vtb.rmsnorm_bwd(dev(x, "bf16"), dev(g), dev(dy, "bf16"), 1e-6)
    torch.cuda.synchronize()
    assert_close("rmsnorm bf16", host(out), L.rmsnorm_backward_rows(x, g, dy, 1e-6), TOL["bf16"])
