#!/usr/bin/env python3
"""Benchmark of the attention-layer backward on one MI355X.

One step = one attn_bwd call (query-parallel dq pass, key-parallel dk/dv pass) over the
causal training workload B4 H20 T512 d128: q, k, v, dO bf16 ~ N(0, 1), saved
row log-sum-exp fp32 (from the library's own attn_fwd_lse, computed before timing),
scale 1/sqrt(128), bf16 outputs with fp32 accumulation. Inputs are resident in HBM
before the timed region. By default the step rotates over 8 copies of inputs, outputs
and workspace (~760 MB) so no step finds its data in the 256 MB Infinity Cache ("cold");
a warm number (one set reused) is reported beside it.

The K timed steps are captured once into a HIP graph (the same two launches per step)
and replayed between two HIP events, so the host's launch cost is not in the step time;
the graph's outputs are checked bit for bit against an eager call before timing.

Prints ONE JSON line. `value` is TFLOP/s of the five contractions the method counts
(S recompute, dP, dQ, dK, dV) on the exact causal triangle: 10 * d * B * H * T(T+1)/2.
The roofline object is for the dominant kernel (the longer of the two passes), timed
live over the eager steps with HIP events that attn_bwd_timed has the kernel's own
dispatch record at its start and end, on the launch stream.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn-backward TFLOP/s & HBM GB/s at B4·H20·T512·d128; % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_MFMA_PEAK_TFLOPS = 157.3
MAIN_KERNEL_SRC = os.path.join(ROOT, "verified_transformer_backward_amd", "csrc", "attn_bwd_mfma.hip")
PMC_SUMMARY = {k: os.path.join(ROOT, "profiles", f"attn_{k}_causal_train_B4H20T512d128_pmc.json") for k in ("dq", "dkdv")}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=8, help="rotating input/output sets (1 = warm only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU-baseline sample time")
    ap.add_argument("--no-extra", action="store_true", help="skip the other hot-path workloads")
    ap.add_argument("--only", default="", help="run only these other workloads (comma list, e.g. layer_chain) "
                                               "and print their results; no headline step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 256 MiB device copy (for scaling profiler byte counters)")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (one runtime per process)."""

    def __init__(self):
        import torch

        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def workload_numbers(B, T, H, d):
    """Algorithmic work of the step and of each pass (causal triangle, bf16 in/out).

    dq pass:   S, dP, (P o dP) K, P K contractions; reads q, k, v, dO, lse once, writes D, dQ.
    dkdv pass: S, dP, dV, dK contractions; reads q, k, v, dO, lse, D once, writes dK, dV.
    Per-pass flops are the contractions the pass executes on the causal triangle.
    """
    pairs = B * H * T * (T + 1) // 2                      # visible (query, key) pairs
    flops = 10 * d * pairs                                # the 5 contractions the method counts
    n = B * T * H * d
    rows = B * H * T
    compulsory = 4 * n * 2 + rows * 4 + 3 * n * 2         # q,k,v,dO + lse in, dq,dk,dv bf16 out
    per_kernel = {
        "dq": {"flops": 8 * d * pairs, "bytes": 4 * n * 2 + rows * 4 + rows * 4 + n * 2},
        "dkdv": {"flops": 8 * d * pairs, "bytes": 4 * n * 2 + 2 * rows * 4 + 2 * n * 2},
    }
    return flops, compulsory, per_kernel


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when it is missing or was taken on a different version of the kernel source."""
    try:
        rec = json.load(open(PMC_SUMMARY[kernel]))
        src = hashlib.sha256(open(MAIN_KERNEL_SRC, "rb").read()).hexdigest()
        if rec.get("source_sha256") != src:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def graph_ms(torch, hip, fn, reps):
    """ms per call of fn(), from one HIP graph holding `reps` calls replayed between events."""
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        fn()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    start, stop = hip.create(2)
    sp = torch.cuda.current_stream().cuda_stream
    hip.record(start, sp)
    g.replay()
    hip.record(stop, sp)
    torch.cuda.synchronize()
    ms = hip.ms(start, stop) / reps
    hip.destroy([start, stop])
    return ms


EXTRA_NAMES = ("single_query", "decode_gqa", "decode_fwd", "long_causal", "causal_train_f32out", "causal_train_saved_o", "rope_rmsnorm_res", "rope_bwd",
               "rmsnorm_bwd", "layer_chain", "attn_fwd", "layernorm_bwd", "relu2_mul_bwd", "ffn_bwd", "attn_block_bwd", "rms_attn_block_bwd")


def copy_bandwidth(torch, hip):
    """A plain 1 GiB device-to-device copy (torch copy_: read 1 GiB, write 1 GiB), graph-replayed,
    for context beside the spec peak. Not a ceiling (the library's streaming kernels run faster)
    and never a roofline denominator."""
    src = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = graph_ms(torch, hip, lambda: dst.copy_(src), 5)
    byts = 2 * src.numel() * 4
    del src, dst
    return {"what": "1 GiB device copy (torch copy_), read + write", "ms": round(ms, 4),
            "gbps": round(byts / (ms * 1e-3) / 1e9, 1), "frac_of_spec": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def library_gemm_rates(torch, hip):
    """Measured matrix-core reference: a square 8192^3 torch matmul (the vendor BLAS, contiguous
    operands) in bf16 and in fp32, graph-replayed. Context beside the spec peaks, never a
    roofline denominator."""
    out = {}
    for name, dt, reps in (("bf16", torch.bfloat16, 10), ("fp32", torch.float32, 2)):
        n = 8192
        g = torch.Generator(device="cuda:0").manual_seed(1)
        a = torch.randn(n, n, generator=g, device="cuda:0").to(dt)
        b = torch.randn(n, n, generator=g, device="cuda:0").to(dt)
        c = torch.empty(n, n, device="cuda:0", dtype=dt)
        ms = graph_ms(torch, hip, lambda: torch.mm(a, b, out=c), reps)
        out[name] = {"what": f"torch.mm {n}^3 {name}", "ms": round(ms, 3), "tflops": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)}
        del a, b, c
    return out


def extra_workloads(torch, vtb, hip, only=None):
    """The other rows of the hot path at their workload sizes, each against its roofline.
    Inputs are seeded synthetic tensors; the layer chain's saved activations come from a
    plain torch fp32 forward of each layer (setup only, untimed). `only`: names to run."""
    import numpy as np
    import synth

    dev = torch.device("cuda:0")
    out = {}
    H, d = 20, 128
    C = H * d

    def want(name):
        return only is None or name in only

    def hbm_line(name, what, ms, byts):
        out[name] = {"workload": what, "ms": round(ms, 5), "value": round(byts / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                     "roofline": {"bound": "hbm", "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes": byts}}

    def up(a, dtype="f32"):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(synth.bf16_bits(a))).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    if want("single_query"):
        # the single-head, single-query case: attention backward (q[64], K, V [16 x 64], no lse),
        # RoPE backward on 32 pairs at position 5 and RMSNorm backward on n = 64, all fp32;
        # a step is the three calls. Launch latency sets the time, so only us per step is reported.
        x = synth.tiny_inputs()
        t = {n: up(x[n]) for n in ("q", "k", "v", "dout")}
        o = {n: torch.empty_like(t[n]) for n in ("q", "k", "v")}
        desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], False, torch.float32, t["dout"], o["q"], o["k"], o["v"], t["v"])
        ws = torch.empty(max(1, vtb.attn_bwd_workspace_size(desc)), dtype=torch.uint8, device=dev)
        rdy, rx, rdy2, rg = up(x["rope_dy"]), up(x["rms_x"]), up(x["rms_dy"]), up(x["rms_gamma"])
        rdx, rdx2 = torch.empty_like(rdy), torch.empty_like(rx)

        def f():
            st = torch.cuda.current_stream()
            vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], x["scale"], False, dq=o["q"], dk=o["k"], dv=o["v"],
                         workspace=ws, stream=st)
            vtb.rope_bwd(rdy, pos0=x["rope_pos"], base=x["rope_base"], dx=rdx, stream=st)
            vtb.rmsnorm_bwd(rx, rg, rdy2, eps=x["rms_eps"], dx=rdx2, stream=st)

        ms = graph_ms(torch, hip, f, 50)
        out["single_query"] = {"workload": "single-head single-query attention backward (Tk 16, d 64) + RoPE backward "
                                           "(32 pairs) + RMSNorm backward (n 64), fp32",
                               "ms": round(ms, 5), "value": round(ms * 1e3, 2), "unit": "us per step",
                               "higher_is_better": False, "roofline": None}
        del t, o, ws

    if want("decode_gqa"):
        # decode-shaped GQA: B8 Tq1 Hq20 Hkv5 Tk1024 d128 fp32, no lse (HBM-bound: K, V in, dK, dV out)
        x = synth.decode_gqa_inputs()
        t = {n: up(x[n]) for n in ("q", "k", "v", "dout")}
        o = {n: torch.empty_like(t[n]) for n in ("q", "k", "v")}
        desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], False, torch.float32, t["dout"], o["q"], o["k"], o["v"], t["v"])
        ws = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
        f = lambda: vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], x["scale"], False, dq=o["q"], dk=o["k"], dv=o["v"],
                                 workspace=ws, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 50)
        byts = sum(v.numel() * 4 for v in t.values()) + sum(v.numel() * 4 for v in o.values())
        out["decode_gqa"] = {"workload": "GQA decode B8 Tq1 Hq20 Hkv5 Tk1024 d128 fp32, lse computed", "ms": round(ms, 5),
                             "value": round(byts / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                             "roofline": {"bound": "hbm", "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                          "algorithmic_bytes": byts}}
        del t, o, ws

    if want("decode_fwd"):
        # split-KV decode forward (O and lse) on the GQA decode shape, B8 Tq1 Hq20 Hkv5 Tk1024
        # d128 fp32; 8 rotating input sets (336 MB of K and V) so that no call finds its K and
        # V in the Infinity Cache. HBM-bound: K and V read once.
        x = synth.decode_gqa_inputs()
        base = {n: up(x[n]) for n in ("q", "k", "v")}
        sets = []
        for _ in range(8):
            t = {n: v.clone() for n, v in base.items()}
            t["o"] = torch.empty_like(t["q"])
            t["lse"] = torch.empty((8, 20, 1), dtype=torch.float32, device=dev)
            desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], False, torch.float32, dq=t["o"], v=t["v"])
            t["ws"] = torch.empty(vtb.attn_fwd_workspace_size(desc), dtype=torch.uint8, device=dev)
            sets.append(t)
        it = iter(range(10 ** 9))

        def f():
            t = sets[next(it) % 8]
            vtb.attn_fwd(t["q"], t["k"], t["v"], x["scale"], False, o=t["o"], lse=t["lse"], workspace=t["ws"],
                         stream=torch.cuda.current_stream())

        ms = graph_ms(torch, hip, f, 40)
        byts = sum(base[n].numel() * 4 for n in ("q", "k", "v")) + base["q"].numel() * 4 + 8 * 20 * 4
        hbm_line("decode_fwd", "split-KV decode attention forward (O, lse) GQA B8 Tq1 Hq20 Hkv5 Tk1024 d128 fp32, "
                               "8 rotating sets", ms, byts)
        del sets, base

    if want("long_causal"):
        # long-context causal: B1 H32 T8192 d128 bf16, lse given (bf16 MFMA-bound)
        x = synth.long_causal_inputs()
        t = {n: up(x[n], "bf16") for n in ("q", "k", "v", "dout")}
        lse = vtb.attn_fwd_lse(t["q"], t["k"], x["scale"], True)
        o = {n: torch.empty_like(t[n]) for n in ("q", "k", "v")}
        desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], True, torch.bfloat16, t["dout"], o["q"], o["k"], o["v"], t["v"])
        ws = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
        f = lambda: vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], x["scale"], True, lse=lse, dq=o["q"], dk=o["k"],
                                 dv=o["v"], workspace=ws, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 5)
        fl = 10 * 128 * 32 * 8192 * 8193 // 2
        out["long_causal"] = {"workload": "causal B1 H32 T8192 d128 bf16, lse given", "ms": round(ms, 4),
                              "value": round(fl / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                              "roofline": {"bound": "mfma", "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                           "algorithmic_flops": fl}}
        del t, o, ws, lse

    if want("attn_fwd"):
        # attention forward (O and lse, online softmax) on the training shape: causal B4 H20 T512 d128 bf16
        x = synth.causal_inputs()
        t = {n: up(x[n], "bf16") for n in ("q", "k", "v")}
        o = torch.empty_like(t["q"])
        lse = torch.empty((4, 20, 512), dtype=torch.float32, device=dev)
        f = lambda: vtb.attn_fwd(t["q"], t["k"], t["v"], x["scale"], True, o=o, lse=lse, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        fl = 4 * 128 * 4 * 20 * 512 * 513 // 2     # S and P V: 2 contractions of 2 d FLOP per visible pair
        byts = 4 * t["q"].numel() * 2 + lse.numel() * 4   # q, k, v read, o written (bf16), lse written
        out["attn_fwd"] = {"workload": "attention forward (O, lse), causal B4 H20 T512 d128 bf16", "ms": round(ms, 5),
                           "value": round(fl / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                           "hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
                           "roofline": {"bound": "mfma", "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                        "algorithmic_flops": fl, "algorithmic_bytes": byts}}
        del t, o, lse

    if want("causal_train_f32out"):
        # the headline workload with fp32 outputs (bf16 in, fp32 accumulation, dQ/dK/dV fp32),
        # 4 rotating input sets so the step does not find its data in the Infinity Cache
        x = synth.causal_inputs()
        base = {n: up(x[n], "bf16") for n in ("q", "k", "v", "dout")}
        sets = []
        for _ in range(4):
            t = {n: v.clone() for n, v in base.items()}
            t["lse"] = vtb.attn_fwd_lse(t["q"], t["k"], x["scale"], True)
            t["o"] = [torch.empty(t[n].shape, dtype=torch.float32, device=dev) for n in ("q", "k", "v")]
            desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], True, torch.float32, t["dout"], *t["o"], t["v"])
            t["ws"] = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
            sets.append(t)
        it = iter(range(10 ** 9))

        def f():
            t = sets[next(it) % 4]
            vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], x["scale"], True, lse=t["lse"], out_dtype=torch.float32,
                         dq=t["o"][0], dk=t["o"][1], dv=t["o"][2], workspace=t["ws"], stream=torch.cuda.current_stream())

        ms = graph_ms(torch, hip, f, 20)
        fl = 10 * 128 * 4 * 20 * 512 * 513 // 2
        byts = 4 * base["q"].numel() * 2 + 4 * 20 * 512 * 4 + 3 * base["q"].numel() * 4
        ceil = min(BF16_MFMA_PEAK_TFLOPS, fl / byts * HBM_PEAK_GBS / 1e3)
        out["causal_train_f32out"] = {"workload": "causal attention backward B4 H20 T512 d128, bf16 in, fp32 out, lse given, "
                                                  "4 rotating sets", "ms": round(ms, 5),
                                      "value": round(fl / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                                      "hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
                                      "roofline": {"bound": "hbm", "ceiling_tflops": round(ceil, 1),
                                                   "frac": round(fl / (ms * 1e-3) / 1e12 / ceil, 4),
                                                   "frac_bf16_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                                   "algorithmic_flops": fl, "algorithmic_bytes": byts}}
        del sets, base

    if want("causal_train_saved_o"):
        # the headline workload for callers that saved the forward's O (attn_bwd_o): the row
        # term is dO . O, so the query pass takes three contractions per key block; 8 rotating
        # sets, O and lse from the library's own forward (untimed)
        x = synth.causal_inputs()
        base = {n: up(x[n], "bf16") for n in ("q", "k", "v", "dout")}
        sets = []
        for _ in range(8):
            t = {n: v.clone() for n, v in base.items()}
            t["o"], t["lse"] = vtb.attn_fwd(t["q"], t["k"], t["v"], x["scale"], True)
            t["g"] = [torch.empty_like(t[n]) for n in ("q", "k", "v")]
            desc = vtb.make_attn_desc(t["q"], t["k"], x["scale"], True, torch.bfloat16, t["dout"], *t["g"], t["v"])
            t["ws"] = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
            sets.append(t)
        it = iter(range(10 ** 9))

        def f():
            t = sets[next(it) % 8]
            vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], x["scale"], True, lse=t["lse"], o=t["o"], dq=t["g"][0],
                         dk=t["g"][1], dv=t["g"][2], workspace=t["ws"], stream=torch.cuda.current_stream())

        ms = graph_ms(torch, hip, f, 40)
        fl = 10 * 128 * 4 * 20 * 512 * 513 // 2      # the same counted work as the headline
        byts = 5 * base["q"].numel() * 2 + 4 * 20 * 512 * 4 + 3 * base["q"].numel() * 2
        out["causal_train_saved_o"] = {"workload": "causal attention backward B4 H20 T512 d128 bf16 with saved O and lse "
                                                   "(attn_bwd_o), 8 rotating sets", "ms": round(ms, 5),
                                       "value": round(fl / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                                       "hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
                                       "roofline": {"bound": "mfma",
                                                    "frac": round(fl / (ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                                    "algorithmic_flops": fl, "algorithmic_bytes": byts}}
        del sets, base

    if want("rope_rmsnorm_res") or want("rope_bwd") or want("rmsnorm_bwd"):
        # fused RoPE -> RMSNorm -> residual tail on the stack shape (30 x 256 rows, hidden 2560), fp32
        rows, H, d = 30 * 256, 20, 128
        C = H * d
        rng = np.random.default_rng(1007)
        dq_, xx, dh = (torch.from_numpy(rng.standard_normal((rows, C)).astype(np.float32)).to(dev) for _ in range(3))
        gam = torch.from_numpy(rng.uniform(0.5, 1.5, C).astype(np.float32)).to(dev)
        dh_in = torch.empty_like(dh)
        f = lambda: vtb.rope_rmsnorm_res_bwd(dq_, xx, gam, dh, H, d, dh_in=dh_in, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        byts = 4 * rows * C * 4
        out["rope_rmsnorm_res"] = {"workload": "fused RoPE+RMSNorm+residual backward, 7680 x 2560 fp32", "ms": round(ms, 5),
                                   "value": round(byts / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                   "roofline": {"bound": "hbm", "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                                "algorithmic_bytes": byts}}
        dy3 = dq_.view(rows, H, d)
        dx3 = torch.empty_like(dy3)
        f = lambda: vtb.rope_bwd(dy3, dx=dx3, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        byts = 2 * rows * C * 4
        out["rope_bwd"] = {"workload": "RoPE backward, 7680 x 20 x 128 fp32", "ms": round(ms, 5),
                           "value": round(byts / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                           "roofline": {"bound": "hbm", "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "algorithmic_bytes": byts}}
        f = lambda: vtb.rmsnorm_bwd(xx, gam, dh, dx=dh_in, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        byts = 3 * rows * C * 4
        out["rmsnorm_bwd"] = {"workload": "RMSNorm backward, 7680 x 2560 fp32", "ms": round(ms, 5),
                              "value": round(byts / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                              "roofline": {"bound": "hbm", "frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                           "algorithmic_bytes": byts}}
        # the same RoPE and RMSNorm backwards in bf16 storage (fp32 arithmetic, gamma fp32)
        xb, db = xx.to(torch.bfloat16), dh.to(torch.bfloat16)
        dy3b, dx3b, dxb = db.view(rows, H, d), torch.empty_like(db).view(rows, H, d), torch.empty_like(db)
        f = lambda: vtb.rope_bwd(dy3b, dx=dx3b, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        hbm_line("rope_bwd_bf16", "RoPE backward, 7680 x 20 x 128 bf16", ms, 2 * rows * C * 2)
        f = lambda: vtb.rmsnorm_bwd(xb, gam, db, dx=dxb, stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 20)
        hbm_line("rmsnorm_bwd_bf16", "RMSNorm backward, 7680 x 2560 bf16", ms, 3 * rows * C * 2 + C * 4)
        del dq_, xx, dh, dh_in, dy3, dx3, xb, db, dy3b, dx3b, dxb

    if want("layernorm_bwd"):
        # LayerNorm (no affine) backward, 7680 x 2560: dy, y read, dx written, sigma per row
        rows, n = 30 * 256, 2560
        for dt, tdt, es in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
            inp = synth.layernorm_inputs(rows, n, dt)
            x = up(inp["x"], dt).float()
            mu = x.mean(1, keepdim=True)
            sig = torch.sqrt(((x - mu) ** 2).mean(1) + 1e-5).contiguous()
            y = ((x - mu) / sig[:, None]).to(tdt).contiguous()
            dy, dx = up(inp["dy"], dt), torch.empty_like(y)
            f = lambda: vtb.layernorm_bwd(dy, y, sig, dx=dx, stream=torch.cuda.current_stream())
            ms = graph_ms(torch, hip, f, 20)
            hbm_line("layernorm_bwd" + ("" if dt == "f32" else "_bf16"), f"LayerNorm backward, {rows} x {n} {dt}", ms,
                     3 * rows * n * es + rows * 4)
            del x, y, dy, dx, sig

    if want("relu2_mul_bwd"):
        # ReLU^2 x Mul backward over the FFN activations of 30 x 256 tokens x 6912: gate, up, dh read, dgate, dup written
        n = 30 * 256 * 6912
        gen = torch.Generator(device=dev).manual_seed(1007)
        for tdt, es, tag in ((torch.float32, 4, "f32"), (torch.bfloat16, 2, "bf16")):
            g, u, dh = (torch.randn(n, generator=gen, device=dev).to(tdt) for _ in range(3))
            dg, du = torch.empty_like(g), torch.empty_like(g)
            f = lambda: vtb.relu2_mul_bwd(g, u, dh, dgate=dg, dup=du, stream=torch.cuda.current_stream())
            ms = graph_ms(torch, hip, f, 20)
            hbm_line("relu2_mul_bwd" + ("" if tag == "f32" else "_bf16"), f"ReLU^2 x Mul backward, 7680 x 6912 {tag}", ms,
                     5 * n * es)
            del g, u, dh, dg, du

    if want("ffn_bwd"):
        # one FFN block's backward, T256 C2560 F6912 fp32; saved activations from a torch fp32 forward (setup only)
        T, Cf, F = 256, 2560, 6912
        p = synth.ffn_inputs(T, Cf, F)
        x, g1, wgu, g2, wd, dout = (up(p[n]) for n in ("x", "gamma1", "w_gu", "gamma2", "w_down", "dout"))
        rms = lambda z, g: z * torch.rsqrt((z * z).mean(1, keepdim=True) + 1e-6) * g
        xn = rms(x, g1).contiguous()
        gu = (xn @ wgu).contiguous()
        hn = rms(torch.relu(gu[:, :F]) ** 2 * gu[:, F:], g2).contiguous()
        saved = {"x": x, "gamma1": g1, "xn": xn, "w_gu": wgu, "gu": gu, "gamma2": g2, "hn": hn, "w_down": wd}
        dx, dwgu, dwd = torch.empty_like(dout), torch.empty_like(wgu), torch.empty_like(wd)
        fws = torch.empty(vtb.ffn_bwd_workspace_size(vtb.make_ffn_cfg(T, Cf, F)), dtype=torch.uint8, device=dev)
        f = lambda: vtb.ffn_bwd(saved, dout, dx=dx, dw_gu=dwgu, dw_down=dwd, workspace=fws,
                                stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 5)
        fl = 12 * T * Cf * F
        out["ffn_bwd"] = {"workload": "FFN block backward, T256 C2560 F6912 fp32 (gate/up/down GEMMs, norms, ReLU^2 x Mul)",
                          "ms": round(ms, 4), "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                          "roofline": {"bound": "mfma", "peak": FP32_MFMA_PEAK_TFLOPS,
                                       "frac": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                                       "algorithmic_flops": fl}}
        del saved, x, xn, gu, hn, wgu, wd, dx, dwgu, dwd, fws

    if want("attn_block_bwd"):
        # one transformer attention block's backward (LayerNorm, QKV and output projections,
        # causal attention with the saved softmax), T256 20 x 128 fp32; saved activations
        # from a torch fp32 forward (setup only)
        Tb, Hb, db = 256, 20, 128
        Cb = Hb * db
        sc = 1.0 / np.sqrt(db)
        p = synth.block_inputs(1, Tb, Hb, db)
        xin, wqkv, wo, dx2 = (up(p[n]) for n in ("xin", "w_qkv", "w_o", "dx2"))
        mu = xin.mean(1, keepdim=True)
        sig = torch.sqrt(((xin - mu) ** 2).mean(1) + 1e-5).contiguous()
        ln_y = ((xin - mu) / sig[:, None]).contiguous()
        qkv = (ln_y @ wqkv).contiguous()
        hsplit = lambda z: z.reshape(Tb, Hb, db).permute(1, 0, 2).contiguous()
        q, k, v = hsplit(qkv[:, :Cb]), hsplit(qkv[:, Cb:2 * Cb]), hsplit(qkv[:, 2 * Cb:])
        mask = torch.tril(torch.ones(Tb, Tb, dtype=torch.bool, device=dev))
        S = torch.matmul(q, k.transpose(1, 2).contiguous()) * sc
        P = torch.softmax(S.masked_fill(~mask, float("-inf")), -1).contiguous()
        ctx = torch.matmul(P, v).permute(1, 0, 2).reshape(Tb, Cb).contiguous()
        saved = {"ln_y": ln_y, "ln_sig": sig, "w_qkv": wqkv, "qkv": qkv, "P": P, "ctx": ctx, "w_o": wo}
        dx, dwq, dwo = torch.empty_like(dx2), torch.empty_like(wqkv), torch.empty_like(wo)
        bws = torch.empty(vtb.attn_block_bwd_workspace_size(vtb.make_block_cfg(1, Tb, Hb, db, sc)), dtype=torch.uint8,
                          device=dev)
        f = lambda: vtb.attn_block_bwd(saved, dx2, 1, Hb, sc, True, dx=dx, dw_qkv=dwq, dw_o=dwo, workspace=bws,
                                       stream=torch.cuda.current_stream())
        ms = graph_ms(torch, hip, f, 10)
        pairs = Hb * Tb * (Tb + 1) // 2
        fl = 4 * Tb * Cb * Cb + 4 * Tb * Cb * 3 * Cb + 8 * db * pairs   # Wo, Wqkv products; 4 attention contractions
        out["attn_block_bwd"] = {"workload": "attention block backward (LayerNorm, QKV/output projections, saved-softmax "
                                             "causal attention), T256 20 x 128 fp32",
                                 "ms": round(ms, 4), "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                                 "roofline": {"bound": "mfma", "peak": FP32_MFMA_PEAK_TFLOPS,
                                              "frac": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                                              "algorithmic_flops": fl}}
        del saved, xin, wqkv, wo, dx2, ln_y, qkv, P, ctx, dx, dwq, dwo, bws

    if want("rms_attn_block_bwd"):
        # one Hesper-form attention layer's backward (RMSNorm with gain, QKV projection, RoPE
        # on q and k, causal attention with the saved softmax, output projection), T256
        # 20 x 128 fp32; saved activations from a torch fp32 forward (setup only)
        Tb, Hb, db = 256, 20, 128
        Cb = Hb * db
        sc = 1.0 / np.sqrt(db)
        p = synth.rms_block_inputs(1, Tb, Hb, db)
        x, gam, wqkv, wo, dx2 = (up(p[n]) for n in ("x", "gamma", "w_qkv", "w_o", "dx2"))
        n_ = (gam * x / torch.sqrt((x * x).mean(1, keepdim=True) + 1e-6)).contiguous()
        abv = n_ @ wqkv
        th = torch.arange(Tb, device=dev, dtype=torch.float64)[:, None] * \
            10000.0 ** (-2.0 * torch.arange(db // 2, device=dev, dtype=torch.float64)[None, :] / db)
        cs, sn = torch.cos(th).float()[:, None, :], torch.sin(th).float()[:, None, :]

        def rot(z):
            z = z.reshape(Tb, Hb, db // 2, 2)
            return torch.stack([z[..., 0] * cs - z[..., 1] * sn, z[..., 0] * sn + z[..., 1] * cs], -1).reshape(Tb, Cb)

        qkv = torch.cat([rot(abv[:, :Cb]), rot(abv[:, Cb:2 * Cb]), abv[:, 2 * Cb:]], 1).contiguous()
        hsplit = lambda z: z.reshape(Tb, Hb, db).permute(1, 0, 2).contiguous()
        q, k, v = hsplit(qkv[:, :Cb]), hsplit(qkv[:, Cb:2 * Cb]), hsplit(qkv[:, 2 * Cb:])
        mask = torch.tril(torch.ones(Tb, Tb, dtype=torch.bool, device=dev))
        P = torch.softmax((torch.matmul(q, k.transpose(1, 2).contiguous()) * sc).masked_fill(~mask, float("-inf")),
                          -1).contiguous()
        ctx = torch.matmul(P, v).permute(1, 0, 2).reshape(Tb, Cb).contiguous()
        saved = {"x": x, "gamma": gam, "n": n_, "w_qkv": wqkv, "qkv": qkv, "P": P, "ctx": ctx, "w_o": wo}
        outs = dict(dx=torch.empty_like(dx2), dgamma=torch.empty_like(gam), dw_qkv=torch.empty_like(wqkv),
                    dw_o=torch.empty_like(wo))
        rws = torch.empty(vtb.rms_attn_block_bwd_workspace_size(vtb.make_rms_block_cfg(1, Tb, Hb, db, sc)),
                          dtype=torch.uint8, device=dev)
        f = lambda: vtb.rms_attn_block_bwd(saved, dx2, 1, Hb, sc, True, workspace=rws, stream=torch.cuda.current_stream(),
                                           **outs)
        ms = graph_ms(torch, hip, f, 10)
        pairs = Hb * Tb * (Tb + 1) // 2
        fl = 4 * Tb * Cb * Cb + 4 * Tb * Cb * 3 * Cb + 8 * db * pairs   # Wo, Wqkv products; 4 attention contractions
        out["rms_attn_block_bwd"] = {"workload": "Hesper-form attention layer backward (RMSNorm with gain, QKV "
                                                 "projection, RoPE on q and k, saved-softmax causal attention, output "
                                                 "projection), T256 20 x 128 fp32",
                                     "ms": round(ms, 4), "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                                     "roofline": {"bound": "mfma", "peak": FP32_MFMA_PEAK_TFLOPS,
                                                  "frac": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                                                  "algorithmic_flops": fl}}
        del saved, outs, rws, x, gam, wqkv, wo, dx2, n_, abv, qkv, P, ctx

    if want("layer_chain"):
        # 30-layer chain: T256, hidden 2560 = 20 x 128, fp32, saved softmax P per layer
        L, T = 30, 256
        sc = 1.0 / np.sqrt(d)
        pos = torch.arange(T, device=dev, dtype=torch.float64)
        inv = 10000.0 ** (-2.0 * torch.arange(d // 2, device=dev, dtype=torch.float64) / d)
        ang = pos[:, None] * inv[None, :]
        cos, sin = torch.cos(ang).float()[:, None, :], torch.sin(ang).float()[:, None, :]
        mask = torch.tril(torch.ones(T, T, dtype=torch.bool, device=dev))
        saved = []
        for l in range(L):
            li = synth.layer_inputs(l, T, H, d)
            h, K, V, W, gm = (up(li[n]) for n in ("h", "K", "V", "W", "gamma"))
            xn = h * torch.rsqrt((h * h).mean(1, keepdim=True) + 1e-6) * gm
            xr = xn.view(T, H, d)
            a, b2 = xr[..., 0::2], xr[..., 1::2]
            q = torch.stack((a * cos - b2 * sin, a * sin + b2 * cos), -1).reshape(T, H, d).contiguous()
            S = torch.matmul(q.permute(1, 0, 2).contiguous(), K.permute(1, 2, 0).contiguous()) * sc
            P = torch.softmax(S.masked_fill(~mask, float("-inf")), -1).contiguous()
            ob = torch.matmul(P, V.permute(1, 0, 2).contiguous()).permute(1, 0, 2).reshape(T, C).contiguous()
            saved.append({"x": h, "gamma": gm, "w": W, "o": ob, "q": q, "k": K.contiguous(), "v": V.contiguous(), "P": P})
        g0 = up(synth.layer_upstream_grad(T, H, d))
        gs = [torch.empty_like(g0) for _ in range(L)]
        dws = [torch.empty_like(saved[0]["w"]) for _ in range(L)]
        dks = [torch.empty_like(saved[0]["k"]) for _ in range(L)]
        dvs = [torch.empty_like(saved[0]["v"]) for _ in range(L)]
        cfg = vtb.make_layer_cfg(T, H, d, sc)
        lws = torch.empty(vtb.layer_bwd_workspace_size(cfg), dtype=torch.uint8, device=dev)

        def chain():
            g = g0
            for l in reversed(range(L)):
                vtb.layer_bwd(saved[l], g, sc, dh_in=gs[l], dw=dws[l], dk=dks[l], dv=dvs[l], workspace=lws,
                              stream=torch.cuda.current_stream())
                g = gs[l]

        ms = graph_ms(torch, hip, chain, 3)
        pairs = H * T * (T + 1) // 2
        fl = L * (4 * T * C * C + 8 * d * pairs)
        out["layer_chain"] = {"workload": "30-layer backward chain, T256 hidden 2560 (20 x 128) fp32, saved P",
                              "ms": round(ms, 4), "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                              "roofline": {"bound": "mfma", "peak": FP32_MFMA_PEAK_TFLOPS,
                                           "frac": round(fl / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                                           "algorithmic_flops": fl}}
    return out


def mfma_probe_rates(torch, hip):
    """Sustained bf16 matrix-core rate on this GPU (libvtb_probe.so: independent MFMA
    accumulations, operands in registers, no memory traffic), with the shader clock the
    chip ran at meanwhile. Context beside the published peak, never a roofline denominator."""
    import numpy as np

    path = os.path.join(ROOT, "verified_transformer_backward_amd", "libvtb_probe.so")
    L = ctypes.CDLL(path)
    L.vtb_probe_mfma_bf16.restype = ctypes.c_int
    L.vtb_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    blocks, iters = 256 * 2, 4096                        # two workgroups of 4 waves per CU: 2 waves per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    clk = torch.empty(blocks * 8, dtype=torch.int64, device="cuda:0")
    sptr = torch.cuda.current_stream().cuda_stream
    out = {}
    for shape, name, flop in ((0, "32x32x16", 32 * 32 * 16 * 2), (1, "16x16x32", 16 * 16 * 32 * 2)):
        args = (shape, iters, blocks, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                ctypes.c_void_p(sptr))
        if L.vtb_probe_mfma_bf16(*args) != 0:
            raise RuntimeError("mfma probe launch failed")
        torch.cuda.synchronize()
        start, stop = hip.create(2)
        hip.record(start, sptr)
        if L.vtb_probe_mfma_bf16(*args) != 0:
            raise RuntimeError("mfma probe launch failed")
        hip.record(stop, sptr)
        torch.cuda.synchronize()
        ms = hip.ms(start, stop)
        hip.destroy([start, stop])
        c = clk.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.mean(c[:, 0]) / (np.mean(c[:, 1]) * 10.0))     # 100 MHz wall-clock ticks
        total = 4.0 * iters * flop * blocks * 4
        tf = total / (ms * 1e-3) / 1e12
        out[f"bf16_{name}"] = {"tflops": round(tf, 1), "clock_ghz": round(ghz, 3),
                               "frac_of_spec": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                               "per_clock_frac": round(tf * 1e12 / (256 * 4096 * ghz * 1e9), 4)}
    del sink, clk
    return out


def oracle_per_config():
    """The float64 oracle timed on each workload on this host, with every core BLAS uses and
    (for the three smaller workloads) with one thread: a baseline only. Workloads too large to
    run whole here are sampled and scaled to the full work (the sample is stated)."""
    import numpy as np
    import synth
    from oracle import attention as A
    from oracle import layer as Lr
    from oracle import specs

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:                                   # no thread control: all-cores figures only
        threadpool_info = threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    if threadpool_info is not None:
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])

    def clock(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def pairs(B, H, Tq, Tk, causal):
        return B * H * (Tq * (Tq + 1) // 2 + Tq * (Tk - Tq) if causal else Tq * Tk)

    x1 = synth.tiny_inputs()

    def c1():
        A.attention_backward(x1["q"], x1["k"], x1["v"], x1["dout"], x1["scale"], False)
        Lr.rope_backward_rows(x1["rope_dy"], np.array([x1["rope_pos"]]), x1["rope_base"])
        specs.rmsnorm_backward(x1["rms_x"][0], x1["rms_gamma"], x1["rms_dy"][0], x1["rms_eps"])

    x2 = synth.decode_gqa_inputs()
    c2 = lambda: A.attention_backward(x2["q"], x2["k"], x2["v"], x2["dout"], x2["scale"], False)
    x3 = synth.causal_inputs()
    l3 = A.attention_lse(x3["q"], x3["k"], x3["scale"], True)
    x4 = [Lr.layer_saved(**{k: v for k, v in synth.layer_inputs(l).items() if k != "W"}, W=synth.layer_inputs(l)["W"],
                         H=20, scale=1.0 / np.sqrt(128.0)) for l in range(2)]
    g4 = synth.layer_upstream_grad()
    x5 = synth.long_causal_inputs()
    h5 = [0, 1, 2, 3]
    one5 = {n: x5[n][:, :, h5] for n in ("q", "k", "v", "dout")}
    l5 = A.attention_lse(one5["q"], one5["k"], x5["scale"], True)

    def c3(heads):
        sub = {n: x3[n][:, :, :heads] for n in ("q", "k", "v", "dout")}
        return lambda: A.attention_backward(sub["q"], sub["k"], sub["v"], sub["dout"], x3["scale"], True,
                                            lse=l3[:, :heads])

    work = {
        "tiny_single_query": (10 * 64 * 16, c1, 1.0, "whole workload"),
        "decode_gqa": (10 * 128 * pairs(8, 20, 1, 1024, False), c2, 1.0, "whole workload"),
        "causal_train": (10 * 128 * pairs(4, 20, 512, 512, True), c3(20), 20 / 20, "whole workload (B4, all 20 heads)"),
        "layer_chain": (30 * (4 * 256 * 2560 * 2560 + 8 * 128 * pairs(1, 20, 256, 256, True)),
                        lambda: Lr.stack_backward(x4, g4, 20, 1.0 / np.sqrt(128.0)), 30 / 2,
                        "2 of the 30 layers, scaled by 15"),
        "long_causal": (10 * 128 * pairs(1, 32, 8192, 8192, True),
                        lambda: A.attention_backward(one5["q"], one5["k"], one5["v"], one5["dout"], x5["scale"], True,
                                                     lse=l5), 32 / len(h5), f"{len(h5)} of the 32 heads, scaled by 8"),
    }
    out = {"cores": int(cores), "kind": "oracle", "note": "float64 numpy oracle on the host; a baseline only"}
    for name, (flops, fn, scale_up, sample) in work.items():
        s = clock(fn) * scale_up
        rec = {"seconds": round(s, 4), "gflops": round(flops / s / 1e9, 3), "sample": sample}
        if name in ("tiny_single_query", "decode_gqa", "causal_train") and threadpool_limits is not None:
            fn1, sc1, samp1 = (c3(4), 20 / 4, "4 of the 20 heads, scaled by 5") if name == "causal_train" else (fn, 1.0, sample)
            with threadpool_limits(limits=1, user_api="blas"):
                s1 = clock(fn1) * sc1
            rec["one_thread"] = {"seconds": round(s1, 4), "gflops": round(flops / s1 / 1e9, 3), "sample": samp1}
        out[name] = rec
    return out


def cpu_baseline(x, seconds):
    """The float64 oracle on the same workload, on this host's cores (a baseline only).
    Each sampled head's lse comes from the oracle's own forward statistic, outside the timing."""
    import numpy as np
    from oracle import attention as A

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    B, T, H, d = x["q"].shape
    # bounded sample: whole (b, h) heads of the same workload, cycling, until ~`seconds` of work
    heads = [(b, h) for b in range(B) for h in range(H)]
    dt, done = 0.0, 0
    while dt < seconds and done < 200 * len(heads):
        b, h = heads[done % len(heads)]
        one = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "dout")}
        lse = A.attention_lse(one["q"], one["k"], x["scale"], True)
        t0 = time.perf_counter()
        A.attention_backward(one["q"], one["k"], one["v"], one["dout"], x["scale"], True, lse=lse)
        dt += time.perf_counter() - t0
        done += 1
    flops = 10 * d * done * T * (T + 1) // 2
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle", "cpu_model": cpu,
            "sample": f"{done} single-head backwards cycling over the {len(heads)} (b,h) heads of "
                      f"B{B} H{H} T{T} d{d}, float64 numpy, {dt:.1f} s timed"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}). Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import verified_transformer_backward_amd as vtb

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.only:                                         # one or more of the other workloads alone (profiling)
        names = [n for n in args.only.split(",") if n]
        bad = [n for n in names if n not in EXTRA_NAMES]
        if bad:
            print(f"bench.py: unknown workload(s) {bad}; choose from {list(EXTRA_NAMES)}", file=sys.stderr)
            return 2
        torch.cuda.init()
        if args.calibrate_copy:   # same known-size copy as the headline run
            src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda:0")
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
            del src
        print(json.dumps({"only": names, "other_workloads": extra_workloads(torch, vtb, HipEvents(), set(names))}))
        return 0
    B, T, H, d = 4, 512, 20, 128
    x = synth.causal_inputs(B, T, H, d)
    sc = float(x["scale"])
    flops, compulsory, per_kernel = workload_numbers(B, T, H, d)

    dev = torch.device("cuda:0")
    base = {n: torch.from_numpy(synth.bf16_bits(x[n])).view(torch.bfloat16).to(dev) for n in ("q", "k", "v", "dout")}
    nsets = max(1, args.sets)
    sets = []
    for s in range(nsets):
        t = {n: v.clone() for n, v in base.items()}
        t["lse"] = vtb.attn_fwd_lse(t["q"], t["k"], sc, True)
        t["dq"] = torch.empty_like(t["q"])
        t["dk"] = torch.empty_like(t["k"])
        t["dv"] = torch.empty_like(t["v"])
        desc = vtb.make_attn_desc(t["q"], t["k"], sc, True, torch.bfloat16, t["dout"], t["dq"], t["dk"], t["dv"], t["v"])
        t["ws"] = torch.empty(vtb.attn_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
        sets.append(t)
    torch.cuda.synchronize()

    if args.calibrate_copy:   # known-size reference for FETCH_SIZE / WRITE_SIZE: 256 MiB read + 256 MiB written
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    hip = HipEvents()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(t, events=None):
        vtb.attn_bwd(t["q"], t["k"], t["v"], t["dout"], sc, True, lse=t["lse"], dq=t["dq"], dk=t["dk"], dv=t["dv"],
                     workspace=t["ws"], stream=torch.cuda.current_stream(), events=events)

    def capture(setlist):
        """One HIP graph holding one step per entry of setlist, captured on a side stream."""
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step(setlist[0])
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            for t in setlist:
                step(t)
        torch.cuda.synchronize()
        return g

    def graph_timed(nsteps, rot):
        """ms per step of nsteps steps (rotating over `rot` sets) replayed from one graph."""
        g = capture([sets[i % rot] for i in range(nsteps)])
        g.replay()                                        # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        ref = {n: sets[0][n].clone() for n in ("dq", "dk", "dv")}
        step(sets[0])                                     # eager call on the same inputs
        torch.cuda.synchronize()
        same = all(torch.equal(ref[n], sets[0][n]) for n in ref)
        start, stop = hip.create(2)
        hip.record(start, sptr)
        g.replay()
        hip.record(stop, sptr)
        torch.cuda.synchronize()
        total = hip.ms(start, stop)
        hip.destroy([start, stop])
        return total / nsteps, same

    def timed(nsteps, rot):
        phase = hip.create(4 * nsteps)
        start, stop = hip.create(2)
        torch.cuda.synchronize()
        hip.record(start, sptr)
        for i in range(nsteps):
            step(sets[i % rot], phase[4 * i:4 * i + 4])
        hip.record(stop, sptr)
        torch.cuda.synchronize()
        total = hip.ms(start, stop)
        per = {k: [] for k in ("dq", "dkdv")}
        for i in range(nsteps):
            e = phase[4 * i:4 * i + 4]
            per["dq"].append(hip.ms(e[0], e[1]))             # start/end of each kernel's dispatch
            per["dkdv"].append(hip.ms(e[2], e[3]))
        hip.destroy(phase + [start, stop])
        spread = {k: [round(1e3 * float(np.percentile(v, q)), 2) for q in (10, 50, 90)] for k, v in per.items()}
        return total / nsteps, {k: 1e3 * float(np.mean(v)) for k, v in per.items()}, spread

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    eager_ms, kern_us, kern_spread = timed(args.steps, nsets)   # per-pass times from eager steps
    warm_eager_ms, warm_us, _ = timed(max(10, args.steps // 2), 1)
    ms_step, same = graph_timed(args.steps, nsets)
    warm_ms, same_w = graph_timed(max(10, args.steps // 2), 1)
    if not (same and same_w):                             # graph replay must match eager calls
        print("bench.py: graph replay differs from eager calls; reporting eager timing", file=sys.stderr)
        ms_step, warm_ms = eager_ms, warm_eager_ms

    tflops = flops / (ms_step * 1e-3) / 1e12
    dom = max(kern_us, key=kern_us.get)                   # dominant kernel of the step
    dom_s = kern_us[dom] * 1e-6
    achieved = per_kernel[dom]["bytes"] / dom_s / 1e9
    traffic = traffic_from_profile(dom)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal attention backward B4 H20 T512 d128, bf16 in/out, fp32 accumulation, "
                               "lse given, scale 1/sqrt(128)",
                   "B": B, "H": H, "T": T, "d": d,
                   "cache": f"cold: {nsets} rotating input/output sets" if nsets > 1 else "warm"},
        "hbm_gbps": round(compulsory / (ms_step * 1e-3) / 1e9, 1),
        "frac_bf16_mfma_peak": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        # the whole step against its own roofline: min(MFMA peak, arithmetic intensity x HBM)
        "step_roofline": {"achieved_tflops": round(tflops, 1),
                          "intensity_flop_per_byte": round(flops / compulsory, 1),
                          "ceiling_tflops": round(min(BF16_MFMA_PEAK_TFLOPS, flops / compulsory * HBM_PEAK_GBS / 1e3), 1),
                          "frac": round(tflops / min(BF16_MFMA_PEAK_TFLOPS, flops / compulsory * HBM_PEAK_GBS / 1e3), 4),
                          "compulsory_bytes": compulsory, "algorithmic_flops": flops},
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "kernel_us_p10_p50_p90": kern_spread,
        "timing": "hip graph replay" if (same and same_w) else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "warm": {"ms_per_step": round(warm_ms, 5), "value": round(flops / (warm_ms * 1e-3) / 1e12, 2),
                 "kernel_us": {k: round(v, 2) for k, v in warm_us.items()}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"{dom}_mfma_kernel (bf16, d128)",
                     "algorithmic_bytes": per_kernel[dom]["bytes"],
                     "algorithmic_flops": per_kernel[dom]["flops"],
                     "mfma_tflops": round(per_kernel[dom]["flops"] / dom_s / 1e12, 1),
                     "mfma_frac": round(per_kernel[dom]["flops"] / dom_s / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
    }
    if not args.no_extra:
        out["other_workloads"] = extra_workloads(torch, vtb, hip)
        out["measured_hbm_copy"] = copy_bandwidth(torch, hip)
        out["measured_library_gemm"] = library_gemm_rates(torch, hip)
        out["measured_mfma_probe"] = mfma_probe_rates(torch, hip)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
        out["oracle_per_config"] = oracle_per_config()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
