#!/usr/bin/env python3
"""Benchmark of the delta-rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one dr_chunk_fwd over the headline batch: Gated DeltaNet gating
(scalar log alpha ~ U(-0.1, -0.001), scalar beta = sigmoid(N(0,1)), q and k
L2-normalised, bf16 q/k/v, fp32 S0 ~ N(0, 0.01), fp32 output), B=2, H=16,
L=16384, d_k=d_v=128.  `value` is tokens/s of that step (B*L per step).
The same run also times the recurrent decode: 512 consecutive dr_decode_step
calls on 256 sequences x 16 heads of 128x128 fp32 states with bf16 tokens,
reported as HBM GB/s under "decode".  Inputs are synthetic, seeded, and
resident in device memory before any timed region.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix peak, TFLOP/s
# algorithmic work per token-head of the chunked forward at d = 128, chunk 64:
# 2 * (5 C d + 3 d^2) flops; bytes = q, k, v bf16 (768) + o fp32 (512) + log alpha
# and beta fp32 (8) + S0 and S_final amortised over L (2 * 64 KiB / L)
FLOPS_PER_TOKEN_HEAD = 2 * (5 * 64 * 128 + 3 * 128 * 128)
DECODE_BYTES_PER_STATE = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 4 + 4 + 128 * 4


def chunk_bytes_per_token_head(L: int) -> float:
    return 3 * 128 * 2 + 128 * 4 + 4 + 4 + 2 * 128 * 128 * 4 / L


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see DESIGN.md for how it would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import delta_rule_linear_amd as drl
    from delta_rule_linear_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    drl.lib()

    def to_dev(a, bf16=False):
        if a is None:
            return None
        if bf16:
            return torch.from_numpy(inputs.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    # ------------------------------------------------------------ chunked forward
    name = "gdn_b2h16_16k"
    p = inputs.workload(name)
    B, H, L, D = p.B, p.H, p.L, p.Dk
    q, k, v = to_dev(p.q, True), to_dev(p.k, True), to_dev(p.v, True)
    la, be, S0 = to_dev(p.log_alpha), to_dev(p.beta), to_dev(p.S0)
    o = torch.empty((B, H, L, D), dtype=torch.float32, device=dev)
    Sf = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    desc = drl.chunk_desc(B, H, L, D, D, drl.DR_BF16, drl.DR_F32, "scalar", "scalar")
    ws = torch.empty(drl.dr_chunk_fwd_workspace_bytes(desc), dtype=torch.uint8, device=dev)

    def step():
        drl.dr_chunk_fwd(q, k, v, la, be, S0, gate="scalar", beta_mode="scalar", o=o, S_final=Sf,
                         workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]   # ms per call
    ms = float(np.mean(per))
    tok_s = B * L / (ms * 1e-3)
    token_heads = B * H * L
    alg_bytes = chunk_bytes_per_token_head(L) * token_heads
    alg_flops = FLOPS_PER_TOKEN_HEAD * token_heads
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12

    # ------------------------------------------------------------ decode
    dec = None
    if args.decode_steps > 0:
        dp = inputs.make_decode_problem(256, 16, 128, 128, args.decode_steps)
        S = to_dev(dp.S)
        dq, dk, dv_ = to_dev(dp.q, True), to_dev(dp.k, True), to_dev(dp.v, True)
        dla, dbe = to_dev(dp.log_alpha), to_dev(dp.beta)
        do = torch.empty((dp.steps, 256, 16, 128), dtype=torch.float32, device=dev)
        ddesc = drl.DecodeDesc(256, 16, 128, 128, drl.DR_BF16, drl.DR_F32, drl.GATES["scalar"],
                               drl.BETAS["scalar"])
        lib = drl.lib()
        import ctypes

        def dstep(t):
            rc = lib.dr_decode_step(ctypes.byref(ddesc), dq[t].data_ptr(), dk[t].data_ptr(),
                                    dv_[t].data_ptr(), dla[t].data_ptr(), dbe[t].data_ptr(),
                                    S.data_ptr(), do[t].data_ptr(), stream.cuda_stream)
            if rc:
                raise drl.DeltaRuleError(rc, drl.dr_last_error())

        Swarm = S.clone()
        for t in range(min(3, dp.steps)):     # warm-up on a scratch copy of the states
            rc = lib.dr_decode_step(ctypes.byref(ddesc), dq[t].data_ptr(), dk[t].data_ptr(),
                                    dv_[t].data_ptr(), dla[t].data_ptr(), dbe[t].data_ptr(),
                                    Swarm.data_ptr(), do[t].data_ptr(), stream.cuda_stream)
        del Swarm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(dp.steps):
            dstep(t)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / dp.steps
        dbytes = DECODE_BYTES_PER_STATE * 256 * 16
        dgbs = dbytes / (dms * 1e-3) / 1e9
        dec = {"workload": "256 sequences x 16 heads, 128x128 fp32 states, bf16 tokens, GDN gating",
               "steps": dp.steps, "us_per_step": round(dms * 1e3, 2),
               "tokens_per_s": round(256 / (dms * 1e-3), 1),
               "GB_per_s": round(dgbs, 1), "hbm_frac": round(dgbs / HBM_PEAK_GBS, 4),
               "alg_bytes_per_step": dbytes}

    # ------------------------------------------------------------ CPU baseline (oracle)
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        nthr = len(os.sched_getaffinity(0))
        heads = [(0, h) for h in range(min(H, max(1, nthr)))]
        sub = p.head(0, 0)
        sl = slice(heads[0][1], heads[-1][1] + 1)
        sub.H = len(heads)
        for fld in ("q", "k", "v", "log_alpha", "beta", "S0"):
            setattr(sub, fld, getattr(p, fld)[0:1, sl])
        tc = time.perf_counter()
        oy, Sy = oracle.forward_problem(sub, nthreads=nthr)
        tcpu = time.perf_counter() - tc
        th = len(heads) * L
        cpu = {"value": round(th / tcpu / H, 1), "unit": "tokens/s", "cores": nthr, "kind": "oracle",
               "sample": f"heads (b=0, h={heads[0][1]}..{heads[-1][1]}) of the B=2 H=16 L=16384 "
                         f"workload at full length, fp64, {tcpu:.1f} s; tokens/s = token-heads/s / H"}
        og = o[0, sl].double().cpu().numpy()
        Sg = Sf[0, sl].double().cpu().numpy()
        parity = {"heads": len(heads), "o_max_rel_err": float(np.abs(og - oy[0]).max() / np.abs(oy[0]).max()),
                  "S_max_rel_err": float(np.abs(Sg - Sy[0]).max() / np.abs(Sy[0]).max()), "tol": 3e-3}

    out = {
        "metric": "tokens/s + % bf16 MFMA peak, chunked GDN fwd H=16 d=128 L=16K; decode GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp16 MFMA operands, fp32 accumulate/state",
        "data": "synthetic (seeded)",
        "config": {"workload": "chunked GDN forward, B=2 H=16 L=16384 d_k=d_v=128, scalar gate, "
                               "scalar beta, bf16 q/k/v, fp32 S0 and o",
                   "global_batch": B, "seq_len": L, "heads": H, "d": D, "chunk": 64,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "dr_chunk_fwd (prep_kernel + scan_kernel)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "alg_bytes_per_launch": int(alg_bytes)},
        "mfma": {"achieved_tflops": round(tflops, 1), "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "alg_flops_per_launch": int(alg_flops)},
        "decode": dec,
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
