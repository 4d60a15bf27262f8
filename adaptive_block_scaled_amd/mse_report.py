"""Per-config quantization-error report: IF4 against its two fixed encodings.

IF4 keeps, per group of 16, whichever of FP4 (E2M1) and 6/7-descaled INT4
gives the smaller squared error ("Adaptive Block-Scaled Data Types",
gist.science summary, section 2, selection mechanism).  Forcing the flag gives
the two fixed formats the pages compare against: FP4 with E4M3 per-16 scales
(NVFP4's algorithm) and the INT4 comparator.  This module quantizes each
workload tensor in the three modes with libif4 on the GPU, dequantizes with
libif4, and reports the mean squared error in original units, the share of
groups that chose INT4, and how many groups ended with a larger error than
the better fixed format (possible only where the fp32 selection and exact
arithmetic disagree on a near-tie).

Run: `python -m adaptive_block_scaled_amd.mse_report [--configs c1,c2,...]
[--bits 4,3,6]` (IF3 and IF6 against their own fixed float and INT formats).
The error arithmetic here (fp64 torch ops) is measurement, not part of the
quantization path.
"""
import argparse
import json
import sys

import numpy as np
import torch

from . import if4
from . import workloads as wl

MODES = {"if4": if4.MODE_ADAPTIVE, "fp4": if4.MODE_FORCE_FP4, "int4": if4.MODE_FORCE_INT4}


def group_sse(x: torch.Tensor, codes, scales, scale_exp: int) -> torch.Tensor:
    """Per-group sum of squared errors (fp64) of the libif4 round trip."""
    y = if4.dequantize(codes, scales, scale_exp, torch.float32)
    d = (x.to(torch.float64) - y.to(torch.float64))
    return (d * d).reshape(x.shape[0], -1, if4.GROUP).sum(dim=2)


def report_tensor(t: wl.Tensor, scale_exp=None, rtol: float = 1e-5) -> dict:
    dev = torch.device("cuda:0")
    e = t.scale_exp if scale_exp is None else scale_exp
    xd = torch.from_numpy(t.values).to(dev)
    x = xd.to(torch.bfloat16) if t.dtype == "bf16" else xd
    sse, flags = {}, None
    for name, mode in MODES.items():
        codes, scales = if4.quantize(x, e, mode=mode)
        sse[name] = group_sse(xd, codes, scales, e)
        if name == "if4":
            flags = (scales >= 0x80)
    best_fixed = torch.minimum(sse["fp4"], sse["int4"])
    worse = int((sse["if4"] > best_fixed * (1 + rtol) + 1e-300).sum().item())
    n = x.numel()
    return {
        "tensor": t.name, "scale_exp": int(e), "groups": int(flags.numel()),
        "mse_if4": float(sse["if4"].sum().item() / n),
        "mse_fp4": float(sse["fp4"].sum().item() / n),
        "mse_int4": float(sse["int4"].sum().item() / n),
        "int4_share": float(flags.double().mean().item()),
        "groups_if4_above_best_fixed": worse,
    }


def report_tensor_ifn(t: wl.Tensor, bits: int, rtol: float = 1e-5) -> dict:
    """As report_tensor for IF3 / IF6 (bits 3 or 6) against their fixed float
    and INT formats; the exponent follows the same rule with the format's top
    value (4 or 7.5) in place of 6."""
    dev = torch.device("cuda:0")
    top = 7.5 if bits == 6 else 4.0
    amax = float(np.max(np.abs(t.values))) if t.values.size else 0.0
    e = wl.tensor_scale_exp(amax * 6.0 / top)
    xd = torch.from_numpy(t.values).to(dev)
    x = xd.to(torch.bfloat16) if t.dtype == "bf16" else xd
    sse, flags = {}, None
    for name, mode in MODES.items():
        codes, scales = if4.quantize_ifn(x, bits, e, mode=mode)
        y = if4.dequantize_ifn(codes, scales, bits, e, torch.float32)
        d = xd.to(torch.float64) - y.to(torch.float64)
        sse[name] = (d * d).reshape(x.shape[0], -1, if4.GROUP).sum(dim=2)
        if name == "if4":
            flags = (scales >= 0x80)
    best_fixed = torch.minimum(sse["fp4"], sse["int4"])
    n = x.numel()
    return {
        "tensor": t.name, "format": f"IF{bits}", "scale_exp": int(e),
        "mse_if": float(sse["if4"].sum().item() / n),
        "mse_fp": float(sse["fp4"].sum().item() / n),
        "mse_int": float(sse["int4"].sum().item() / n),
        "int_share": float(flags.double().mean().item()),
        "groups_if_above_best_fixed": int((sse["if4"] > best_fixed * (1 + rtol) + 1e-300).sum().item()),
    }


def config_tensors(name: str):
    if name == "c1":
        t = wl.c1_mixed_fp32()
        return [(t, 0), (t, None)]
    if name == "c2":
        return [(wl.c2_activations(), None)]
    if name == "c3":
        t = wl.c3_rht_gradient()
        return [(t, None), (t, 0)]
    if name == "c4":
        a, w = wl.c4_gemm()
        return [(a, None), (w, None)]
    if name == "c5":
        a, w = wl.c5_ffn()
        return [(a, None), (w, None)]
    raise ValueError(name)


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--configs", default="c1,c2,c3,c4,c5")
    p.add_argument("--json", action="store_true", help="one JSON line per tensor")
    p.add_argument("--bits", default="4", help="comma list of widths: 4 (IF4), 3 (IF3), 6 (IF6)")
    args = p.parse_args(argv)
    widths = [int(b) for b in args.bits.split(",")]
    if any(b != 4 for b in widths):
        rows, seen = [], set()
        for c in args.configs.split(","):
            for t, _ in config_tensors(c.strip()):
                if t.name in seen:  # listed twice for IF4's two exponents
                    continue
                seen.add(t.name)
                for b in widths:
                    if b == 4:
                        continue
                    r = report_tensor_ifn(t, b)
                    rows.append(r)
                    if args.json:
                        print(json.dumps(r), flush=True)
        if not args.json:
            print(f"{'tensor':34s} {'fmt':>4s} {'E':>4s} {'MSE IF':>11s} {'MSE FP':>11s} "
                  f"{'MSE INT':>11s} {'IF/FP':>7s} {'IF/INT':>7s} {'INT grp':>7s} {'worse':>5s}")
            for r in rows:
                print(f"{r['tensor']:34s} {r['format']:>4s} {r['scale_exp']:4d} {r['mse_if']:11.4e} "
                      f"{r['mse_fp']:11.4e} {r['mse_int']:11.4e} "
                      f"{r['mse_if'] / r['mse_fp'] if r['mse_fp'] else float('nan'):7.4f} "
                      f"{r['mse_if'] / r['mse_int'] if r['mse_int'] else float('nan'):7.4f} "
                      f"{r['int_share']:7.3f} {r['groups_if_above_best_fixed']:5d}")
        if 4 not in widths:
            return rows
    rows = []
    for c in args.configs.split(","):
        for t, e in config_tensors(c.strip()):
            r = report_tensor(t, e)
            rows.append(r)
            if args.json:
                print(json.dumps(r), flush=True)
    if not args.json:
        hdr = (f"{'tensor':34s} {'E':>4s} {'MSE IF4':>11s} {'MSE FP4':>11s} {'MSE INT4':>11s} "
               f"{'IF4/FP4':>8s} {'IF4/INT4':>8s} {'INT4 grp':>8s} {'worse':>5s}")
        print(hdr)
        for r in rows:
            def ratio(a, b):
                return a / b if b > 0 else float("nan")
            print(f"{r['tensor']:34s} {r['scale_exp']:4d} {r['mse_if4']:11.4e} {r['mse_fp4']:11.4e} "
                  f"{r['mse_int4']:11.4e} {ratio(r['mse_if4'], r['mse_fp4']):8.4f} "
                  f"{ratio(r['mse_if4'], r['mse_int4']):8.4f} {r['int4_share']:8.3f} "
                  f"{r['groups_if4_above_best_fixed']:5d}")
    return rows


if __name__ == "__main__":
    sys.exit(0 if main() else 1)
