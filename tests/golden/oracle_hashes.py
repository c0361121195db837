"""Record / check SHA-256 hashes of the oracle's results on the workload shapes.

    python tests/golden/oracle_hashes.py --record   # writes oracle_hashes.json
    python tests/golden/oracle_hashes.py --check    # recomputes and compares

This is the golden-baseline idea of the Metal fusion page ("llama.cpp b10909：
Metal后端融合表重构...", section "融合统计与回归测试": record a baseline once,
check later runs against it) applied to the oracle: any change to what the
oracle computes on these inputs -- a code, a scale, a block sum or an fp32
output bit -- changes a hash.  Only ``oracle/`` and the seeded input
generators run here.  The GPU tests hash the library's codes, scales and
block sums of the same inputs and compare them with these records (the fp32
outputs are compared within tolerance there, so their hashes serve the
oracle's own regression check only).

Inputs come from ``inputs(name)``: host draws of ``workloads`` with seed 11,
at the shapes of the workloads they are named after.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HASH_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_hashes.json")
SEED = 11
EPS = wl.RMS_EPS

CONFIGS = (
    "tiny_gemv_256x512",
    "llama1b_decode_layer0_b1",
    "llama8b_decode_layer0_b8",
    "llama8b_prefill_kproj_t512",
    "moe_64x16_top8_down",
)


def digest(a: np.ndarray) -> str:
    """'dtype[shape] sha256-of-the-row-major-bytes'."""
    a = np.ascontiguousarray(a)
    shape = ",".join(str(n) for n in a.shape)
    return f"{a.dtype}[{shape}] {hashlib.sha256(a.tobytes()).hexdigest()}"


def inputs(name: str) -> dict:
    """Seeded host inputs of a configuration (no arithmetic of the method)."""
    if name == "tiny_gemv_256x512":
        return {"w": [wl.weight(SEED, 0, 0, 256, 512)], "x": {0: wl.activation(SEED, 0, 0, 1, 512)},
                "g": {0: wl.norm_weight(SEED, 0, 0, 512)}, "slots": [0]}
    if name in ("llama1b_decode_layer0_b1", "llama8b_decode_layer0_b8"):
        layer, B = (wl.LLAMA_3_2_1B, 1) if "1b" in name else (wl.LLAMA_3_8B, 8)
        ks = wl.slot_k(layer)
        return {"w": [wl.weight(SEED, 0, i, m.M, m.K) for i, m in enumerate(layer)],
                "x": {s: wl.activation(SEED, 0, s, B, K) for s, K in ks.items()},
                "g": {s: wl.norm_weight(SEED, 0, s, K) for s, K in ks.items()},
                "slots": [m.slot for m in layer]}
    if name == "llama8b_prefill_kproj_t512":
        m = wl.LLAMA_3_8B[1]
        return {"w": [wl.weight(SEED, 0, 1, m.M, m.K)], "x": {0: wl.activation(SEED, 0, 0, 512, m.K)},
                "g": {0: wl.norm_weight(SEED, 0, 0, m.K)}, "slots": [0]}
    if name == "moe_64x16_top8_down":
        s = wl.MOE
        return {"w": [wl.weight(SEED, e, 0, s.hidden, s.ffn) for e in range(s.E)],
                "x": {0: wl.activation(SEED, 0, 0, s.T * s.top_k, s.ffn)},
                "g": {0: wl.norm_weight(SEED, 0, 0, s.ffn)},
                "ids": wl.expert_ids(SEED, s.T, s.E, s.top_k), "slots": [0]}
    raise KeyError(name)


def compute(name: str) -> dict[str, str]:
    import oracle

    inp = inputs(name)
    out = {}
    planes = {}
    for s in sorted(inp["x"]):
        xq, xd, xs = oracle.q8_quantize_rmsnorm(inp["x"][s], inp["g"][s], EPS)
        planes[s] = (xq, xd)
        out[f"x{s}.xq"], out[f"x{s}.xd"], out[f"x{s}.xs"] = digest(xq), digest(xd), digest(xs)
    quant = [oracle.q4_quantize(w) for w in inp["w"]]
    for i, (qs, d) in enumerate(quant):
        out[f"w{i}.qs"], out[f"w{i}.d"] = digest(qs), digest(d)
    if "ids" in inp:
        s = wl.MOE
        qs = np.stack([q for q, _ in quant])
        d = np.stack([dd for _, dd in quant])
        xq, xd = planes[0]
        xq = xq.reshape(s.T, s.top_k, s.ffn)
        xd = xd.reshape(s.T, s.top_k, s.ffn // 32)
        out["ids"] = digest(inp["ids"])
        out["y"] = digest(oracle.mul_mat_id(qs, d, xq, xd, inp["ids"], nthreads=8))
        return out
    for i, ((qs, d), slot) in enumerate(zip(quant, inp["slots"])):
        xq, xd = planes[slot]
        if name != "llama1b_decode_layer0_b1":
            out[f"w{i}.I"] = digest(oracle.block_dots(qs, qs.shape[1] * 2, xq))
        y, _ = oracle.mul_mat(qs, d, xq, xd, nthreads=8, want_y64=False)
        out[f"w{i}.y"] = digest(y)
    return out


def load() -> dict:
    with open(HASH_FILE) as f:
        return json.load(f)


def main():
    ap = argparse.ArgumentParser()
    g = ap.add_mutually_exclusive_group(required=True)
    g.add_argument("--record", action="store_true")
    g.add_argument("--check", action="store_true")
    args = ap.parse_args()
    if args.record:
        rec = {"_about": "SHA-256 of the oracle's planes on seeded inputs (tests/golden/oracle_hashes.py); "
                         "x<slot>: Q8 planes of RMSNorm*g of the activations, w<i>: Q4 planes of matrix i, "
                         "I: block sums, y: fp32 outputs (oracle's in-order sum)"}
        for name in CONFIGS:
            rec[name] = compute(name)
            print(f"recorded {name}: {len(rec[name])} arrays", flush=True)
        with open(HASH_FILE, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
            f.write("\n")
        return
    rec = load()
    bad = 0
    for name in CONFIGS:
        got = compute(name)
        for k, v in rec[name].items():
            if got.get(k) != v:
                bad += 1
                print(f"MISMATCH {name} {k}")
        print(f"checked {name}", flush=True)
    sys.exit(1 if bad else 0)


if __name__ == "__main__":
    main()
