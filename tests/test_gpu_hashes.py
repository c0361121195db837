"""The library's codes, scales and exact block sums on the workload-shaped
seeded inputs against the oracle's recorded SHA-256 baseline
(tests/golden/oracle_hashes.json): full-size bit-exact checks without running
the oracle on the GPU machine.  fp32 outputs are compared within tolerance by the
other GPU tests; their hashes are the oracle's own regression record."""
import numpy as np
import pytest

from tests.golden import oracle_hashes as oh

pytestmark = pytest.mark.gpu


def _np(t, view=None):
    a = t.cpu().numpy()
    return a.view(view) if view is not None else a


@pytest.mark.parametrize("name", oh.CONFIGS)
def test_library_planes_match_recorded_hashes(name):
    import torch

    import block_quantized_matmul_q8_amd as q

    print(f"[hashes] {name}", flush=True)
    rec = oh.load()[name]
    inp = oh.inputs(name)
    dev = torch.device("cuda:0")
    got = {}
    planes = {}
    for s in sorted(inp["x"]):
        x = torch.from_numpy(inp["x"][s]).to(dev)
        g = torch.from_numpy(inp["g"][s]).to(dev)
        xq, xd, xs = q.q8_quantize_rmsnorm(x, g, oh.EPS, want_xs=True)
        planes[s] = (xq, xd)
        got[f"x{s}.xq"], got[f"x{s}.xd"], got[f"x{s}.xs"] = (oh.digest(_np(xq)), oh.digest(_np(xd)),
                                                              oh.digest(_np(xs)))
    quant = []
    for i, w in enumerate(inp["w"]):
        qs, d = q.q4_quantize(torch.from_numpy(w).to(dev))
        quant.append((qs, d))
        got[f"w{i}.qs"], got[f"w{i}.d"] = oh.digest(_np(qs)), oh.digest(_np(d, np.uint16))
    if "ids" in inp:
        got["ids"] = oh.digest(inp["ids"])
    else:
        for i, ((qs, d), slot) in enumerate(zip(quant, inp["slots"])):
            if f"w{i}.I" not in rec:
                continue
            xq, xd = planes[slot]
            y, I = q.mul_mat_q4q8_blocksums(qs, d, xq, xd)
            torch.cuda.synchronize()
            assert torch.isfinite(y).all()
            got[f"w{i}.I"] = oh.digest(_np(I))
            del y, I
    torch.cuda.synchronize()
    exact = {k: v for k, v in rec.items() if not k.endswith(".y") and k != "y"}
    assert set(exact) <= set(got), sorted(set(exact) - set(got))
    bad = [k for k in exact if got[k] != exact[k]]
    assert not bad, f"{name}: {bad}"
