"""Writes sensitivity_c3.json: how far the oracle's own 30-layer bf16 stack
moves when its input is perturbed by half a bf16 unit in the last place.

The decoder stack of the 256-slot workload (4096-position prompt KV) is run
twice by the oracle on the embedded initial canvas: once as is, once with
every input element scaled by (1 +- 2^-9) (seeded random signs), with the
second run forced onto the first run's expert choices.  The per-layer
difference of the residual streams, max |x_b - x_a| / max |x_a|, is the
scale of rounding noise the stack itself amplifies; the end-to-end parity
tolerances of the GPU path at this size are derived from it.

Usage: python tests/golden/sensitivity_c3.py   (about 5 minutes, 45 GB RAM)
Calls only the oracle and the seeded input generators."""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import model as om  # noqa: E402
from oracle.inputs import prompt_kv_fn, weights_for  # noqa: E402
from synth import C3, gen  # noqa: E402


def main():
    w = C3
    m = w.model
    W = weights_for(w, cache_layers=True)
    kvf = prompt_kv_fn(w)
    tok0, _ = gen.canvas(w)
    x = om.bf16_bits_to_f64(gen.embed(w)[tok0.reshape(-1)])
    t0 = time.time()
    trace, xa = [], [x]
    for l in range(m.n_layers):
        xa.append(om.forward_hidden(xa[-1], W, m, kvf, [w.prompt_len], layers=[l], trace=trace))
        print(f"run a, layer {l} ({time.time() - t0:.0f} s)", flush=True)
    rng = np.random.default_rng(20260)
    xb = x * (1.0 + 2.0 ** -9 * rng.choice([-1.0, 1.0], size=x.shape))
    sh = om.Shadow(route_idx=[t["route_idx"] for t in trace], delta_route=1.0)
    per_layer = []
    for l in range(m.n_layers):
        xb = om.forward_hidden(xb, W, m, kvf, [w.prompt_len], layers=[l], shadow=sh)
        ref = xa[l + 1]
        per_layer.append(float(np.max(np.abs(xb - ref)) / np.max(np.abs(ref))))
        print(f"run b, layer {l}: {per_layer[-1]:.3e}", flush=True)
    out = {
        "_source": "written by tests/golden/sensitivity_c3.py from the oracle alone",
        "workload": w.name,
        "perturbation": "x_in * (1 +- 2^-9), seeded signs; routing forced to the unperturbed run",
        "forced_route_failures": len(sh.failures),
        "rel_diff_per_layer": per_layer,
        "rel_diff_max": max(per_layer),
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "sensitivity_c3.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
