"""Write tests/golden/brute_small.json from the 40-digit brute-force route only.

The pages print no worked example of the operation, so the stored values are
computed here by oracle/brute.py (explicit transition-matrix products in
mpmath at 40 significant digits), never by the C oracle or the HIP library.
Inputs are seeded draws from workloads.py.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle import brute  # noqa: E402


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def main():
    cases = []
    specs = [("K4_T6_decay", dict(T=6, H=2, K=4, lb=-5.0, init="fp32", seed=11)),
             ("K4_T5_nodecay", dict(T=5, H=1, K=4, lb=0.0, init=None, seed=12)),
             ("K8_T8_weak", dict(T=8, H=1, K=8, lb=-2.0, init="fp32", seed=13, g_mean=-4.0))]
    for name, s in specs:
        w = W.make(name, 1, s["T"], s["H"], s["seed"], K=s["K"], V=s["K"], lower_bound=s["lb"],
                   init=s["init"], g_mean=s.get("g_mean", 0.0))
        h0 = None if w.initial_state is None else w.initial_state[0].double().numpy()
        out, fin = brute.run(bits(w.q[0]), bits(w.k[0]), bits(w.v[0]), bits(w.g[0]), bits(w.beta[0]),
                             w.scale, w.A_log.numpy(), w.dt_bias.numpy(), w.lower_bound, h0)
        cases.append({
            "name": name,
            "shape": {"T": w.T, "H": w.H, "K": w.K, "V": w.V},
            "q": bits(w.q).ravel().tolist(), "k": bits(w.k).ravel().tolist(),
            "v": bits(w.v).ravel().tolist(), "g": bits(w.g).ravel().tolist(),
            "beta": bits(w.beta).ravel().tolist(),
            "A_log": [float(x) for x in w.A_log.numpy()],
            "dt_bias": [float(x) for x in w.dt_bias.numpy().ravel()],
            "lower_bound": w.lower_bound, "scale": w.scale,
            "initial_state": None if h0 is None else [float(x) for x in h0.ravel()],
            "out": [repr(float(x)) for x in out.ravel()],
            "final_state": [repr(float(x)) for x in fin.ravel()],
        })
    doc = {
        "source": "oracle/brute.py: S_t = A_t...A_1 S_0 + sum_j (A_t...A_{j+1}) b_j k_j v_j^T with "
                  "A_t = (I - b_t k_t k_t^T) Diag(exp(a_t)), o_t = scale S_t^T q_t, mpmath 40 digits; "
                  "the gated delta rule with per-channel decay as described in 'What is Kimi Delta "
                  "Attention (KDA)' (kongchang.com/en) and '¿Qué es la atención Kimi Delta…' (7minutos.es)",
        "inputs": "bf16 bit patterns (uint16), row-major [1,T,H,K|V]; A_log [H], dt_bias [H,K] fp32",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_small.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
