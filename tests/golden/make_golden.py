"""Write tiny_layer_oracle.npz: the fp64 oracle on the tiny workload.

Calls only ``oracle`` and ``synth``.  Re-run after a deliberate change to the
oracle's arithmetic (and say in the commit which passage justifies it).
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import moe_oracle as mo  # noqa: E402


def tiny_oracle():
    wl = synth.TINY
    x = mo.act_bits_to_f64(synth.tokens(wl), wl.act_dtype)
    wr = mo.f16_bits_to_f64(synth.router_weights(wl, 0))

    def load(e, shared=False):
        raw = synth.expert_raw(wl, 0, e, shared=shared)
        return mo.ExpertWeights.from_quant(raw["gate"], raw["up"], raw["down"], wl.group)

    out = mo.layer_forward(x, wr, None, lambda e: load(e), load(0, shared=True), wl.top_k)
    return out


if __name__ == "__main__":
    out = tiny_oracle()
    np.savez(os.path.join(HERE, "tiny_layer_oracle.npz"), y=out["y"], idx=out["idx"], w=out["w"],
             gamma=out["gamma"], z=out["z"])
    print("wrote tiny_layer_oracle.npz", out["idx"].tolist())
