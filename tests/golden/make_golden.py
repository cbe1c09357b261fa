"""Writes tests/golden/tiny_layer.json: a tiny MoE layer (inputs drawn with numpy,
seed 7) and the FP64 oracle's outputs for it, dropless and with capacity C = 1/2.
Calls only the oracle; rerun only when the oracle's arithmetic changes for a reason
the pages justify.  Usage: python tests/golden/make_golden.py"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle as O  # noqa: E402


def main():
    r = np.random.default_rng(7)
    T, d, E, k, F = 6, 4, 4, 2, 3
    x = np.round(r.normal(size=(T, d)), 3)
    wr = np.round(r.normal(size=(E, d)), 3)
    bias = np.round(r.normal(size=E) * 0.5, 3)
    ex = [[np.round(r.normal(size=s) * 0.5, 3).tolist() for s in ((F, d), (F, d), (d, F))] for _ in range(E)]
    fn = lambda e: [np.array(m) for m in ex[e]]  # noqa: E731
    cases = {}
    for name, cap in (("dropless", None), ("cap_half", (1, 2))):
        res = O.moe_layer(x, wr, fn, E, k, logit_bias=bias, capacity=cap)
        cases[name] = dict(capacity=cap, out=res["out"].tolist(), idx=res["idx"].tolist(),
                           gates=res["gates"].tolist(), drop=res["drop"].tolist(),
                           offsets=res["offsets"].tolist(), slot_row=res["slot_row"].tolist())
    doc = dict(about="tiny MoE layer; expected values written by make_golden.py from the FP64 oracle",
               T=T, d=d, E=E, k=k, ffn=F, x=x.tolist(), w_router=wr.tolist(), logit_bias=bias.tolist(),
               experts=ex, cases=cases)
    with open(os.path.join(HERE, "tiny_layer.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
