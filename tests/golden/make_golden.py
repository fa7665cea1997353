"""Writes tests/golden/oracle_tiny_d8.json.

Inputs come from the seeded generator (gdn_inputs); expected outputs come from
the fp64 oracle only (oracle.forward).  Nothing here touches the HIP library.
The fixture freezes the oracle's answer on a small packed batch (two sequences,
ragged lengths 70 and 9, GVA with G = 2, nonzero initial state) so that a later
change to the oracle's arithmetic cannot pass unnoticed.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import gdn_inputs  # noqa: E402
import oracle  # noqa: E402


def main():
    inp = gdn_inputs.make_prefill(seed=123, seqlens=[70, 9], H_q=1, H_v=2, d_k=8, d_v=8, dtype="f32",
                                  state_std=0.5)
    out, fin = oracle.forward(inp.q32(), inp.k32(), inp.v32(), inp.g, inp.beta, inp.cu_seqlens, inp.H_q, inp.H_v,
                              inp.scale, initial_state=inp.initial_state.astype("float64"))
    fx = dict(
        source="oracle.forward (fp64 token recurrence), inputs gdn_inputs.make_prefill(seed=123, seqlens=[70, 9], "
               "H_q=1, H_v=2, d_k=8, d_v=8, dtype='f32', state_std=0.5)",
        H_q=inp.H_q, H_v=inp.H_v, scale=inp.scale,
        arrays=dict(q=inp.q32().tolist(), k=inp.k32().tolist(), v=inp.v32().tolist(), g=inp.g.tolist(),
                    beta=inp.beta.tolist(), cu_seqlens=inp.cu_seqlens.tolist(),
                    initial_state=inp.initial_state.astype("float64").tolist(), out=out.tolist(),
                    final_state=fin.tolist()),
    )
    with open(os.path.join(HERE, "oracle_tiny_d8.json"), "w") as f:
        json.dump(fx, f, separators=(",", ":"))


if __name__ == "__main__":
    main()
