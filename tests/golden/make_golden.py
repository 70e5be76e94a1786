"""Write the oracle's regression fixtures (calls only oracle/ and the input generator).

    python tests/golden/make_golden.py

The pages print no worked numerical example of the merge or of the integer linear
layer, so these fixtures are not pins of the oracle: they record what the oracle
computes on the single-linear workload (320 x 320, W8A8, MUL with an 8-bit U, r = 4,
64 tokens) so that any later change to the oracle's arithmetic shows up in a test and
has to be made deliberately (regenerate with this script and say why in the commit).
"""
from __future__ import annotations

import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from integer_rank_adaptation_amd import synth  # noqa: E402

FIXTURE = os.path.join(HERE, "single_linear_320_mul8_r4.txt")


def compute():
    wl = synth.WORKLOADS[0]
    L = wl.layers[0]
    W = synth.weight(wl, 0)
    A, Bm = synth.lora(wl, 0)
    X = synth.activations(wl, L.n, wl.tokens[0])
    lid = synth.layer_id(0, 0)
    st = oracle.setup_layer(W, synth.PHILOX_SEED, lid, wl.w_bits, synth.ALPHA)
    ref = oracle.merge_mul(st["wround"], st["z"], st["s"], st["rstar"], A, Bm, 8)
    xq, sx, _ = oracle.quant_act(X)
    exact, _, y = oracle.linear(xq, sx, ref["m"].astype(np.int32), ref["sbar"])

    def sha(a):
        return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()

    return {
        "wround_sha256": sha(st["wround"]),
        "rstar_sha256": sha(st["rstar"]),
        "m_sha256": sha(ref["m"]),
        "sbar_sha256": sha(ref["sbar"]),
        "zbar_sha256": sha(ref["zbar"]),
        "exact_sha256": sha(exact),
        "y_bf16_sha256": sha(y),
        "m_row0_first16": " ".join(str(int(v)) for v in ref["m"][0, :16]),
        "saturated": str(int(ref["sat"])),
    }


def main():
    rec = compute()
    with open(FIXTURE, "w") as fh:
        fh.write("# oracle regression fixture: single linear 320 x 320, W8A8, MUL U 8-bit, r = 4, M = 64\n")
        fh.write("# written by tests/golden/make_golden.py (oracle/ only)\n")
        for k, v in rec.items():
            fh.write(f"{k} = {v}\n")
    print(FIXTURE)


if __name__ == "__main__":
    main()
