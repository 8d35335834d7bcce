"""Writes decode_32k_step_seed0.txt: the oracle's output for one fused decode
step of the 32K-context GQA-8 layer (seed 0), which the benchmark's
correctness guard compares against.

The step quantizes the new token's K/V row into its pool row (the last table
entry) and attends over all 32,768 positions (FreeToken PR #853 "Follow-up
model/workload search": each new row is quantized on write, scales are loaded
during attention).  Only the oracle and the seeded input generator are used.

    python tests/golden/make_decode_32k_step.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from fp8_kv_cache_row_amd import workloads as wl  # noqa: E402

OUT = os.path.join(HERE, "decode_32k_step_seed0.txt")


def main():
    case = wl.layer_decode(0)
    kc, ks = oracle.quantize_rows(case.k_rows)
    vc, vs = oracle.quantize_rows(case.v_rows)
    row = int(case.table[0, -1])
    nkc, nks = oracle.quantize_rows(case.new_k)
    nvc, nvs = oracle.quantize_rows(case.new_v)
    kc[row], ks[row], vc[row], vs[row] = nkc[0], nks[0], nvc[0], nvs[0]
    out = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale,
                                  case.n_kv_heads)[0]
    with open(OUT, "w") as f:
        f.write("# Oracle output (fp64) of one fused decode step of layer_decode(seed=0): 32 q / 4 KV heads,\n")
        f.write("# head dim 128, 32,768 positions (the last one the new token, quantized on write into\n")
        f.write("# pool row table[0][32767]); one line per query head, 128 values.\n")
        f.write("# Written by tests/golden/make_decode_32k_step.py from the oracle alone.\n")
        for h in range(out.shape[0]):
            f.write(" ".join(f"{v:.9e}" for v in out[h]) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
