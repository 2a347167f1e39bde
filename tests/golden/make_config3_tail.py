"""Write config3_tail.npz: what the oracle computes for the long-context workload (one
sequence of 32768 tokens after 128 meta tokens, window 1024, state 128) on the seeded
inputs of synth, for the rows and state the GPU test compares but cannot afford to
recompute at test time (the oracle's scan over 32896 positions x 4096 channels x 128
states takes minutes on a CPU).

Stored: y of the last 256 positions [256, 2048], the final state h of 512 sampled
channels [512, 128] with their indices, all in the oracle's storage-contract mode (the
mode the GPU parity tests compare against), as float32.  Inputs are regenerated from
synth by the test, and the file records the seeds' case id so a mismatch is detected.

Run from the repository root:  python tests/golden/make_config3_tail.py
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as orc  # noqa: E402
from synth import CASES, gen_activations, gen_layer_weights  # noqa: E402

TAIL = 256
N_CHAN = 512


def main():
    case = CASES[3]
    dims = case.dims
    L = case.seq_len
    w = gen_layer_weights(dims, case.case_id)
    _, meta, _, x = gen_activations(dims, case.case_id, 1, L)
    t0 = time.time()
    ref = orc.prefill(dims, w, meta, x, contract=True)
    print(f"oracle prefill of {L} tokens: {time.time() - t0:.0f} s", flush=True)
    chans = np.sort(np.random.default_rng(33).choice(dims.d_inner, N_CHAN, replace=False))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "config3_tail.npz")
    np.savez_compressed(out, case_id=case.case_id, seq_len=L, tail=TAIL,
                        y_tail=ref["y"][0, L - TAIL:].astype(np.float32),
                        chans=chans.astype(np.int32),
                        h_chans=ref["h"][0][chans].astype(np.float32))
    print("wrote", out)


if __name__ == "__main__":
    main()
