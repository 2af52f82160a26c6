"""Writes the oracle's free-running 32-block stack chain (256 decoded tokens) to
``stack_chain.npz`` beside this file.

The chain is the stack workload (32 blocks of q8_0 linears 4096/11008, adapters
rank 16 at 1.0 then rank 64 at 0.5 on every projection, 256 tokens, each token's
input the previous token's output) computed by the oracle alone: the oracle's
quantiser, the oracle's float64 dual path and glue, and the seeded inputs of
``synth``.  Nothing here touches the GPU library.  Stored: tokens 0..31 and 63,
127, 191, 255 (float64), plus the x0 and the workload parameters they came from.

Run:  python tests/golden/make_stack_chain.py   (about 10-20 minutes on 8 cores)
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import workloads  # noqa: E402

KEEP = list(range(32)) + [63, 127, 191, 255]
OUT = os.path.join(HERE, "stack_chain.npz")


def oracle_layers(wl):
    layers = []
    for i, L in enumerate(wl.linears):
        blocks = oracle.quantize(L.qtype, wl.weight(i))
        ads = [oracle.Lora(wl.lora_a(i, a), wl.lora_b(i, a), spec.scale) for a, spec in enumerate(wl.adapters)]
        layers.append(oracle.Layer(L.qtype, blocks, L.n_out, L.k_in, ads))
        if i % 7 == 6:
            print(f"block {i // 7} quantised", flush=True)
    return layers


def main(n_tokens: int = 256, seg: int = 8):
    wl = workloads.stack()
    assert wl.tokens == n_tokens
    t0 = time.time()
    layers = oracle_layers(wl)
    print(f"layers ready in {time.time() - t0:.0f} s", flush=True)
    x0 = wl.x0()[0].astype(np.float64)
    y = np.empty((n_tokens, x0.size), np.float64)
    h = x0
    for t in range(0, n_tokens, seg):
        n = min(seg, n_tokens - t)
        y[t:t + n] = oracle.stack(layers, h, n)
        h = y[t + n - 1]
        print(f"tokens {t}..{t + n - 1} done at {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(OUT, tokens=np.array(KEEP, np.int64), y=y[KEEP], x0=x0,
                        workload=np.array([wl.name, "32 blocks 4096/11008 q8_0, r16@1.0 then r64@0.5"]))
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
