"""Find the Zipf exponent of the 16-layer prefill stack (writes nothing; prints it).

The stack's routing is skewed so that its busiest expert gets about four times
the mean load (the switchyard page, §03 "Load balance", measures 4.0x at 2,048
tokens per GPU).  The skew comes from a router bias ``alpha * ln(1/rank)`` over
a seeded ranking of the experts; this script bisects ``alpha`` on layer 0 of
the stack, with the oracle's own RMSNorm, logits and top-k, until
``max_e count_e / (T*k/E)`` is 4.0, and prints the value to store as
``moe_synth.STACK_ZIPF_ALPHA``.  Uses only the oracle and the input generator.

    python -m oracle.tune_zipf_alpha
"""
import dataclasses

import numpy as np

import moe_synth
from oracle import moe_oracle as O


def skew(alpha: float, x_norm, layer) -> float:
    wl = dataclasses.replace(moe_synth.OLMOE_STACK16, zipf_alpha=alpha)
    bias = moe_synth.zipf_bias(wl, 0, 0)
    logits = O.router_logits(x_norm, layer.w_router, bias)
    ids, _ = O.route(logits, wl.k, wl.renormalize)
    counts, _, _, _ = O.permute(ids, wl.E)
    return counts.max() / (x_norm.shape[0] * wl.k / wl.E)


def main():
    wl = moe_synth.OLMOE_STACK16
    T = wl.tokens[0]
    x = moe_synth.make_tokens(wl, T, seed=0, layer=0)
    xn = O.rmsnorm(x, wl.norm_eps)
    # the router only needs W_r; draw the layer once (expert weights unused here)
    layer = moe_synth.make_layer(dataclasses.replace(wl, E=wl.E, I=8), layer=0, seed=0)
    lo, hi = 0.0, 4.0
    for _ in range(12):
        mid = 0.5 * (lo + hi)
        if skew(mid, xn, layer) < 4.0:
            lo = mid
        else:
            hi = mid
    for a in (lo, hi):
        print(f"alpha={a:.8f} max/mean={skew(a, xn, layer):.4f}")
    print(f"stored value {moe_synth.STACK_ZIPF_ALPHA}: max/mean="
          f"{skew(moe_synth.STACK_ZIPF_ALPHA, xn, layer):.4f}")


if __name__ == "__main__":
    main()
