"""Large inputs through moe_forward, checked on sampled tokens against the fp64 oracle:
the OLMoE-shaped layer at T = 32768 (matrix-core router, multi-workgroup sort, ring GEMM)
and a wide layer whose sorted-rows buffer holds more than 2^31 elements, so every offset
into it must be formed in 64 bits.  The token rows repeat a seeded block of 512."""
import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O
from tests import gpu_cases as C

pytestmark = pytest.mark.gpu

WIDE = S.Workload("wide_rows", 98, d=16384, E=8, k=3, I=64, S=1, renormalize=True,
                  tokens=(40000,))


def _check(wl, T):
    from grouped_expert_ffn_amd import DeviceLayer, to_device
    t = C.torch()
    host = S.make_layer(wl, 0)
    dl = DeviceLayer(C.desc_of(wl), host.w_router, host.bias, host.w_gate, host.w_up, host.w_down)
    # 512 seeded token rows repeated: generating every row would take minutes on the host,
    # and the size, not the values, is what these cases test
    base = S.make_tokens(wl, 512)
    x = np.ascontiguousarray(np.tile(base, ((T + 511) // 512, 1))[:T])
    ids = t.empty((T, wl.k), dtype=t.int32, device="cuda")
    y = dl.forward(to_device(x), topk_ids=ids)
    t.cuda.synchronize()
    tok = sorted(set(range(0, T, max(1, T // 24))) | {T - 1})
    ids_g = ids.cpu().numpy()[tok]
    xs = x[tok]
    logits = O.router_logits(xs, host.w_router, host.bias)
    C.check_routing_against_oracle(ids_g, logits, wl.k)
    w_ref = O.gate_weights_for(logits, ids_g, wl.renormalize)
    y_ref = O.moe_layer(xs, O.Experts.from_layer(host), ids_g, w_ref, wl.S, wl.E)
    C.assert_close(C.widen_dev(y[tok]), y_ref, wl.act, f"{wl.name} T={T}")


@pytest.mark.timeout(300)
def test_olmoe_layer_at_32k_tokens():
    _check(S.OLMOE_BF16, 32768)


@pytest.mark.timeout(300)
def test_rows_buffer_past_2_pow_31_elements():
    T = WIDE.tokens[0]
    assert (T * WIDE.k + WIDE.S * T) * WIDE.d > 2 ** 31
    _check(WIDE, T)


# K = 16384 for gate/up: both GEMVs take several rounds over K per row chunk (weights
# reloaded per round), T = 5 on the VALU GEMV, T = 12 on the matrix-core GEMV (64-K blocks,
# 32 per round: eight rounds)
@pytest.mark.parametrize("T", [5, 12])
def test_wide_rows_at_decode_sizes(T):
    _check(WIDE, T)
