"""GPU parity of the layer variants (needs an MI355X; marked gpu): the ablations
the pages study (no value-length normalisation, no sink protection, no merge
gate) and a power-law schedule, each against the oracle under the GPU's
decisions (teacher forcing), prefill and decode.
"""
import numpy as np
import pytest

import oracle.kvm_oracle as O
from kvm_inputs import LayerConfig, make_inputs
from tests.parity import oracle_check, run_prefill, run_prefill_decode

pytestmark = pytest.mark.gpu

VARIANTS = {
    "no_gate": dict(merge_gate=False),
    "no_value_norm": dict(value_norm=False),
    "no_sink_protect": dict(sink_protect=False),
    "power_0.6": dict(sched="power", alpha=3, exponent=0.6),
    "all_ablations": dict(merge_gate=False, value_norm=False, sink_protect=False),
}


def small(dtype, **kw):
    d = dict(name="variant", batch=1, heads=3, n_tokens=900, chunk=64, window=128, n_sinks=4, sched="sqrt",
             alpha=6, dtype=dtype, key_gen="clustered", n_clusters=24, index=9)
    d.update(kw)
    return LayerConfig(**d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,window", [(64, 128), (128, 256)])
@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_variant_prefill_matches_oracle(variant, dtype, chunk, window):
    n = 4 * window + chunk + 21
    w = small(dtype, chunk=chunk, window=window, n_tokens=n, **VARIANTS[variant])
    print(f"case: {variant} {dtype} C={chunk} W={window} n={n}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, out, slot, kind, state, label=variant)
    if not w.sink_protect:
        # the sink rows took merges (the variant is exercised)
        counts = state["count"][:, : w.n_sinks].cpu().numpy()
        assert counts.max() > 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ablations_decode_matches_oracle(dtype):
    n = 700
    w = small(dtype, n_tokens=n, **VARIANTS["all_ablations"])
    print(f"case: all ablations decode {dtype}", flush=True)
    inp = make_inputs(w, n_total=n)
    out, slot, kind, state, _ = run_prefill_decode(w, inp, 256, n - 256)
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, out, slot, kind, state, label="ablations decode")
