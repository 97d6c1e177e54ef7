"""GPU parity of kvm_decode_step (needs an MI355X; marked gpu).

Decode outputs are compared with the oracle's prefill over the same tokens
under the GPU's decisions (the oracle's decode reproduces its prefill; see
test_I11_decode_reproduces_prefill).
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
from kvm_inputs import WORKLOADS, LayerConfig, make_inputs
from tests.parity import check_outputs, oracle_check, run_prefill, run_prefill_decode

pytestmark = pytest.mark.gpu

W4 = WORKLOADS[4]


def small(dtype="bf16", **kw):
    d = dict(name="small", batch=1, heads=3, n_tokens=600, chunk=64, window=128, n_sinks=4, sched="sqrt",
             alpha=6, dtype=dtype, key_gen="clustered", n_clusters=24, index=8)
    d.update(kw)
    return LayerConfig(**d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n0", [0, 192, 256, 300])
def test_decode_matches_oracle(dtype, n0):
    n = 700
    w = small(dtype)
    print(f"case: decode {dtype} prefill {n0} then {n - n0} steps", flush=True)
    inp = make_inputs(w, n_total=n)
    out, slot, kind, state, _ = run_prefill_decode(w, inp, n0, n - n0)
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, out, slot, kind, state, label="decode")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode_equals_prefill(dtype):
    n = 900
    w = small(dtype, chunk=32, window=96)
    print(f"case: prefill+decode == prefill {dtype}", flush=True)
    inp = make_inputs(w, n_total=n)
    a = run_prefill_decode(w, inp, 320, n - 320)
    b = run_prefill(w, inp, n_tokens=n)
    # identical decisions; each path meets the oracle bar on its own
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, a[0], a[1], a[2], a[3], label="prefill+decode")
        oracle_check(w, inp, s, n, b[0], b[1], b[2], b[3], label="prefill")


def test_decode_workload_sampled():
    """Batched decode workload: 64x16 sequences, sqrt-schedule prefill of 16384, then
    130 steps crossing one absorption (position 16384) and the next chunk boundary."""
    steps = 130
    n = W4.n_tokens + steps
    print(f"case: decode workload 64x16, prefill {W4.n_tokens} + {steps} steps", flush=True)
    inp = make_inputs(W4, n_total=n)
    out, slot, kind, state, _ = run_prefill_decode(W4, inp, W4.n_tokens, steps)
    # absorptions at positions 16384 and 16512: 127 chunks absorbed
    assert int(state["n_rows"][0]) == O.schedule(127, O.Params.of(W4))[-1][2] == 1020
    C = W4.chunk
    chunks = {W4.n_tokens // C - 1, W4.n_tokens // C, W4.n_tokens // C + 1}
    rows = np.arange(W4.n_tokens, n)
    for s in list(range(0, 1024, 64)) + [517, 1023]:   # 18 of the 1024 sequences, spread over the batch
        oracle_check(W4, inp, s, n, out, slot, kind, state, attend_chunks=chunks, rows=rows, label="decode-wl")
