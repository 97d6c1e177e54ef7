"""kvm_prefill_noalloc (the entry point for callers that cannot allocate device memory)
against the existing create + prefill path, through the C ABI (needs an MI355X; marked gpu).

Both run the same kernels, so the outputs must agree bit for bit.  Calls come in a row
on one process's scratch, each smaller than or as large as the one before, so a later
call also checks that the entry point clears what must start at zero (counters, the
scan's exchange records) instead of finding the last call's contents.
"""
import numpy as np
import pytest
import torch

from compressed_kv_state_amd import (KVM_E_INVALID_ARG, KVM_E_WORKSPACE, KvmConfig, KvmError, KvmState,
                                     prefill_noalloc)
import oracle.kvm_oracle as O
from kvm_inputs import LayerConfig, make_inputs
from tests.parity import check_outputs, seq_arrays, to_gpu

pytestmark = pytest.mark.gpu


def layer(dtype, seqs, n, chunk, window, **kw):
    d = dict(name="noalloc", batch=seqs, heads=1, n_tokens=n, chunk=chunk, window=window, n_sinks=4,
             sched="sqrt", alpha=8, dtype=dtype, key_gen="clustered", n_clusters=32, index=21)
    d.update(kw)
    return LayerConfig(**d)


CALLS = [   # in order; each input no larger than the one before
    layer("bf16", 4, 1700, 128, 256),                           # scan split over 8 workgroups per sequence
    layer("bf16", 2, 1100, 128, 256, index=22),                 # same split, other offsets in the scratch
    layer("f32", 3, 700, 64, 128, sched="fixed", max_slots=40, index=23),
]


def run_both(w):
    inp = make_inputs(w)
    q, k, v, g = to_gpu(inp)
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens)
    out_na = torch.full_like(q, float("nan"))
    prefill_noalloc(cfg, q, k, v, g, out_na)
    st = KvmState(cfg)
    out_ref = st.prefill(q, k, v, g)
    torch.cuda.synchronize()
    st.check()
    return inp, out_na.cpu(), out_ref.cpu()


def test_noalloc_prefill_matches_the_state_path_on_calls_in_a_row():
    for i, w in enumerate(CALLS):
        print(f"case: noalloc call {i}: {w.dtype} {w.seqs}x{w.n_tokens} C={w.chunk}", flush=True)
        inp, got, want = run_both(w)
        assert torch.equal(got, want), f"call {i}: outputs differ from kvm_prefill"
        if i == len(CALLS) - 1:
            # and against the oracle, to the fp32 bar, on one sequence
            res = O.prefill(*seq_arrays(inp, 0, w.n_tokens), O.Params.of(w))
            ok, worst, bound, _ = check_outputs(w.dtype, got[0].double().numpy(), res.out)
            assert ok, (worst, bound)


def test_noalloc_rejects_what_it_cannot_run():
    w = CALLS[-1]
    inp = make_inputs(w)
    q, k, v, g = to_gpu(inp)
    out = torch.empty_like(q)
    big = KvmConfig.of(layer("bf16", 64, 16384, 128, 256), max_tokens=16384)   # workspace past the scratch
    qb = torch.zeros(64, 16384, 64, dtype=torch.bfloat16, device="cuda")
    gb = torch.zeros(64, 16384, dtype=torch.float32, device="cuda")
    with pytest.raises(KvmError) as e:
        prefill_noalloc(big, qb, qb, qb, gb, torch.empty_like(qb))
    assert e.value.status == KVM_E_WORKSPACE
    traced = KvmConfig.of(w, max_tokens=w.n_tokens, trace=True)
    with pytest.raises(KvmError) as e:
        prefill_noalloc(traced, q, k, v, g, out)
    assert e.value.status == KVM_E_INVALID_ARG
