"""GPU parity of kvm_prefill_backward against the oracle's backward (needs an MI355X; marked gpu).

The oracle differentiates its forward under the GPU's decisions (teacher forcing), so both
sides take the gradient of the same function.  Bars, per sequence and gradient tensor
(d_q, d_k, d_v, d_gate):
  fp32 path: max |diff| <= 1e-4 * max(1, max |oracle|), the forward's fp32 bar scaled to the
  gradient's magnitude;
  bf16 path: the forward's bf16 bar: max |diff| of each row <= 2e-2 * max(RMS(oracle),
  RMS(oracle row)) and RMS(diff) <= 2e-2 * RMS(oracle).
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
import oracle.kvm_oracle_grad as G
from compressed_kv_state_amd import KVM_E_INVALID_ARG, KVM_E_STATE, KvmConfig, KvmError, KvmState
from kvm_inputs import WORKLOADS, LayerConfig, make_inputs
from tests.parity import forced_map, record, seq_arrays, to_gpu

pytestmark = pytest.mark.gpu


def small(dtype, **kw):
    d = dict(name="bwd", batch=1, heads=3, n_tokens=900, chunk=64, window=128, n_sinks=4, sched="sqrt", alpha=6,
             dtype=dtype, key_gen="clustered", n_clusters=24, index=31)
    d.update(kw)
    return LayerConfig(**d)


def run_backward(w, inp, seed=0):
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens, trace=True)
    cfg.batch, cfg.heads = inp.q.shape[0], 1
    st = KvmState(cfg)
    q, k, v, g = to_gpu(inp)
    out = st.prefill(q, k, v, g)
    gen = torch.Generator().manual_seed(1234 + seed)
    d_out = torch.randn(out.shape, generator=gen).to(out.dtype).cuda()
    grads = st.backward(q, k, v, g, d_out)
    state = st.read(trace=True)
    torch.cuda.synchronize()
    st.check()
    slot = state["trace_slot"].long().cpu().numpy()
    kind = state["trace_kind"].long().cpu().numpy()
    kind[kind == 255] = O.KIND_NONE
    return st, d_out.double().cpu().numpy(), [t.double().cpu().numpy() for t in grads], slot, kind, (q, k, v, g, d_out)


def grad_ok(dtype, got, want):
    """(ok, worst, rel_rms) of one gradient tensor of one sequence against the bars above."""
    got = got.reshape(len(got), -1)
    want = want.reshape(len(want), -1)
    err = np.abs(got - want)
    rms = max(float(np.sqrt(np.mean(want ** 2))), 1e-30)
    rel = float(np.sqrt(np.mean(err ** 2)) / rms)
    if dtype == "f32":
        bound = 1e-4 * max(1.0, float(np.abs(want).max()))
        worst = float(err.max()) / bound * 1e-4
        return err.max() <= bound, worst, rel
    ref = np.maximum(np.sqrt(np.mean(want ** 2, axis=1)), rms)
    worst = float(np.max(err.max(axis=1) / ref))
    return worst <= 2e-2 and rel <= 2e-2, worst, rel


def check_seq(w, inp, s, d_out, grads, slot, kind, label):
    p = O.Params.of(w)
    arr = seq_arrays(inp, s, w.n_tokens)
    res = G.prefill_grad(*arr, d_out[s], p, forced=forced_map(slot[s], kind[s]))
    want = (res.dq, res.dk, res.dv, res.dl[:, None])
    names = ("d_q", "d_k", "d_v", "d_gate")
    msgs = []
    ok_all = True
    for name, g_, w_ in zip(names, [grads[0][s], grads[1][s], grads[2][s], grads[3][s][:, None]], want):
        ok, worst, rel = grad_ok(w.dtype, g_, w_)
        record(f"backward {label} {name}", None, worst, rel)
        msgs.append(f"{name} worst {worst:.3g} rms {rel:.3g}")
        ok_all &= bool(ok)
    print(f"   [{label} seq {s}] " + "; ".join(msgs), flush=True)
    assert ok_all, msgs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,window", [(32, 64), (64, 128), (128, 256), (256, 512)])
def test_backward_matches_oracle(dtype, chunk, window):
    n = 3 * window + 2 * chunk + 19               # several absorptions and a ragged tail
    w = small(dtype, chunk=chunk, window=window, n_tokens=n, heads=3 if chunk < 256 else 2)
    print(f"case: backward {dtype} C={chunk} W={window} n={n}", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, _ = run_backward(w, inp)
    for s in range(w.seqs):
        check_seq(w, inp, s, d_out, grads, slot, kind, f"C{chunk} {dtype}")


VARIANTS = {
    "no_gate": dict(merge_gate=False),
    "no_value_norm": dict(value_norm=False),
    "no_sink_protect": dict(sink_protect=False),
    "softmax_scale": dict(softmax_scale=0.23),
    "fixed": dict(sched="fixed", max_slots=40),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_backward_variants(dtype, variant):
    w = small(dtype, chunk=64, window=128, n_tokens=777, **VARIANTS[variant])
    print(f"case: backward {variant} {dtype}", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, _ = run_backward(w, inp)
    for s in range(w.seqs):
        check_seq(w, inp, s, d_out, grads, slot, kind, variant)


def test_backward_state_past_lds_index_cap():
    """bf16 path with snapshots of more than 4096 rows: the attention-backward kernels then read
    the snapshot's version ids from global memory instead of their LDS copy."""
    w = small("bf16", chunk=128, window=256, n_tokens=4819, heads=1, sched="fixed", max_slots=4400)
    print("case: backward, snapshots past 4096 rows", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, _ = run_backward(w, inp)
    assert int((slot[0] >= 4096).sum()) > 0   # rows past the cap exist and are used
    check_seq(w, inp, 0, d_out, grads, slot, kind, "past idx cap")


@pytest.mark.parametrize("n", [1, 70, 200])
def test_backward_short_inputs(n):
    w = small("f32", n_tokens=n, heads=2)
    print(f"case: backward short n={n}", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, _ = run_backward(w, inp)
    for s in range(w.seqs):
        check_seq(w, inp, s, d_out, grads, slot, kind, "short")


def test_backward_is_deterministic_and_checks_its_arguments():
    w = small("bf16", chunk=128, window=256, n_tokens=1500, heads=4)
    print("case: backward determinism", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, (q, k, v, g, do) = run_backward(w, inp)
    again = st.backward(q, k, v, g, do)
    torch.cuda.synchronize()
    for a, b in zip(grads, again):
        assert np.array_equal(a, b.double().cpu().numpy())
    with pytest.raises(KvmError) as e:                  # position differs from n
        st.backward(q[:, :1400].contiguous(), k[:, :1400].contiguous(), v[:, :1400].contiguous(),
                    g[:, :1400].contiguous(), do[:, :1400].contiguous())
    assert e.value.status == KVM_E_STATE
    cfg = KvmConfig.of(w, max_tokens=w.n_tokens)      # no trace: the decisions are not kept
    cfg.batch, cfg.heads = 4, 1
    st2 = KvmState(cfg)
    st2.prefill(q, k, v, g)
    with pytest.raises(KvmError) as e:
        st2.backward(q, k, v, g, do)
    assert e.value.status == KVM_E_INVALID_ARG


@pytest.mark.parametrize("widx,seqs", [(1, (0, 29)), (2, (5,))])
def test_backward_workloads_sampled(widx, seqs):
    w = WORKLOADS[widx]
    print(f"case: backward {w.name}, oracle on sequences {seqs}", flush=True)
    inp = make_inputs(w)
    st, d_out, grads, slot, kind, _ = run_backward(w, inp)
    for s in seqs:
        check_seq(w, inp, s, d_out, grads, slot, kind, w.name)
