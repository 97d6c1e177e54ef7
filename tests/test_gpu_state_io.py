"""GPU tests of the state's life cycle through the C ABI (needs an MI355X; marked gpu):
reset, export (kvm_state_read) and resume (kvm_state_load), and the read of a
past snapshot.

The state is the whole carry of the chunk recurrence (the technical summary,
Core mechanisms 1: a separate state beside the exact window), so a state that
is reset, or exported and loaded into a fresh workspace, must continue exactly
like one that never stopped: outputs, decisions and state are compared bit for
bit.  The read of a past snapshot is compared with the oracle's own snapshot
under the GPU's decisions.
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
from compressed_kv_state_amd import KVM_E_INVALID_ARG, KvmConfig, KvmError, KvmState
from kvm_inputs import LayerConfig, make_inputs
from tests.parity import forced_map, run_prefill, seq_arrays, to_gpu

pytestmark = pytest.mark.gpu

STATE_KEYS = ("key_sum", "val_sum", "count", "rho", "key_read", "val_read", "trace_slot", "trace_kind")


def small(dtype="bf16", **kw):
    d = dict(name="stateio", batch=1, heads=3, n_tokens=1600, chunk=128, window=256, n_sinks=4, sched="sqrt",
             alpha=6, dtype=dtype, key_gen="clustered", n_clusters=24, index=11)
    d.update(kw)
    return LayerConfig(**d)


def new_state(w, n_max, seqs):
    cfg = KvmConfig.of(w, max_tokens=n_max, trace=True)
    cfg.batch, cfg.heads = seqs, 1
    return KvmState(cfg)


def decode_steps(st, inp, a, b):
    q, k, v, g = to_gpu(inp, a, b)
    return [st.decode_step(q[:, i].contiguous(), k[:, i].contiguous(), v[:, i].contiguous(),
                           g[:, i].contiguous())[:, None] for i in range(b - a)]


def snapshot_of(st):
    """The state's current contents on the host (rows beyond n_rows included: they are undefined,
    so only the first n_rows rows are compared)."""
    r = st.read(trace=True)
    torch.cuda.synchronize()
    n = int(r["n_rows"][0])
    out = {k: r[k][:, :n].cpu() if k not in ("trace_slot", "trace_kind") else r[k].cpu() for k in STATE_KEYS}
    out["n_rows"] = n
    return out


def assert_same_state(a, b):
    assert a["n_rows"] == b["n_rows"]
    for k in STATE_KEYS:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype,chunk,window,seqs", [("bf16", 128, 256, 4), ("f32", 64, 128, 3),
                                                     ("bf16", 64, 128, 32)])
def test_reset_is_a_fresh_state(dtype, chunk, window, seqs):
    """prefill, reset, prefill (other inputs) and decode == the same on a fresh state, bit for bit.
    Few sequences share the absorption over several workgroups, whose exchange buffers reset clears."""
    w = small(dtype, chunk=chunk, window=window)
    n1, n2, n3 = 1100, 900, 900 + 2 * chunk + 5
    print(f"case: reset {dtype} C={chunk} seqs={seqs}", flush=True)
    first = make_inputs(w, seqs=range(seqs), n_total=n1)
    second = make_inputs(w.replace(index=12), seqs=range(seqs), n_total=n3)
    st = new_state(w, max(n1, n3), seqs)
    st.prefill(*to_gpu(first, 0, n1))
    st.reset()
    assert st.info()["position"] == 0 and st.info()["absorbed_chunks"] == 0
    outs_a = [st.prefill(*to_gpu(second, 0, n2))] + decode_steps(st, second, n2, n3)
    state_a = snapshot_of(st)
    st.check()
    fresh = new_state(w, max(n1, n3), seqs)
    outs_b = [fresh.prefill(*to_gpu(second, 0, n2))] + decode_steps(fresh, second, n2, n3)
    state_b = snapshot_of(fresh)
    fresh.check()
    assert torch.equal(torch.cat(outs_a, 1).cpu(), torch.cat(outs_b, 1).cpu())
    assert_same_state(state_a, state_b)


@pytest.mark.parametrize("dtype,chunk,window,seqs", [("bf16", 128, 256, 4), ("f32", 64, 128, 3),
                                                     ("bf16", 256, 512, 2), ("bf16", 64, 128, 40)])
@pytest.mark.parametrize("cut", ["chunk boundary", "after decode steps"])
def test_export_load_continue_is_bitwise_uninterrupted(dtype, chunk, window, seqs, cut):
    """Export the state at a cut, load it into a fresh workspace, continue (prefill at a chunk
    boundary, else decode steps, then more decode steps): outputs, decisions and the final state
    equal those of the state that went on without stopping."""
    w = small(dtype, chunk=chunk, window=window)
    p = 6 * chunk + 2 * window                       # several absorbed chunks before the cut
    n_pre = p if cut == "chunk boundary" else p - chunk + 1
    n_end = p + 4 * chunk + 17
    n_dec = n_end + chunk + 3
    print(f"case: export/load {dtype} C={chunk} seqs={seqs} cut at {n_pre} ({cut})", flush=True)
    inp = make_inputs(w, seqs=range(seqs), n_total=n_dec)

    def head(st):
        st.prefill(*to_gpu(inp, 0, p - chunk if cut != "chunk boundary" else p))
        if cut != "chunk boundary":
            decode_steps(st, inp, p - chunk, n_pre)

    def tail(st):
        if cut == "chunk boundary":
            outs = [st.prefill(*to_gpu(inp, p, n_end))]
            outs += decode_steps(st, inp, n_end, n_dec)
        else:
            outs = decode_steps(st, inp, n_pre, n_dec)
        return torch.cat(outs, 1).cpu()

    a = new_state(w, n_dec, seqs)
    head(a)
    at_cut = a.info()
    saved = a.read(trace=True, ring=True)
    torch.cuda.synchronize()
    assert saved["position"] == n_pre
    saved = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in saved.items()}
    out_a = tail(a)
    state_a = snapshot_of(a)
    a.check()

    b = new_state(w, n_dec, seqs)
    b.load(saved)
    torch.cuda.synchronize()
    assert b.info()["position"] == n_pre and b.info()["absorbed_chunks"] == at_cut["absorbed_chunks"]
    assert b.info()["rows"] == at_cut["rows"]
    out_b = tail(b)
    state_b = snapshot_of(b)
    b.check()
    assert torch.equal(out_a, out_b)
    assert_same_state(state_a, state_b)


def test_load_rejects_a_state_of_another_shape():
    w = small("bf16", chunk=64, window=128)
    inp = make_inputs(w, seqs=range(2), n_total=700)
    a = new_state(w, 700, 2)
    a.prefill(*to_gpu(inp, 0, 640))
    saved = a.read(trace=True, ring=True)
    torch.cuda.synchronize()
    b = new_state(w, 700, 2)
    bad = dict(saved)
    bad["n_rows"] = saved["n_rows"] + 1                 # row counts that the schedule does not give
    with pytest.raises(KvmError) as e:
        b.load(bad)
    assert e.value.status == KVM_E_INVALID_ARG
    bad = dict(saved)
    bad["position"] = 10 ** 6                           # past max_tokens
    with pytest.raises(KvmError) as e:
        b.load(bad)
    assert e.value.status == KVM_E_INVALID_ARG
    bad = {k: v for k, v in saved.items() if k != "ring_k"}
    with pytest.raises(KvmError) as e:
        b.load(bad)
    assert e.value.status == KVM_E_INVALID_ARG
    assert b.info()["position"] == 0                    # nothing was queued
    b.load(saved)
    assert b.info()["position"] == 640


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_read_of_a_past_snapshot_matches_oracle(dtype):
    """kvm_state_read(chunk j): counts exactly, radii and read form within the read-form
    storage precision, against the oracle's snapshot after chunk j under the GPU's decisions."""
    w = small(dtype, chunk=64, window=128, n_tokens=1200)
    print(f"case: past snapshot read {dtype}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, st = run_prefill(w, inp)
    p = O.Params.of(w)
    absorbed = st.info()["absorbed_chunks"]
    with pytest.raises(KvmError) as e:                  # raw sums are current-state only
        st.read(chunk=0, sums=True)
    assert e.value.status == KVM_E_INVALID_ARG
    for s in range(w.seqs):
        res = O.prefill(*seq_arrays(inp, s, w.n_tokens), p, forced=forced_map(slot[s], kind[s]),
                        keep_snapshots=True, attend_chunks=set())
        for j in (0, 5, absorbed - 1):
            r = st.read(chunk=j)
            torch.cuda.synchronize()
            snap = res.snapshots[j]
            K, V, n, rho, _ = snap.arrays()
            S = snap.rows
            assert int(r["n_rows"][s]) == S
            np.testing.assert_array_equal(r["count"][s, :S].cpu().numpy(), n)
            np.testing.assert_allclose(r["rho"][s, :S].double().cpu().numpy(), rho, rtol=1e-6)
            kh, vh = O.read_form(snap, p)
            gk = r["key_read"][s, :S].double().cpu().numpy()
            gv = r["val_read"][s, :S].double().cpu().numpy()
            if dtype == "f32":
                assert np.max(np.abs(gk - kh[:, 32:])) <= 1e-5 * max(1.0, np.abs(kh).max())
                assert np.max(np.abs(gv - vh)) <= 1e-5 * max(1.0, np.abs(vh).max())
            else:
                assert np.max(np.abs(gk - kh[:, 32:])) <= 2 ** -8 + 1e-5
                assert np.all(np.abs(gv - vh) <= 2 ** -8 * np.abs(vh) + 1e-5 * np.abs(vh).max())
