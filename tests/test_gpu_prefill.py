"""GPU parity of kvm_prefill against the oracle (needs an MI355X; marked gpu).

Decisions (append sets, merge targets) are compared chunk by chunk with the
oracle replaying the GPU's history (teacher forcing); outputs and state are
compared with the oracle run under the same decisions.  See tests/parity.py
for the bars.
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
from compressed_kv_state_amd import KVM_E_CAPACITY, KVM_E_STATE, KvmConfig, KvmError, KvmState
from kvm_inputs import WORKLOADS, LayerConfig, make_inputs
from tests.parity import (check_outputs, forced_map, free_running_check, oracle_check, run_prefill,
                          run_prefill_decode, seq_arrays, to_gpu)

pytestmark = pytest.mark.gpu

W0, W1, W2, W3 = WORKLOADS[:4]


def small(dtype="bf16", **kw):
    d = dict(name="small", batch=1, heads=3, n_tokens=1000, chunk=64, window=128, n_sinks=4, sched="sqrt",
             alpha=6, dtype=dtype, key_gen="clustered", n_clusters=24, index=7)
    d.update(kw)
    return LayerConfig(**d)


# ------------------------------------------------------------------ full workloads

def test_tiny_f32_workload_exact():
    print("case: tiny fp32 workload, 1x1x1024", flush=True)
    inp = make_inputs(W0)
    out, slot, kind, state, _ = run_prefill(W0, inp)
    rep, worst, _, res = oracle_check(W0, inp, 0, W0.n_tokens, out, slot, kind, state, label="tiny")
    assert rep.append_near_tie_diff == 0 and rep.merge_near_tie_diff == 0
    free = O.prefill(*seq_arrays(inp, 0, W0.n_tokens), O.Params.of(W0))
    assert check_outputs("f32", out[0], free.out)[0]


_RUNS = {}
_FORCED = {}


def workload_run(w):
    """One GPU prefill of a whole workload, shared by the tests of this module."""
    if w.name not in _RUNS:
        inp = make_inputs(w)
        out, slot, kind, state, st = run_prefill(w, inp)
        st.close()
        _RUNS[w.name] = (inp, out, slot, kind, state)
    return _RUNS[w.name]


def test_120m_fixed256_workload_all_sequences():
    print("case: 120M-shaped fixed-256 workload, 4x12x8192, oracle on all 48 sequences", flush=True)
    inp, out, slot, kind, state = workload_run(W1)
    for s in range(W1.seqs):
        rep, _, _, _ = oracle_check(W1, inp, s, W1.n_tokens, out, slot, kind, state, label=W1.name)
        _FORCED[(W1.name, s)] = rep


def test_120m_fixed256_free_running_decisions():
    print("case: 120M-shaped workload, free-running oracle decisions on all 48 sequences", flush=True)
    inp, out, slot, kind, state = workload_run(W1)
    for s in range(W1.seqs):
        free_running_check(W1, inp, s, W1.n_tokens, slot, kind, _FORCED.get((W1.name, s)), W1.name + " free-running")


def test_350m_sqrt_workload_all_sequences_and_planted_keys():
    print("case: 350M-shaped sqrt workload, 2x16x32768, oracle on all 32 sequences", flush=True)
    inp, out, slot, kind, state = workload_run(W2)
    # I12: every planted isolated key is appended, in every sequence
    for s in range(W2.seqs):
        assert np.all(kind[s][inp.planted_pos[s]] == O.KIND_APPEND), s
    assert int(state["n_rows"][0]) == 1440
    for s in range(W2.seqs):
        rep, _, _, _ = oracle_check(W2, inp, s, W2.n_tokens, out, slot, kind, state, label=W2.name)
        _FORCED[(W2.name, s)] = rep


def test_350m_sqrt_free_running_decisions():
    print("case: 350M-shaped workload, free-running oracle decisions on all 32 sequences", flush=True)
    inp, out, slot, kind, state = workload_run(W2)
    for s in range(W2.seqs):
        free_running_check(W2, inp, s, W2.n_tokens, slot, kind, _FORCED.get((W2.name, s)), W2.name + " free-running")
    _RUNS.pop(W2.name, None)


def test_long_saturating_workload_sampled():
    print("case: long saturating workload, 1x16x131072, oracle on 4 sequences, sampled chunks", flush=True)
    inp = make_inputs(W3)
    out, slot, kind, state, _ = run_prefill(W3, inp)
    assert int(state["n_rows"][0]) == 4096
    C = W3.chunk
    chunks = {0, 1, 2, 3, 4, 200, 257, 258, 259, 300, 400, 511}
    rows = np.concatenate([np.arange(c * C, (c + 1) * C) for c in sorted(chunks)])
    for s in (0, 3, 9, 15):
        oracle_check(W3, inp, s, W3.n_tokens, out, slot, kind, state, attend_chunks=chunks, rows=rows,
                     label=W3.name + " (sampled chunks)")


def test_deterministic_repeat():
    print("case: determinism, 120M-shaped workload twice", flush=True)
    w = W1.replace(n_tokens=4096)
    inp = make_inputs(w, seqs=range(16))
    a = run_prefill(w, inp)
    b = run_prefill(w, inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    for key in ("key_sum", "val_sum", "count", "rho", "key_read", "val_read"):
        assert torch.equal(a[3][key], b[3][key]), key


# ------------------------------------------------------------------ shapes and edge cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,window", [(32, 64), (64, 128), (128, 256), (256, 512)])
def test_chunk_sizes_ragged(dtype, chunk, window):
    n = 4 * window + chunk + 37                   # several absorptions and a ragged tail
    w = small(dtype, chunk=chunk, window=window, n_tokens=n, heads=3 if chunk < 256 else 2)
    print(f"case: {dtype} C={chunk} W={window} n={n}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, out, slot, kind, state, label=f"C{chunk}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 127, 200])
def test_short_and_window_covering_inputs(dtype, n):
    w = small(dtype, n_tokens=n, heads=2)
    print(f"case: {dtype} short n={n}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in range(w.seqs):
        oracle_check(w, inp, s, n, out, slot, kind, None, label="short")


def test_window_covers_sequence_is_plain_causal_attention():
    w = small("f32", n_tokens=300, window=320, heads=2)
    print("case: W >= N, fp32", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    assert np.all(kind == O.KIND_NONE)
    for s in range(2):
        oracle_check(w, inp, s, 300, out, slot, kind, None, label="W>=N")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk,window", [(64, 128), (128, 256)])
def test_given_softmax_scale(dtype, chunk, window):
    w = small(dtype, chunk=chunk, window=window, n_tokens=3 * window + chunk + 9, softmax_scale=0.21)
    print(f"case: softmax scale 0.21 {dtype} C={chunk}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in range(w.seqs):
        oracle_check(w, inp, s, w.n_tokens, out, slot, kind, state, label="softmax scale")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_everything(dtype):
    w = small(dtype, sched="fixed", max_slots=100000, n_tokens=900)
    print(f"case: append everything {dtype}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    assert np.all(kind[:, :900 - 192] != O.KIND_MERGE)
    for s in range(w.seqs):
        oracle_check(w, inp, s, 900, out, slot, kind, state, label="append-all")


@pytest.mark.parametrize("chunk,window", [(128, 256), (256, 512)])
def test_state_past_the_lds_version_list(chunk, window):
    """Largest states: every absorbed token appended until a snapshot holds more
    than 8192 rows, past what the staged attention keeps in LDS (those chunks
    take the register-staged bf16 kernel) and past the scan's LDS version list
    (index lists in global memory, one scan workgroup per sequence)."""
    w = small("bf16", heads=2, sched="fixed", max_slots=100000, n_tokens=9472, chunk=chunk, window=window)
    print(f"case: append everything to > 8192 rows, C {chunk}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    absorbed = w.n_tokens - window - chunk
    assert np.all(kind[:, :4] == O.KIND_SINK) and np.all(kind[:, 4:absorbed] == O.KIND_APPEND)
    assert int(state["n_rows"].min()) == absorbed > 8192
    for s in range(w.seqs):
        oracle_check(w, inp, s, w.n_tokens, out, slot, kind, state, label="rows>8192")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("logit", [-1e4, 1e4])
def test_gate_extremes(dtype, logit):
    w = small(dtype, n_tokens=800)
    print(f"case: gate logits {logit} {dtype}", flush=True)
    inp = make_inputs(w)
    inp.gate_logits.fill_(logit)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in range(w.seqs):
        oracle_check(w, inp, s, 800, out, slot, kind, state, label="gate")
    if logit < 0:
        # closed gate: every row keeps its creator's key exactly
        ks = state["key_sum"].cpu().numpy()
        for s in range(w.seqs):
            creators = {int(slot[s, t]): t for t in range(800) if kind[s, t] in (O.KIND_SINK, O.KIND_APPEND)}
            for r, t in creators.items():
                np.testing.assert_array_equal(ks[s, r], inp.k[s, t, 32:].float().numpy())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tie_rules(dtype):
    # Chunk 0 (positions 0-31) is appended whole: rows = unit keys e_t, except row 5 = e_3 (a duplicate
    # of row 3).  Chunk 1 may append one row: token 36 (all -0.5) is the only one with negative
    # surprise, so it is appended.  Token 32 = e_3 ties rows 3 and 5 -> lower row 3.  Token 33 (all
    # 0.5) has the same cosine to every unit row -> row 0.  Token 34 (zero key) has cosine 0 to every
    # candidate -> row 0.
    w = small(dtype, chunk=32, window=32, n_sinks=0, sched="fixed", max_slots=33, n_tokens=160, heads=1)
    print(f"case: tie rules {dtype}", flush=True)
    inp = make_inputs(w)
    k = torch.zeros(1, 160, 64)
    e = torch.eye(32)
    for t in range(32):
        k[0, t, 32:] = e[t]
    k[0, 5, 32:] = e[3]
    k[0, 32, 32:] = e[3]
    k[0, 33, 32:] = 0.5
    k[0, 34, 32:] = 0.0
    for t in range(35, 160):
        k[0, t, 32:] = e[(t * 7) % 32]
    k[0, 36, 32:] = -0.5
    inp.k = k.to(inp.k.dtype)
    out, slot, kind, state, _ = run_prefill(w, inp)
    assert kind[0, 36] == O.KIND_APPEND and slot[0, 36] == 32
    assert kind[0, 32] == O.KIND_MERGE and slot[0, 32] == 3
    assert kind[0, 33] == O.KIND_MERGE and slot[0, 33] == 0
    assert kind[0, 34] == O.KIND_MERGE and slot[0, 34] == 0
    oracle_check(w, inp, 0, 160, out, slot, kind, state, label="ties")


@pytest.mark.parametrize("ns", [0, 64])
def test_sink_counts(ns):
    w = small("bf16", n_sinks=ns, n_tokens=900, alpha=12)
    print(f"case: n_sinks={ns}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    assert int((kind[0] == O.KIND_SINK).sum()) == ns
    for s in range(w.seqs):
        oracle_check(w, inp, s, 900, out, slot, kind, state, label="sinks")


@pytest.mark.parametrize("bh", [1, 3, 8, 24])
def test_sequence_counts(bh):
    w = small("bf16", heads=bh, n_tokens=700)
    print(f"case: {bh} sequences", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, _ = run_prefill(w, inp)
    for s in sorted({0, bh - 1}):
        oracle_check(w, inp, s, 700, out, slot, kind, state, label=f"bh{bh}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_prefill_calls(dtype):
    w = small(dtype, n_tokens=1100)
    print(f"case: prefill split into calls {dtype}", flush=True)
    inp = make_inputs(w)
    one = run_prefill(w, inp)
    many = run_prefill(w, inp, splits=[64, 320, 704])
    np.testing.assert_array_equal(one[1], many[1])
    np.testing.assert_array_equal(one[2], many[2])
    assert check_outputs(dtype, many[0], one[0])[0]
    for s in range(w.seqs):
        oracle_check(w, inp, s, 1100, many[0], many[1], many[2], many[3], label="split")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_snapshots_match_oracle_read_form(dtype):
    w = small(dtype, n_tokens=1000)
    print(f"case: snapshots {dtype}", flush=True)
    inp = make_inputs(w)
    out, slot, kind, state, st = run_prefill(w, inp)
    p = O.Params.of(w)
    for s in range(w.seqs):
        res = O.prefill(*seq_arrays(inp, s, 1000), p, forced=forced_map(slot[s], kind[s]), keep_snapshots=True)
        for j in (0, 3, len(res.snapshots) - 1):
            kr, vr, rr = st.snapshot(j)
            kh, vh = O.read_form(res.snapshots[j], p)
            gk = kr[s].double().cpu().numpy()
            gv = vr[s].double().cpu().numpy()
            np.testing.assert_allclose(rr[s].double().cpu().numpy(), np.linalg.norm(vh, axis=1), rtol=1e-5)
            if dtype == "f32":
                assert np.max(np.abs(gk - kh[:, 32:])) <= 1e-5 * max(1.0, np.abs(kh).max())
                assert np.max(np.abs(gv - vh)) <= 1e-5 * max(1.0, np.abs(vh).max())
            else:
                # fp16 keys (|k| <= sqrt(31) < 8: half ulp <= 2^-8); bf16 values: half ulp
                # <= 2^-8 of the value, plus the fp32 sums' own error
                assert np.max(np.abs(gk - kh[:, 32:])) <= 2 ** -8 + 1e-5
                assert np.all(np.abs(gv - vh) <= 2 ** -8 * np.abs(vh) + 1e-5 * np.abs(vh).max())


def test_error_paths_leave_state_usable():
    w = small("bf16", n_tokens=300, heads=2)
    print("case: error paths", flush=True)
    inp = make_inputs(w, n_total=400)
    cfg = KvmConfig.of(w, max_tokens=400)
    cfg.batch, cfg.heads = 2, 1
    st = KvmState(cfg)
    q, k, v, g = to_gpu(inp, 0, 128)
    st.prefill(q, k, v, g)
    q1, k1, v1, g1 = to_gpu(inp, 128, 129)
    st.decode_step(q1[:, 0].contiguous(), k1[:, 0].contiguous(), v1[:, 0].contiguous(), g1[:, 0].contiguous())
    q2, k2, v2, g2 = to_gpu(inp, 129, 193)
    with pytest.raises(KvmError) as e:
        st.prefill(q2, k2, v2, g2)                # position 129 is not chunk-aligned
    assert e.value.status == KVM_E_STATE
    assert st.info()["position"] == 129
    big = to_gpu(inp, 0, 300)
    with pytest.raises(KvmError) as e:
        st.prefill(*big)
    assert e.value.status in (KVM_E_STATE, KVM_E_CAPACITY)
    with pytest.raises(TypeError):
        st.decode_step(q1[:, 0].float().contiguous(), k1[:, 0].contiguous(), v1[:, 0].contiguous(), g1[:, 0].contiguous())
    out = st.decode_step(q2[:, 0].contiguous(), k2[:, 0].contiguous(), v2[:, 0].contiguous(), g2[:, 0].contiguous())
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert st.info()["position"] == 130 and st.info()["poisoned"] == 0


def test_profile_mask_records_selected_phases():
    w = small("bf16", chunk=128, window=256, n_tokens=2000, heads=2)
    print("case: profile mask", flush=True)
    inp = make_inputs(w)
    cfg = KvmConfig.of(w, max_tokens=2000)
    cfg.batch, cfg.heads = 2, 1
    st = KvmState(cfg)
    q, k, v, g = to_gpu(inp)
    st.profile(2)                       # attention launches only
    st.prefill(q, k, v, g)
    p = st.profile_read()
    assert p["attn_launches"] >= 1 and p["attn_ms"] > 0
    assert p["scan_launches"] == 0 and p["ring_launches"] == 0 and p["prep_launches"] == 0
    with pytest.raises(KvmError):
        st.profile(64)


def test_scan_row_partition_is_invisible():
    """The absorption scan splits a sequence's rows over 1, 2, 4 or 8 workgroups by how many
    sequences share the GPU; the state and outputs of a sequence must not depend on it."""
    w = small("bf16", chunk=128, window=256, n_tokens=2048 + 77, heads=1, alpha=8, n_clusters=64)
    ref = None
    seen = set()
    for nseq in (4, 32, 64, 128):
        print(f"case: partition invariance, {nseq} sequences", flush=True)
        inp = make_inputs(w, seqs=range(nseq))
        out, slot, kind, state, st = run_prefill(w, inp)
        groups = st.info()["scan_groups"]
        seen.add(groups)
        got = (out[:4], slot[:4], kind[:4], {k: state[k][:4].cpu() for k in ("key_sum", "val_sum", "count", "rho",
                                                                           "key_read", "val_read")})
        if ref is None:
            ref = got
            continue
        assert np.array_equal(ref[0], got[0]), f"outputs differ ({groups} vs first)"
        assert np.array_equal(ref[1], got[1]) and np.array_equal(ref[2], got[2]), "decisions differ"
        for key in ref[3]:
            assert torch.equal(ref[3][key], got[3][key]), key
    assert seen == {8, 4, 2, 1}, seen


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_serial_prefill_matches_overlapped(dtype):
    """KVM_FLAG_SERIAL_PREFILL (every absorption, then all the attention, on one stream) gives the
    default overlapped prefill's results bit for bit."""
    w = small(dtype, chunk=128, window=256, n_tokens=3000 + 11, heads=4)
    print(f"case: serial vs overlapped prefill, {dtype}", flush=True)
    inp = make_inputs(w)
    res = []
    for serial in (False, True):
        cfg = KvmConfig.of(w, max_tokens=w.n_tokens, trace=True)
        cfg.batch, cfg.heads = w.seqs, 1
        cfg.serial_prefill = serial
        st = KvmState(cfg)
        q, k, v, g = to_gpu(inp, 0, w.n_tokens)
        out = st.prefill(q, k, v, g)
        state = st.read(trace=True)
        torch.cuda.synchronize()
        st.check()
        res.append((out.cpu(), {k_: t.cpu() for k_, t in state.items() if torch.is_tensor(t)}))
    assert torch.equal(res[0][0], res[1][0])
    for key in ("key_sum", "val_sum", "count", "rho", "key_read", "val_read", "trace_slot", "trace_kind"):
        assert torch.equal(res[0][1][key], res[1][1][key]), key
