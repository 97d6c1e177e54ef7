"""GPU tests of sequences at their own positions (needs an MI355X; marked gpu): ragged prefill,
ragged decode steps and per-sequence slot resets, against the oracle (teacher-forced by the GPU's
decisions) and bit for bit against each sequence run alone in a state of its own.
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
from compressed_kv_state_amd import KVM_E_STATE, KvmConfig, KvmError, KvmState
from kvm_inputs import LayerConfig, make_inputs
from tests.parity import forced_map, oracle_check

pytestmark = pytest.mark.gpu


def layer(dtype, chunk, window, seqs, n):
    return LayerConfig(name="ragged", batch=1, heads=seqs, n_tokens=n, chunk=chunk, window=window, n_sinks=4,
                       sched="sqrt", alpha=6, dtype=dtype, key_gen="clustered", n_clusters=24, index=41)


def new_state(w, seqs, n_max):
    cfg = KvmConfig.of(w, max_tokens=n_max, trace=True)
    cfg.batch, cfg.heads = seqs, 1
    return KvmState(cfg)


def token_step(inp, pos, s_list, dev="cuda"):
    """Decode inputs [S, 64] holding, for each sequence s, its token at position pos[s]."""
    S = inp.q.shape[0]
    idx = torch.tensor([min(p, inp.q.shape[1] - 1) for p in pos])
    ar = torch.arange(S)
    return tuple(t[ar, idx].contiguous().to(dev) for t in (inp.q, inp.k, inp.v, inp.gate_logits))


@pytest.mark.parametrize("dtype,chunk,window", [("bf16", 128, 256), ("f32", 64, 128), ("bf16", 64, 128)])
def test_ragged_prefill_and_decode(dtype, chunk, window):
    lengths = [4 * chunk, 2 * chunk, 0, 5 * chunk, 3 * chunk]
    steps = 2 * chunk + 19
    S = len(lengths)
    n_max_total = max(lengths) + steps + 1
    w = layer(dtype, chunk, window, S, n_max_total)
    print(f"case: ragged {dtype} C={chunk} lengths {lengths}", flush=True)
    inp = make_inputs(w)
    st = new_state(w, S, n_max_total)
    n_max = max(lengths)
    q, k, v, g = (t[:, :n_max].contiguous().cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
    out = st.prefill_ragged(lengths, q, k, v, g)
    assert st.positions() == lengths and st.info()["per_sequence"] == 1
    with pytest.raises(KvmError) as e:                   # the uniform call refuses
        st.prefill(q, k, v, g)
    assert e.value.status == KVM_E_STATE
    outs = [[out[s, :lengths[s]].cpu()] for s in range(S)]
    pos = list(lengths)
    rng = np.random.default_rng(5)
    for i in range(steps):
        active = [bool(rng.random() < 0.8) or s == 3 for s in range(S)]
        qs, ks, vs, gs = token_step(inp, pos, range(S))
        o = st.decode_step_ragged(active, qs, ks, vs, gs)
        for s in range(S):
            if active[s]:
                outs[s].append(o[s:s + 1].cpu())
                pos[s] += 1
    assert st.positions() == pos
    state = st.read(trace=True)
    torch.cuda.synchronize()
    st.check()
    slot = state["trace_slot"].long().cpu().numpy()
    kind = state["trace_kind"].long().cpu().numpy()
    kind[kind == 255] = O.KIND_NONE
    full = [torch.cat(o_, 0).double().numpy() for o_ in outs]
    # each sequence against the oracle over its own tokens
    for s in range(S):
        n = pos[s]
        if n == 0:
            continue
        out_s = np.zeros((S, n, 64))
        out_s[s] = full[s]
        sl = slot.copy()
        kd = kind.copy()
        kd[s, n:] = O.KIND_NONE
        oracle_check(w.replace(n_tokens=n), inp, s, n, out_s, sl, kd, None, label=f"ragged {dtype}")
        assert int(state["n_rows"][s]) == (O.schedule(max(0, -(-n // chunk) - window // chunk - 1),
                                                      O.Params.of(w))[-1][2] if -(-n // chunk) - window // chunk - 1 > 0
                                           else 0)
    # and bit for bit against two sequences run alone (same token stream, one sequence per state)
    for s in (0, 3):
        alone = new_state(w, 1, n_max_total)
        n0 = lengths[s]
        a_out = [alone.prefill(*(t[s:s + 1, :n0].contiguous().cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits)))[0].cpu()]
        for p in range(n0, pos[s]):
            a_out.append(alone.decode_step(*(t[s:s + 1, p].contiguous().cuda() for t in (inp.q, inp.k, inp.v,
                                                                                         inp.gate_logits)))[0:1].cpu())
        torch.cuda.synchronize()
        assert np.array_equal(torch.cat(a_out, 0).double().numpy(), full[s]), f"sequence {s} differs from alone"


def test_slot_reset_takes_a_new_request():
    """Continuous batching: sequence slot 1 finishes, is reset and takes a new request (prefill at
    position 0) while slot 0 keeps decoding; the new request equals a fresh state bit for bit."""
    dtype, chunk, window = "bf16", 128, 256
    w = layer(dtype, chunk, window, 2, 2048)
    print("case: slot reset", flush=True)
    inp = make_inputs(w)
    other = make_inputs(w.replace(index=42))
    st = new_state(w, 2, 2048)
    q, k, v, g = (t[:, :768].contiguous().cuda() for t in (inp.q, inp.k, inp.v, inp.gate_logits))
    st.prefill(q, k, v, g)
    st.reset_sequence(1)
    assert st.positions() == [768, 0]
    # the new request of slot 1: 512 tokens of `other`, padded to 512 rows (slot 0 takes none)
    nq = torch.zeros(2, 512, 64, dtype=q.dtype)
    nq[1] = other.q[1, :512]
    nk = torch.zeros_like(nq); nk[1] = other.k[1, :512]
    nv = torch.zeros_like(nq); nv[1] = other.v[1, :512]
    ng = torch.zeros(2, 512); ng[1] = other.gate_logits[1, :512]
    out = st.prefill_ragged([0, 512], nq.cuda(), nk.cuda(), nv.cuda(), ng.cuda())
    res = [out[1].cpu()]
    pos = [768, 512]
    for i in range(300):
        qs = torch.stack([inp.q[0, pos[0]], other.q[1, pos[1]]]).contiguous().cuda()
        ks = torch.stack([inp.k[0, pos[0]], other.k[1, pos[1]]]).contiguous().cuda()
        vs = torch.stack([inp.v[0, pos[0]], other.v[1, pos[1]]]).contiguous().cuda()
        gs = torch.stack([inp.gate_logits[0, pos[0]], other.gate_logits[1, pos[1]]]).contiguous().cuda()
        o = st.decode_step_ragged([True, True], qs, ks, vs, gs)
        res.append(o[1:2].cpu())
        pos = [pos[0] + 1, pos[1] + 1]
    torch.cuda.synchronize()
    fresh = new_state(w, 1, 2048)
    f = [fresh.prefill(*(t[1:2, :512].contiguous().cuda() for t in (other.q, other.k, other.v, other.gate_logits)))[0].cpu()]
    for p in range(512, 812):
        f.append(fresh.decode_step(*(t[1:2, p].contiguous().cuda() for t in (other.q, other.k, other.v,
                                                                              other.gate_logits)))[0:1].cpu())
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(res, 0), torch.cat(f, 0))
