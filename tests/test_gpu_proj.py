"""GPU parity of the projections around the layer (kvm_project_in / kvm_project_out) against
the oracle (needs an MI355X; marked gpu), and of the whole block x -> projections -> layer ->
output projection against the oracle's chain under the GPU's decisions.

Bars: outputs stored in bf16 (q, k, v, y on the bf16 path) as the layer's bf16 output bar
(per row max |diff| <= 2e-2 * max(RMS(ref), RMS(ref row)), RMS(diff) <= 2e-2 * RMS(ref));
fp32 outputs (everything on the fp32 path, the gate logits always): max |diff| <=
1e-4 * max(1, max |ref|) (fp32 accumulation of exactly represented products).
"""
import numpy as np
import pytest
import torch

import oracle.kvm_oracle as O
import oracle.kvm_oracle_proj as P
from compressed_kv_state_amd import KvmConfig, KvmState, project_in, project_out
from kvm_inputs import LayerConfig
from tests.parity import check_outputs, forced_map, record

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def bar(dtype, got, want, label):
    got = np.asarray(got, dtype=np.float64).reshape(-1, want.shape[-1] if want.ndim > 1 else 1)
    want = np.asarray(want, dtype=np.float64).reshape(got.shape)
    err = np.abs(got - want)
    if dtype == "f32":
        bound = 1e-4 * max(1.0, float(np.abs(want).max()))
        record(label, None, float(err.max()) / max(1.0, float(np.abs(want).max())), None)
        assert err.max() <= bound, (label, float(err.max()), bound)
    else:
        rms = max(float(np.sqrt(np.mean(want ** 2))), 1e-30)
        ref = np.maximum(np.sqrt(np.mean(want ** 2, axis=1)), rms)
        worst = float(np.max(err.max(axis=1) / ref))
        rel = float(np.sqrt(np.mean(err ** 2)) / rms)
        record(label, None, worst, rel)
        assert worst <= 2e-2 and rel <= 2e-2, (label, worst, rel)


def draw(B, H, n, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    D = H * 64
    x = torch.randn(B, n, D, generator=g).to(TD[dtype])
    w_in = (torch.randn(3 * D + H, D, generator=g) / D ** 0.5).to(TD[dtype])
    b_gate = torch.randn(H, generator=g)
    w_out = (torch.randn(D, D, generator=g) / D ** 0.5).to(TD[dtype])
    return x, w_in, b_gate, w_out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,H,n", [(1, 1, 1), (2, 3, 257), (1, 12, 130), (2, 16, 640), (3, 2, 1000)])
def test_projections_match_oracle(dtype, B, H, n):
    print(f"case: projections {dtype} B={B} H={H} n={n}", flush=True)
    x, w_in, b_gate, w_out = draw(B, H, n, dtype, 100 + B * 10 + H + n)
    cfg = KvmConfig(batch=B, heads=H, chunk=64, window=128, n_sinks=4, sched="sqrt", alpha=6, max_tokens=max(n, 1),
                    dtype=dtype)
    q, k, v, gl = project_in(cfg, x.cuda(), w_in.cuda(), b_gate.cuda())
    o = torch.randn(B * H, n, 64, generator=torch.Generator().manual_seed(n)).to(TD[dtype])
    y = project_out(cfg, o.cuda(), w_out.cuda())
    torch.cuda.synchronize()
    wq, wk, wv, wg = P.project_in(x.double().numpy(), w_in.double().numpy(), b_gate.double().numpy(), H)
    wy = P.project_out(o.double().numpy(), w_out.double().numpy(), B)
    for name, got, want in (("q", q, wq), ("k", k, wk), ("v", v, wv), ("y", y, wy)):
        bar(dtype, got.double().cpu().numpy(), want, f"projection {name} {dtype}")
    bar("f32", gl.double().cpu().numpy(), wg, f"projection gate logits {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_matches_oracle_chain(dtype):
    """x -> q, k, v, gate logits -> KVM layer -> output projection, against the oracle's chain
    fed the GPU's own projected inputs (so the layer's decisions are compared on the same
    inputs) and, separately, the oracle's projections."""
    B, H, n = 1, 2, 900
    print(f"case: block chain {dtype}", flush=True)
    x, w_in, b_gate, w_out = draw(B, H, n, dtype, 7)
    w = LayerConfig(name="block", batch=B, heads=H, n_tokens=n, chunk=64, window=128, n_sinks=4, sched="sqrt",
                    alpha=6, dtype=dtype)
    cfg = KvmConfig.of(w, max_tokens=n, trace=True)
    q, k, v, gl = project_in(cfg, x.cuda(), w_in.cuda(), b_gate.cuda())
    st = KvmState(cfg)
    o = st.prefill(q, k, v, gl)
    y = project_out(cfg, o, w_out.cuda())
    state = st.read(trace=True)
    torch.cuda.synchronize()
    slot = state["trace_slot"].long().cpu().numpy()
    kind = state["trace_kind"].long().cpu().numpy()
    kind[kind == 255] = O.KIND_NONE
    # the oracle's projections agree with the GPU's (projection bar) ...
    wq, wk, wv, wg = P.project_in(x.double().numpy(), w_in.double().numpy(), b_gate.double().numpy(), H)
    bar(dtype, q.double().cpu().numpy(), wq, "block q")
    # ... and the oracle's layer on the GPU's projected inputs, under the GPU's decisions, then the
    # oracle's output projection, gives y
    qn, kn, vn, gn = (t.double().cpu().numpy() for t in (q, k, v, gl))
    p = O.Params.of(w)
    outs = np.stack([O.prefill(qn[s], kn[s], vn[s], gn[s], p, forced=forced_map(slot[s], kind[s])).out
                     for s in range(B * H)])
    ok, worst, bound, rel = check_outputs(dtype, o.double().cpu().numpy(), outs)
    assert ok, (worst, bound, rel)
    wy = P.project_out(outs, w_out.double().numpy(), B)
    bar(dtype, y.double().cpu().numpy(), wy, "block y")
