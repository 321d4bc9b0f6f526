"""The no-allocation MoE entry point (moe_expert_ffn_noalloc) against the
workspace entry point (moe_expert_ffn), through the C ABI: two calls in a
row on the library's shared device scratch, the second with a smaller
layer, each bit-identical to moe_expert_ffn on the same inputs (and within
the oracle's bound); a layer above the scratch's stated maximum is
rejected before anything is launched."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import moe as OM

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _layer(fmt, e, h, i, seed):
    gu, dn, wg, wu, wd = [], [], [], [], []
    for j in range(e + 1):
        g = workloads.student_t_weights(i, h, seed, 3 * j)
        u = workloads.student_t_weights(i, h, seed, 3 * j + 1)
        d = workloads.student_t_weights(h, i, seed, 3 * j + 2)
        b_gu, b_dn = OF.quantize(fmt, OM.interleave_gate_up(g, u)), OF.quantize(fmt, d)
        gu.append(OF.pack(fmt, b_gu))
        dn.append(OF.pack(fmt, b_dn))
        deq = OF.dequant(fmt, b_gu)
        wg.append(deq[0::2])
        wu.append(deq[1::2])
        wd.append(OF.dequant(fmt, b_dn))
    return _dev(np.concatenate(gu)), _dev(np.concatenate(dn)), (wg, wu, wd)


def _both(fmt, e, h, i, top_k, t, seed):
    gu, dn, (wg, wu, wd) = _layer(fmt, e, h, i, seed)
    x = workloads.normal((t, h), seed, 1)
    res = workloads.normal((t, h), seed, 2)
    logits = workloads.normal((t, e), seed, 3)
    s = workloads.normal((t,), seed, 4)
    assert np.all(OM.route_margin(logits, top_k) > 1e-6), "near-tied route; change the seed"
    args = (fmt, gu, dn, e, h, i, top_k, _dev(x), _dev(res), _dev(logits), _dev(s), t)
    ws_bytes = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    assert 0 < ws_bytes <= qg.QG_MOE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out_ws = torch.full((t, h), float("nan"), device="cuda")
    out_na = torch.full((t, h), float("nan"), device="cuda")
    qg.moe_expert_ffn(*args, out_ws, ws, ws_bytes)
    qg.moe_expert_ffn_noalloc(*args, out_na)
    torch.cuda.synchronize()
    ref = OM.moe_ref(wg, wu, wd, x, res, logits, s, top_k)
    tol = OM.out_tolerance(wg, wu, wd, x, res, ref)
    got = out_na.cpu().numpy()
    assert np.all(np.abs(got.astype(np.float64) - ref["out"]) <= tol)
    return out_ws, out_na


@pytest.mark.parametrize("fmt", ["q4_k", "q2_k"])
def test_noalloc_matches_workspace_entry_point_twice(fmt):
    # first call: the larger layer; second: a smaller one on the same scratch,
    # which still holds the first call's records and rows
    big = _both(fmt, 24, 1024, 512, 4, 8, seed=71)
    small = _both(fmt, 9, 512, 256, 2, 3, seed=72)
    for out_ws, out_na in (big, small):
        assert torch.equal(out_ws.view(torch.int32), out_na.view(torch.int32))


def test_noalloc_rejects_layers_above_the_scratch():
    # T = 8, top_k = 8: 68 h rows of 2 * I floats; I = 4096 needs ~2.2 MB
    e, h, i, t, top_k = 16, 256, 4096, 8, 8
    need = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    assert need > qg.QG_MOE_NOALLOC_SCRATCH_BYTES
    gu = torch.empty((e + 1) * qg.qg_packed_size("q4_k", 2 * i, h), dtype=torch.uint8, device="cuda")
    dn = torch.empty((e + 1) * qg.qg_packed_size("q4_k", h, i), dtype=torch.uint8, device="cuda")
    act = torch.zeros((t, h), device="cuda")
    out = torch.zeros((t, h), device="cuda")
    with pytest.raises(qg.QGError) as info:
        qg.moe_expert_ffn_noalloc("q4_k", gu, dn, e, h, i, top_k, act, act, torch.zeros((t, e), device="cuda"),
                                  torch.zeros(t, device="cuda"), t, out)
    assert info.value.code == -4
    assert torch.equal(out, torch.zeros_like(out))  # nothing launched
