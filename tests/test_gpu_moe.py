"""GPU parity of the routed MoE expert layer (moe_expert_ffn) against the
oracle's moe_ref, through the C ABI.

Experts are oracle-quantized Student-t(5)*0.02 matrices; x, residual, router
and shared-gate logits are N(0,1).  Small layers use fully independent
experts; the full layer (512 experts + 1 shared, hidden 4096, intermediate
1024) writes real experts only into the slots the oracle's router selects and
fills every other slot with 0xFF bytes (fp16 NaN scales), so a kernel that
reads a wrong expert produces NaN."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import moe as OM
from oracle import norm as ON

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

KFORMATS = ["q4_k", "q2_k"]


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class Expert:
    """One expert: packed gate/up (2I x H, rows interleaved) and down (H x I)
    bytes, and the dequantized fp32 gate, up and down matrices."""

    def __init__(self, fmt, wg, wu, wd):
        gu = OF.quantize(fmt, OM.interleave_gate_up(wg, wu))
        dn = OF.quantize(fmt, wd)
        self.gu_packed = OF.pack(fmt, gu)
        self.dn_packed = OF.pack(fmt, dn)
        gu_deq = OF.dequant(fmt, gu)
        self.gate, self.up = gu_deq[0::2], gu_deq[1::2]
        self.down = OF.dequant(fmt, dn)


def random_expert(fmt, h, i, seed, e):
    return Expert(fmt, workloads.student_t_weights(i, h, seed, 3 * e),
                  workloads.student_t_weights(i, h, seed, 3 * e + 1),
                  workloads.student_t_weights(h, i, seed, 3 * e + 2))


class Layer:
    """Sequence-like views of the experts for moe_ref (index E = shared)."""

    def __init__(self, experts):
        self.experts = experts

    def view(self, attr):
        ex = self.experts

        class _V:
            def __len__(self):
                return len(ex)

            def __getitem__(self, j):
                return getattr(ex[j], attr)

        return _V()


def inputs(t, e, h, seed):
    x = workloads.normal((t, h), seed, 9001)
    residual = workloads.normal((t, h), seed, 9002)
    logits = workloads.normal((t, e), seed, 9003)
    s = workloads.normal((t,), seed, 9004)
    return x, residual, logits, s


def run_moe(fmt, gu_d, dn_d, e, h, i, top_k, x, residual, logits, s, flags=0, alias_residual=False):
    t = x.shape[0]
    x_d = dev(x)
    r_d = x_d if alias_residual else dev(residual)
    out = torch.full((t, h), float("nan"), device="cuda")
    ws_bytes = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qg.moe_expert_ffn(fmt, gu_d, dn_d, e, h, i, top_k, x_d, r_d, dev(logits), dev(s), t, out, ws, ws_bytes,
                      flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(out, layer, x, residual, logits, s, top_k, renorm, label):
    if top_k < logits.shape[1]:
        assert np.all(OM.route_margin(logits, top_k) > 1e-6), f"{label}: near-tied route; change the seed"
    wg, wu, wd = layer.view("gate"), layer.view("up"), layer.view("down")
    ref = OM.moe_ref(wg, wu, wd, x, residual, logits, s, top_k, renorm)
    tol = OM.out_tolerance(wg, wu, wd, x, residual, ref)
    err = np.abs(out.astype(np.float64) - ref["out"])
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert np.all(err <= tol), f"{label}: |err|/tol = {err[worst] / tol[worst]:.3g} at {worst}"
    return ref


def small_layer(fmt, e, h, i, seed):
    experts = [random_expert(fmt, h, i, seed, j) for j in range(e + 1)]
    gu = np.concatenate([ex.gu_packed for ex in experts])
    dn = np.concatenate([ex.dn_packed for ex in experts])
    assert gu.size == (e + 1) * qg.qg_packed_size(fmt, 2 * i, h)
    assert dn.size == (e + 1) * qg.qg_packed_size(fmt, h, i)
    return Layer(experts), dev(gu), dev(dn)


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("renorm", [False, True])
def test_moe_small(fmt, t, renorm):
    e, h, i, top_k = 16, 512, 256, 4
    layer, gu, dn = small_layer(fmt, e, h, i, seed=11)
    x, residual, logits, s = inputs(t, e, h, seed=100 + t)
    flags = qg.QG_MOE_RENORM if renorm else 0
    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s, flags)
    check(out, layer, x, residual, logits, s, top_k, renorm, f"{fmt} T={t} renorm={renorm}")


def workspace_stages(ws, t, e, h, i, top_k):
    """(hsel [T][K+1] int32, h rows as a function of (t, k)) read back from a
    finished call's workspace at the offsets the library reports."""
    hs_off, h_off = qg.moe_expert_ffn_workspace_layout(t, e, h, i, top_k)
    raw = ws.cpu().numpy()
    hsel = raw[hs_off:hs_off + 4 * t * (top_k + 1)].view(np.int32).reshape(t, top_k + 1).copy()
    rows = raw[h_off:h_off + (raw.size - h_off) // 4 * 4].view(np.float32)
    return hsel, (lambda tt, k: rows[hsel[tt, k] * i:(hsel[tt, k] + 1) * i].astype(np.float64))


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 3, 8])
def test_moe_stagewise_h_then_teacher_forced_down(fmt, t):
    """Stage-wise check (EPM README, section "正確性"): the SwiGLU intermediate
    h of every (token, slot) is read from the workspace and checked on its own
    against the oracle within the gate/up bound; then the GPU's h is fed to the
    oracle's down projection and combine (teacher forcing), and the GPU's
    output must match that within the down + combine bound alone."""
    e, h, i, top_k = 16, 512, 256, 4
    layer, gu, dn = small_layer(fmt, e, h, i, seed=21)
    x, residual, logits, s = inputs(t, e, h, seed=300 + t)
    assert np.all(OM.route_margin(logits, top_k) > 1e-6), "near-tied route; change the seed"
    ws_bytes = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.full((t, h), float("nan"), device="cuda")
    qg.moe_expert_ffn(fmt, gu, dn, e, h, i, top_k, dev(x), dev(residual), dev(logits), dev(s), t, out, ws,
                      ws_bytes)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    hsel, h_row = workspace_stages(ws, t, e, h, i, top_k)
    assert len(set(hsel.ravel().tolist())) == t * (top_k + 1), "every (token, slot) has its own h row"
    wg, wu, wd = layer.view("gate"), layer.view("up"), layer.view("down")
    ref = OM.moe_ref(wg, wu, wd, x, residual, logits, s, top_k)
    for tt in range(t):
        slots = list(ref["ids"][tt]) + [e]
        coef = list(ref["weights"][tt]) + [float(ref["sigma"][tt])]
        out_tf = residual[tt].astype(np.float64).copy()
        tol = OM.COMBINE_REL * np.abs(residual[tt].astype(np.float64))
        for k, ex in enumerate(slots):
            hg = h_row(tt, k)
            dh = OM.h_tolerance(wg[ex], wu[ex], x[tt:tt + 1])[0]
            err = np.abs(hg - ref["h"][tt, k])
            assert np.all(err <= dh), f"h of token {tt} slot {k}: |err|/tol = {np.max(err / dh):.3g}"
            d64 = np.asarray(wd[ex], np.float32).astype(np.float64)
            o_tf = d64 @ hg
            out_tf += coef[k] * o_tf
            tol += coef[k] * OM.o_tolerance(wd[ex], hg[None], np.zeros((1, i)))[0] + OM.COMBINE_REL * coef[k] * np.abs(o_tf)
        err = np.abs(out[tt] - out_tf)
        assert np.all(err <= tol), f"teacher-forced token {tt}: |err|/tol = {np.max(err / tol):.3g}"


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("e,top_k,t", [(4, 4, 5), (9, 1, 8), (12, 8, 7), (1, 1, 3)])
def test_moe_topk_edges(fmt, e, top_k, t):
    """Every expert selected (top_k = E), a single pick, the widest top_k, and a
    single-expert layer; odd T leaves a one-token shared-expert item."""
    h, i = 256, 512
    layer, gu, dn = small_layer(fmt, e, h, i, seed=12)
    x, residual, logits, s = inputs(t, e, h, seed=200 + e)
    if e == 1:
        logits = np.zeros_like(logits)  # one expert: p = 1 whatever the logit
    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    check(out, layer, x, residual, logits, s, top_k, False, f"{fmt} E={e} top_k={top_k} T={t}")


@pytest.mark.parametrize("fmt", KFORMATS)
def test_moe_shared_routes(fmt):
    """All 8 tokens route to the same 4 experts, in different orders, so every
    expert item carries two tokens; a -inf shared logit turns the shared
    expert off for one token and +inf fully on for another; residual aliases x."""
    e, h, i, top_k, t = 10, 512, 256, 4, 8
    layer, gu, dn = small_layer(fmt, e, h, i, seed=13)
    x, _, logits, s = inputs(t, e, h, seed=300)
    logits = logits.copy()
    favourites = [7, 2, 9, 4]
    for tok in range(t):
        for rank, ex in enumerate(np.roll(favourites, tok)):
            logits[tok, ex] = 6.0 - 0.5 * rank
    s = s.copy()
    s[1], s[6] = -np.inf, np.inf
    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, x, logits, s, alias_residual=True)
    ref = check(out, layer, x, x, logits, s, top_k, False, f"{fmt} shared routes")
    assert all(set(ref["ids"][tok]) == set(favourites) for tok in range(t))


@pytest.mark.parametrize("fmt", KFORMATS)
def test_moe_route_ties_nan_inf_zero(fmt):
    """Exact ties (lower expert index first), NaN logits (counted as -inf),
    -inf logits and signed zeros: the routed output equals the oracle's, whose
    stable sort settles ties the same way."""
    e, h, i, top_k, t = 16, 256, 256, 4, 6
    layer, gu_d, dn_d = small_layer(fmt, e, h, i, 31)
    x, residual, logits, s = inputs(t, e, h, 31)
    logits[0, :] = 0.5                                            # all tied
    logits[1, :] = -1.0
    logits[1, [2, 9, 11]] = 1.0                                   # three tied leaders
    logits[1, [0, 5]] = np.nan
    logits[2, :] = -1.0
    logits[2, [3, 9]] = -0.0
    logits[2, [7]] = 0.0                                          # signed zeros tie
    logits[3, :] = -np.inf
    logits[3, [4, 12]] = 0.25                                     # two finite, rest -inf
    logits[4, :] = np.nan
    logits[4, [1, 6, 8, 15]] = [0.1, 0.1, -0.3, 0.1]             # NaN elsewhere
    out = run_moe(fmt, gu_d, dn_d, e, h, i, top_k, x, residual, logits, s)
    wg, wu, wd = layer.view("gate"), layer.view("up"), layer.view("down")
    ref = OM.moe_ref(wg, wu, wd, x, residual, logits, s, top_k)
    tol = OM.out_tolerance(wg, wu, wd, x, residual, ref)
    err = np.abs(out.astype(np.float64) - ref["out"])
    assert np.all(err <= tol), f"|err|/tol = {np.max(err / tol):.3g}"


def test_moe_dominant_logit_matches_single_expert():
    """One dominant logit per token: the routed part reduces to that expert's
    forward with weight ~1, checked against expert_forward directly."""
    fmt, e, h, i, top_k, t = "q4_k", 8, 256, 256, 1, 2
    layer, gu, dn = small_layer(fmt, e, h, i, seed=14)
    x, residual, logits, _ = inputs(t, e, h, seed=400)
    logits = logits.copy()
    logits[0, 5] = logits[1, 3] = 60.0
    s = np.full((t,), -np.inf, np.float32)  # no shared expert
    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    check(out, layer, x, residual, logits, s, top_k, False, "dominant")
    for tok, ex in [(0, 5), (1, 3)]:
        ee = layer.experts[ex]
        _, _, _, o = OM.expert_forward(ee.gate, ee.up, ee.down, x[tok:tok + 1])
        np.testing.assert_allclose(out[tok], residual[tok] + o[0], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("e", [100, 1000, 4096])
def test_moe_many_experts(e):
    """Router sizes past 512 (more experts per lane in the route kernel, up to
    the 4096 limit); only the selected experts hold weights, every other slot
    is 0xFF (NaN scales)."""
    fmt, h, i, top_k, t = "q4_k", 256, 256, 8, 5
    x, residual, logits, s = inputs(t, e, h, seed=900 + e)
    ids, _, _ = OM.route(logits, top_k)
    used = sorted(set(ids.reshape(-1).tolist()) | {e})
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i, h), qg.qg_packed_size(fmt, h, i)
    gu = torch.full(((e + 1) * gu_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    dn = torch.full(((e + 1) * dn_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    experts = {}
    for ex in used:
        experts[ex] = random_expert(fmt, h, i, 17, ex)
        gu[ex * gu_sz:(ex + 1) * gu_sz].copy_(dev(experts[ex].gu_packed))
        dn[ex * dn_sz:(ex + 1) * dn_sz].copy_(dev(experts[ex].dn_packed))

    class Sparse:
        def __len__(self):
            return e + 1

        def __getitem__(self, j):
            # the oracle reads slot 0 for the intermediate width only
            return experts[j] if j in experts else experts[e]

    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    assert np.all(np.isfinite(out)), "a kernel read an unselected expert"
    check(out, Layer(Sparse()), x, residual, logits, s, top_k, False, f"E={e}")


def tie_logits(e, t=6):
    """Router logits with exact ties at large E: all equal; equal leaders
    that share a route-kernel lane (experts 5, 69, 133, ... are lane 5's) next
    to another lane's; signed zeros; -inf and NaN fill-ins; one random row
    whose three leaders tie."""
    lg = workloads.normal((t, e), 41, e).copy()
    lg[0, :] = 0.5
    lg[1, :] = -1.0
    lg[1, [5, 69, 133, 197, 261, 4, 68]] = 2.0
    lg[1, [0, 64]] = np.nan
    lg[2, :] = -1.0
    lg[2, [300, 7, 450]] = -0.0
    lg[2, [193]] = 0.0
    lg[3, :] = -np.inf
    lg[3, [511, 256]] = 0.25
    lg[4, :] = np.nan
    lg[4, [1, 6, 8, 15]] = [0.1, 0.1, -0.3, 0.1]
    lg[5, [10, 500, e - 1]] = 9.0
    return lg.astype(np.float32)


@pytest.mark.parametrize("e", [512, 4096])
def test_moe_route_ties_many_experts(e):
    """Ties settled by the lower expert index where each lane of the route
    kernel holds 8 or 64 experts; only the oracle's picks hold weights (every
    other slot is 0xFF, NaN scales), so a different pick shows as NaN."""
    fmt, h, i, top_k = "q4_k", 256, 256, 8
    lg = tie_logits(e)
    t = lg.shape[0]
    ids, _, _ = OM.route(lg, top_k)
    assert ids[1].tolist() == [4, 5, 68, 69, 133, 197, 261, 1]
    assert OM.route_margin(lg[5:6], top_k)[0] > 1e-6
    x, residual, _, s = inputs(t, e, h, seed=42)
    used = sorted(set(ids.reshape(-1).tolist()) | {e})
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i, h), qg.qg_packed_size(fmt, h, i)
    gu = torch.full(((e + 1) * gu_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    dn = torch.full(((e + 1) * dn_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    experts = {}
    for ex in used:
        experts[ex] = random_expert(fmt, h, i, 43, ex)
        gu[ex * gu_sz:(ex + 1) * gu_sz].copy_(dev(experts[ex].gu_packed))
        dn[ex * dn_sz:(ex + 1) * dn_sz].copy_(dev(experts[ex].dn_packed))

    class Sparse:
        def __len__(self):
            return e + 1

        def __getitem__(self, j):
            return experts[j] if j in experts else experts[e]

    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, lg, s)
    assert np.all(np.isfinite(out)), "a tie went to an expert the oracle did not pick"
    layer = Layer(Sparse())
    wg, wu, wd = layer.view("gate"), layer.view("up"), layer.view("down")
    ref = OM.moe_ref(wg, wu, wd, x, residual, lg, s, top_k)
    tol = OM.out_tolerance(wg, wu, wd, x, residual, ref)
    err = np.abs(out.astype(np.float64) - ref["out"])
    assert np.all(err <= tol), f"E={e}: |err|/tol = {np.max(err / tol):.3g}"


def test_moe_deterministic():
    fmt, e, h, i, top_k, t = "q2_k", 16, 512, 256, 4, 8
    layer, gu, dn = small_layer(fmt, e, h, i, seed=15)
    x, residual, logits, s = inputs(t, e, h, seed=500)
    a = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    b = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------- full layer

FULL_E, FULL_H, FULL_I, FULL_K = 512, 4096, 1024, 4


class PooledExperts:
    """Experts of the full layer, made on demand: each is a seeded row
    permutation of one Student-t(5)*0.02 pool matrix per role (i.i.d. rows, so
    each expert still has the workload's weight distribution), quantized by
    permuting the pool's quantized rows (quantization is row by row)."""

    def __init__(self, fmt, seed):
        self.fmt = fmt
        h, i = FULL_H, FULL_I
        gu_pool = OM.interleave_gate_up(workloads.student_t_weights(i, h, seed, 0),
                                        workloads.student_t_weights(i, h, seed, 1))
        self.gu_blk = OF.quantize(fmt, gu_pool)
        self.dn_blk = OF.quantize(fmt, workloads.student_t_weights(h, i, seed, 2))
        self.seed = seed
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            g = workloads.rng_for(self.seed, 1000 + e)
            # permute gate/up pairs together so rows 2i, 2i+1 stay one pair
            pairs = g.permutation(FULL_I)
            gu_rows = np.stack([2 * pairs, 2 * pairs + 1], axis=1).reshape(-1)
            dn_rows = g.permutation(FULL_H)
            gu = {k: v[gu_rows] for k, v in self.gu_blk.items()}
            dn = {k: v[dn_rows] for k, v in self.dn_blk.items()}
            ex = Expert.__new__(Expert)
            ex.gu_packed = OF.pack(self.fmt, gu)
            ex.dn_packed = OF.pack(self.fmt, dn)
            gu_deq = OF.dequant(self.fmt, gu)
            ex.gate, ex.up = gu_deq[0::2], gu_deq[1::2]
            ex.down = OF.dequant(self.fmt, dn)
            self.cache[e] = ex
        return self.cache[e]

    def __len__(self):
        return FULL_E + 1


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 4, 8])
def test_moe_full_layer(fmt, t):
    e, h, i, top_k = FULL_E, FULL_H, FULL_I, FULL_K
    x, residual, logits, s = inputs(t, e, h, seed=600 + t)
    ids, _, _ = OM.route(logits, top_k)
    used = sorted(set(ids.reshape(-1).tolist()) | {e})
    pool = PooledExperts(fmt, seed=21)
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i, h), qg.qg_packed_size(fmt, h, i)
    gu = torch.full(((e + 1) * gu_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    dn = torch.full(((e + 1) * dn_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    for ex in used:
        gu[ex * gu_sz:(ex + 1) * gu_sz].copy_(dev(pool[ex].gu_packed))
        dn[ex * dn_sz:(ex + 1) * dn_sz].copy_(dev(pool[ex].dn_packed))
    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    assert np.all(np.isfinite(out)), "a kernel read an unselected expert"
    check(out, Layer(pool), x, residual, logits, s, top_k, False, f"{fmt} full T={t}")



def test_moe_experts_past_4gib():
    """1024 experts at the full layer's sizes (gate/up array 4.8 GB): the
    router is steered to experts 1000-1023, whose gate/up rows lie past 2^32
    bytes, like the shared expert's (index 1024); unselected slots hold 0xFF
    (NaN scales)."""
    fmt, e, h, i, top_k, t = "q4_k", 1024, FULL_H, FULL_I, FULL_K, 2
    x, residual, logits, s = inputs(t, e, h, seed=650)
    logits = logits.copy()
    logits[:, 1000:] += 10.0
    ids, _, _ = OM.route(logits, top_k)
    assert ids.min() >= 1000
    pool = PooledExperts(fmt, seed=22)
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i, h), qg.qg_packed_size(fmt, h, i)
    assert 1000 * gu_sz > (1 << 32)
    gu = torch.full(((e + 1) * gu_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    dn = torch.full(((e + 1) * dn_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    for ex in sorted(set(ids.reshape(-1).tolist()) | {e}):
        gu[ex * gu_sz:(ex + 1) * gu_sz].copy_(dev(pool[ex].gu_packed))
        dn[ex * dn_sz:(ex + 1) * dn_sz].copy_(dev(pool[ex].dn_packed))

    class Wide:
        def __len__(self):
            return e + 1

        def __getitem__(self, j):
            return pool[j]

    out = run_moe(fmt, gu, dn, e, h, i, top_k, x, residual, logits, s)
    del gu, dn
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(out)), "a kernel read an unselected expert"
    check(out, Layer(Wide()), x, residual, logits, s, top_k, False, "experts past 4 GiB")

# ------------------------------------------------- RMS-norm-fed expert layer

def norm_inputs(t, e, h, seed):
    """A pre-norm block's input (a residual stream, N(0,1)*6), the norm's gain
    1 + 0.25*N(0,1), and the routing inputs."""
    x, residual, logits, s = inputs(t, e, h, seed)
    gamma = (1.0 + 0.25 * workloads.normal((1, h), seed, 9005)[0]).astype(np.float32)
    return (x * np.float32(6.0)).astype(np.float32), gamma, residual, logits, s


def run_moe_norm(fmt, gu_d, dn_d, e, h, i, top_k, x, gamma, eps, residual, logits, s, flags=0,
                 alias_residual=False):
    t = x.shape[0]
    x_d = dev(x)
    r_d = x_d if alias_residual else dev(residual)
    out = torch.full((t, h), float("nan"), device="cuda")
    ws_bytes = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    qg.moe_expert_ffn_rmsnorm(fmt, gu_d, dn_d, e, h, i, top_k, x_d, None if gamma is None else dev(gamma), eps, r_d,
                              dev(logits), dev(s), t, out, ws, ws_bytes, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_norm(out, layer, x, gamma, eps, residual, logits, s, top_k, renorm, label):
    if top_k < logits.shape[1]:
        assert np.all(OM.route_margin(logits, top_k) > 1e-6), f"{label}: near-tied route; change the seed"
    wg, wu, wd = layer.view("gate"), layer.view("up"), layer.view("down")
    ref = ON.moe_rmsnorm_ref(wg, wu, wd, x, gamma, eps, residual, logits, s, top_k, renorm)
    tol = ON.moe_rmsnorm_tolerance(wg, wu, wd, x, gamma, eps, residual, ref)
    err = np.abs(out.astype(np.float64) - ref["out"])
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert np.all(err <= tol), f"{label}: |err|/tol = {err[worst] / tol[worst]:.3g} at {worst}"
    return ref


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 2, 3, 5, 7, 8])
def test_moe_rmsnorm_small(fmt, t):
    e, h, i, top_k = 16, 512, 256, 4
    layer, gu, dn = small_layer(fmt, e, h, i, seed=11)
    x, gamma, residual, logits, s = norm_inputs(t, e, h, seed=150 + t)
    out = run_moe_norm(fmt, gu, dn, e, h, i, top_k, x, gamma, 1e-6, residual, logits, s)
    check_norm(out, layer, x, gamma, 1e-6, residual, logits, s, top_k, False, f"{fmt} norm T={t}")


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 8])
def test_moe_rmsnorm_unit_gain(fmt, t):
    """gamma = NULL (the gain folded into the experts' gate/up weights): the
    oracle with a gain of ones."""
    e, h, i, top_k = 16, 512, 256, 4
    layer, gu, dn = small_layer(fmt, e, h, i, seed=11)
    x, _, residual, logits, s = norm_inputs(t, e, h, seed=170 + t)
    out = run_moe_norm(fmt, gu, dn, e, h, i, top_k, x, None, 1e-6, residual, logits, s)
    check_norm(out, layer, x, np.ones(h, np.float32), 1e-6, residual, logits, s, top_k, False, f"{fmt} unit T={t}")


@pytest.mark.parametrize("fmt", KFORMATS)
def test_moe_rmsnorm_pre_norm_block(fmt):
    """out = x + MoE(rmsnorm(x)): residual aliases x; all 8 tokens share four
    experts (two-token items), renormalised weights, eps = 1e-5."""
    e, h, i, top_k, t = 10, 512, 256, 4, 8
    layer, gu, dn = small_layer(fmt, e, h, i, seed=13)
    x, gamma, _, logits, s = norm_inputs(t, e, h, seed=350)
    logits = logits.copy()
    favourites = [7, 2, 9, 4]
    for tok in range(t):
        for rank, ex in enumerate(np.roll(favourites, tok)):
            logits[tok, ex] = 6.0 - 0.5 * rank
    out = run_moe_norm(fmt, gu, dn, e, h, i, top_k, x, gamma, 1e-5, x, logits, s, flags=qg.QG_MOE_RENORM,
                       alias_residual=True)
    check_norm(out, layer, x, gamma, 1e-5, x, logits, s, top_k, True, f"{fmt} pre-norm block")


@pytest.mark.parametrize("fmt", KFORMATS)
@pytest.mark.parametrize("t", [1, 8])
def test_moe_rmsnorm_full_layer(fmt, t):
    e, h, i, top_k = FULL_E, FULL_H, FULL_I, FULL_K
    x, gamma, residual, logits, s = norm_inputs(t, e, h, seed=650 + t)
    ids, _, _ = OM.route(logits, top_k)
    used = sorted(set(ids.reshape(-1).tolist()) | {e})
    pool = PooledExperts(fmt, seed=21)
    gu_sz, dn_sz = qg.qg_packed_size(fmt, 2 * i, h), qg.qg_packed_size(fmt, h, i)
    gu = torch.full(((e + 1) * gu_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    dn = torch.full(((e + 1) * dn_sz,), 0xFF, dtype=torch.uint8, device="cuda")
    for ex in used:
        gu[ex * gu_sz:(ex + 1) * gu_sz].copy_(dev(pool[ex].gu_packed))
        dn[ex * dn_sz:(ex + 1) * dn_sz].copy_(dev(pool[ex].dn_packed))
    out = run_moe_norm(fmt, gu, dn, e, h, i, top_k, x, gamma, 1e-6, residual, logits, s)
    assert np.all(np.isfinite(out)), "a kernel read an unselected expert"
    check_norm(out, Layer(pool), x, gamma, 1e-6, residual, logits, s, top_k, False, f"{fmt} norm full T={t}")


def test_moe_graph_replay():
    """The four launches captured in a graph replay bit-equal to eager, with
    eager work in between that overwrites the workspace."""
    fmt, e, h, i, top_k, t = "q4_k", 16, 512, 256, 4, 8
    _, gu, dn = small_layer(fmt, e, h, i, seed=16)
    x, residual, logits, s = inputs(t, e, h, seed=700)
    x_d, r_d, l_d, s_d = dev(x), dev(residual), dev(logits), dev(s)
    ws_bytes = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    eager = torch.empty((t, h), device="cuda")
    qg.moe_expert_ffn(fmt, gu, dn, e, h, i, top_k, x_d, r_d, l_d, s_d, t, eager, ws, ws_bytes)
    torch.cuda.synchronize()
    out = torch.empty((t, h), device="cuda")
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qg.moe_expert_ffn(fmt, gu, dn, e, h, i, top_k, x_d, r_d, l_d, s_d, t, out, ws, ws_bytes,
                              stream=stream)
    torch.cuda.synchronize()
    for _ in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))
