"""GPU parity: libmala (through its C ABI) against the CPU fp64 oracle on the
same seeded inputs. Decisions must match outside the near-tie band (forward
near ties are replayed so that later decisions stay comparable), kept-tile
counters exactly, and values within the stated tolerances."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import mala_oracle as O
from parity_util import (BAND, add_output_rounding, assert_bitwise_where_agree, check_dq_o_rounding,
                         check_forward, check_lse, check_nesting, check_ties, compare_values,
                         dtype_name, grad_rounding_bounds, is_bounded, np64, o_rounding_dk_term,
                         o_rounding_dq_term, tiling)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():   # collected on CPU only to be deselected
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda"


def lib():
    import contribution_gated_sparse_amd as m
    return m


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def check_backward(x, tau, g_fwd, r_fwd, causal=True, qblocks=None, key_rows=None,
                   gate_pass=False, fwd_mask=None, max_ties=4, strict=True, dq_o_rounding=False,
                   fro_o_rounding=False):
    m = lib()
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    kind = dtype_name(q)
    _, (bq, bk, _), _ = tiling()
    g = m.mala_bwd(q, k, v, g_fwd["o"], g_fwd["lse"], do, tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, gate_pass=gate_pass,
                   fwd_mask=fwd_mask)
    torch.cuda.synchronize()
    gmask = g["mask"].cpu().numpy()
    r = O.mala_bwd(np64(q), np64(k), np64(v), r_fwd["o"], r_fwd["lse"], np64(do), tau,
                   x["scale"], causal, bq, bk, qblocks=qblocks, replay=gmask, band=BAND[kind],
                   o_storage=kind, lse_storage="f32")
    checked = r["mask"] != O.NOT_VISITED
    clear = checked & ~(np.abs(r["margin"]) < BAND[kind])
    assert np.array_equal(gmask[clear], r["mask"][clear]), (
        f"backward decisions differ: {int((gmask[clear] != r['mask'][clear]).sum())}")
    if qblocks is None:
        assert np.array_equal(gmask != O.NOT_VISITED, checked)
        kept_o = (gmask == O.KEPT).sum(-1)
        assert np.array_equal(kept_o, g["kept"].cpu().numpy())
    nq = q.shape[2]
    if qblocks is None:
        rows = np.ones(q.shape[:3], bool)
    else:
        rows = np.zeros(q.shape[:3], bool)
        for i in qblocks:
            rows[:, :, i * bq:min(nq, (i + 1) * bq)] = True
    st = {}
    # the derived rounding bounds, for the comparisons that take them
    bd = {"dq": None, "dk": None, "dv": None}
    if any(is_bounded(nm, kind) for nm in ("dQ", "dK", "dV")):
        bd = grad_rounding_bounds(np64(q), np64(k), np64(v), np64(do), x["scale"], causal, r_fwd,
                                  r["mask"], kind, lse_gpu=g_fwd["lse"].cpu().numpy(),
                                  o_gpu=np64(g_fwd["o"]))
        bd = add_output_rounding(bd, r, kind)
    if dq_o_rounding:     # inputs whose dQ is conditioned by the bf16 rounding of the stored O
        term = o_rounding_dq_term(np64(q), np64(k), np64(v), np64(do), x["scale"], causal,
                                  r_fwd, r, rows)
        check_dq_o_rounding("dQ", np64(g["dq"])[rows], r["dq"][rows], term)
    else:
        # fro_o_rounding (bf16): the Frobenius bars of dQ and dK widened by the
        # bf16-O rounding terms, for inputs whose gradients can be near zero
        # (their relative error is then that rounding's); the element-wise
        # bars stay as they are
        ft = None
        if fro_o_rounding and kind == "bf16":
            ft = o_rounding_dq_term(np64(q), np64(k), np64(v), np64(do), x["scale"], causal,
                                    r_fwd, r)
        st["dq"] = compare_values("dQ", np64(g["dq"]), r["dq"], kind, rows, strict=strict,
                                  bound=bd["dq"], fro_term=ft)
    if key_rows is not None or qblocks is None:
        kr = slice(None) if key_rows is None else key_rows
        fk = None
        if fro_o_rounding and kind == "bf16":
            fk = o_rounding_dk_term(np64(q), np64(k), np64(v), np64(do), x["scale"], causal,
                                    r_fwd, r)[:, :, kr]
        st["dk"] = compare_values("dK", np64(g["dk"])[:, :, kr], r["dk"][:, :, kr], kind,
                                  strict=strict,
                                  bound=None if bd["dk"] is None else bd["dk"][:, :, kr],
                                  fro_term=fk)
        st["dv"] = compare_values("dV", np64(g["dv"])[:, :, kr], r["dv"][:, :, kr], kind,
                                  strict=strict,
                                  bound=None if bd["dv"] is None else bd["dv"][:, :, kr])
    st["ties"] = int((checked & ~clear).sum())
    check_ties("backward near ties", st["ties"], max_ties, kind)
    return g, r, st


# ------------------------------------------------------------- tiny fp32 config

@pytest.mark.parametrize("tau", [1e-4, 0.0, 1.0, 2.0, 10.0, 1e3])
def test_config1_fp32_fwd_bwd(tau):
    x = to_dev(W.make_prefill(W.CONFIGS[1]))
    g, r, st = check_forward(x, tau, max_ties=2)
    gb, rb, stb = check_backward(x, tau, g, r)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


# ------------------------------------------------------------- bf16 shapes

SHAPES = [
    # (batch, hq, hkv, nq, nk, d)
    (1, 2, 2, 1, 1, 128),
    (1, 2, 1, 63, 63, 128),
    (1, 4, 1, 65, 65, 128),
    (2, 4, 2, 200, 200, 128),
    (1, 8, 2, 777, 777, 128),
    (1, 2, 2, 300, 300, 64),
    (1, 4, 4, 100, 356, 128),     # chunked prefill: bottom-right causal alignment
    (1, 2, 2, 1, 700, 128),       # one query row against a long prefix
    (1, 16, 1, 130, 130, 128),    # a 16-head GQA group on one KV head
    (3, 4, 2, 33, 97, 64),        # d = 64, batch 3, ragged tiles, chunked
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_bf16_shapes_fwd_bwd(shape, tau):
    b, hq, hkv, nq, nk, d = shape
    cfg = W.CONFIGS[2]
    x = W.make_prefill(cfg, n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:   # queries are the last nq rows
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    g, r, st = check_forward(x, tau, max_ties=4)
    gb, rb, stb = check_backward(x, tau, g, r)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


# The d = 128 forward and dQ kernels stage K and V three tiles deep and run
# their steps unrolled by three: the forward's walk starts at a tile with
# index 2 mod 3 (up to two steps past the top tile), and dQ's walk leaves after
# whichever of its three steps meets the last needed tile. Problems of 1 to 7
# key tiles (and a ragged length) take every start and exit position.
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n", [64, 128, 192, 256, 320, 384, 448, 470])
def test_bf16_tile_counts_fwd_bwd(n, causal):
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=n, hq=2, hkv=1, d=128, batch=1, planted=4, seed=11 + n))
    for tau in (0.0, 1.0):
        g, r, st = check_forward(x, tau, causal=causal, max_ties=4)
        gb, rb, stb = check_backward(x, tau, g, r, causal=causal)
        check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noncausal(dtype):
    cfg = W.CONFIGS[2] if dtype == torch.bfloat16 else W.CONFIGS[1]
    d = 128 if dtype == torch.bfloat16 else 64
    x = W.make_prefill(cfg, n=160, hq=2, hkv=1, d=d, planted=3)
    x = to_dev(x)
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False)


def test_fp32_d128_and_gqa():
    x = W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=128, planted=4)
    x["scale"] = 1 / math.sqrt(128)
    x = to_dev(x)
    for tau in (0.0, 1e-4, 3.0):
        g, r, _ = check_forward(x, tau, max_ties=2)
        check_backward(x, tau, g, r)


# ------------------------------------------------------------- skipping inputs

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tau", [1e-4, 1e-2, 1.0])
def test_structured_skipping_fwd_bwd(dtype, tau):
    """Structured logits (sinks, local band, retrieval keys) make the gate
    skip most far tiles; decisions, counters and values still match."""
    d = 128 if dtype == "bf16" else 64
    x = to_dev(W.make_structured(1000, hq=4, hkv=2, d=d, dtype=dtype,
                                 freqs=48 if d == 128 else 24))
    g, r, st = check_forward(x, tau, max_ties=4)
    assert st["kept_frac"] < 0.8
    gb, rb, stb = check_backward(x, tau, g, r)
    bm = gb["mask"].cpu().numpy()
    assert (bm == O.SKIPPED).sum() > 0
    check_nesting(g["mask"].cpu().numpy(), bm)


@pytest.mark.parametrize("tau", [1e-2, 1.0])
def test_structured_calibrated_fwd_bwd(tau):
    """The calibrated structured preset (a local band about a thousand keys
    wide, as the paper's operating point at tau = 1): at 3000 positions the
    gate skips the far tiles; decisions, counters and values match the
    oracle, and the gate pass and nested call take the same decisions."""
    x = to_dev(W.make_structured_preset("calibrated", 3000, hq=4, hkv=2, d=128))
    g, r, st = check_forward(x, tau, max_ties=4)
    assert st["kept_frac"] < 0.95
    # dQ on these inputs is held to the stated bar plus the bf16-O rounding
    # term (o_rounding_dq_term): in rows led by the sink keys dP - D cancels
    # (about 280,000 backward decisions: a dozen near ties at most)
    gb, rb, stb = check_backward(x, tau, g, r, dq_o_rounding=True, max_ties=12)
    bm = gb["mask"].cpu().numpy()
    assert (bm == O.SKIPPED).sum() > 0
    check_nesting(g["mask"].cpu().numpy(), bm)
    for kw in (dict(gate_pass=True), dict(fwd_mask=g["mask"])):
        check_backward(x, tau, g, r, dq_o_rounding=True, max_ties=12, **kw)


# ------------------------------------------------------------- gate pass

@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_gate_pass_shapes(shape, tau):
    """MALA_FLAG_GATE_PASS: decisions from the separate score pass, dK/dV over
    the steps with a kept tile only; same bar against the oracle."""
    b, hq, hkv, nq, nk, d = shape
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    print(f"[gate pass] shape={shape} tau={tau}", flush=True)
    g, r, _ = check_forward(x, tau, max_ties=4)
    gb, _, _ = check_backward(x, tau, g, r, gate_pass=True)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())


@pytest.mark.parametrize("tau", [1e-4, 1.0])
def test_gate_pass_structured(tau):
    """On skipping inputs the gate pass takes the default path's decisions
    (outside the near-tie band) and reproduces its gradients."""
    m = lib()
    x = to_dev(W.make_structured(1500, hq=8, hkv=2, d=128))
    g, r, st = check_forward(x, tau, max_ties=4)
    assert st["kept_frac"] < 0.8
    gb, rb, _ = check_backward(x, tau, g, r, gate_pass=True)
    ref = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                     softmax_scale=x["scale"], want_mask=True)
    torch.cuda.synchronize()
    a, b_ = gb["mask"].cpu().numpy(), ref["mask"].cpu().numpy()
    clear = (a != O.NOT_VISITED) & ~(np.abs(rb["margin"]) < BAND["bf16"])
    assert np.array_equal(a[clear], b_[clear])
    assert (a == O.SKIPPED).sum() > 0
    for n in ("dq", "dk", "dv"):
        u, w = np64(gb[n]), np64(ref[n])
        assert np.abs(u - w).max() <= 2e-2 * max(1.0, np.abs(w).max()), n
    # the dQ kernel is shared: the same decisions give the same dQ bits
    assert_bitwise_where_agree(a, b_, gb, ref, 4, dkdv=False)
    # on the forward's kept tiles only: the same decisions and gradients
    _, a2, b2, want = nested_vs_gate_pass(x, tau, g["mask"])
    assert_bitwise_where_agree(a2["mask"].cpu().numpy(), want, a2, b2, 4)
    assert int((a2["mask"].cpu().numpy() != want).sum()) <= 2


def test_gate_pass_with_fast_grad():
    """Both flags: the gate pass's decisions and dK/dV with the single-bf16 dS
    of MALA_FLAG_FAST_GRAD in dQ; same decisions as the fast default path."""
    m = lib()
    x = to_dev(W.make_structured(900, hq=4, hkv=1, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-2, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, gate_pass=True)
    torch.cuda.synchronize()
    ma, mb = a["mask"].cpu().numpy(), b["mask"].cpu().numpy()
    assert int((ma != mb).sum()) <= 2 and (mb == O.SKIPPED).sum() > 0
    assert_bitwise_where_agree(ma, mb, a, b, 4, dkdv=False)
    for n in ("dq", "dk", "dv"):
        u, w = np64(b[n]), np64(a[n])
        assert np.abs(u - w).max() <= 1e-2 * max(1.0, np.abs(w).max()), n
    # the automatic choice keeps the flag: its result is one of the two fast walks
    c = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, fwd_kept=f["kept"])
    torch.cuda.synchronize()
    assert any(all(torch.equal(c[n], r[n]) for n in ("dq", "dk", "dv", "mask")) for r in (a, b))


def test_gate_pass_noncausal_and_f32():
    """Non-causal walks through the gate pass; the flag is ignored for fp32."""
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=160, hq=2, hkv=1, d=128, planted=3))
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False, gate_pass=True)
    x = to_dev(W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=64, planted=4))
    g, r, _ = check_forward(x, 1.0, max_ties=2)
    check_backward(x, 1.0, g, r, gate_pass=True)


def fwd_legal_tiles(nq, nk, causal):
    """The forward's legal tiles of one head: each 32-row block's tiles up to
    the one holding its last row's last visible key."""
    (fbq, fbk, _), _, _ = tiling()
    legal = 0
    for i in range(-(-nq // fbq)):
        last = min(i * fbq + fbq - 1, nq - 1)
        lastkey = min(last + nk - nq, nk - 1) if causal else nk - 1
        legal += lastkey // fbk + 1 if lastkey >= 0 else 0
    return legal


def auto_takes_gate_pass(fwd_kept, gate_mask, nq, nk, causal):
    """The walk mala_bwd_auto documents. At these sizes (at most 1,984 keys,
    fewer than 512 blocks of 256 rows) its sample is the whole backward gate,
    so it sees the backward's own decisions (``gate_mask``: the gate
    pass's tile mask): with at least 256 legal 16-key columns the gate-pass
    walks are taken when fewer than 60% of them are kept; with fewer, the
    forward's counters decide (fewer than 70% of its legal tiles kept)."""
    gm = gate_mask.cpu().numpy()
    assert nk <= 1984 and gm.shape[0] * gm.shape[1] * -(-nq // 256) < 512
    legal_s, kept_s = int((gm != O.NOT_VISITED).sum()), int((gm == O.KEPT).sum())
    if legal_s >= 256:
        return 10 * kept_s < 6 * legal_s
    kt = fwd_kept.cpu().numpy()
    return 10 * int(kt.sum()) < 7 * fwd_legal_tiles(nq, nk, causal) * kt.shape[0] * kt.shape[1]


def assert_auto_is_chosen_walk(x, tau, causal=True, want_gate=None):
    """mala_bwd_auto against the explicit call of the walk its rule picks:
    gradients, tile mask and kept counters equal bit for bit. Returns the
    walk and the forward's kept fraction."""
    m = lib()
    nq, nk = x["q"].shape[2], x["k"].shape[2]
    f = m.mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"])
    kw = dict(causal=causal, softmax_scale=x["scale"], want_mask=True)
    g = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, gate_pass=True, **kw)
    d = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, **kw)
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, fwd_kept=f["kept"], **kw)
    torch.cuda.synchronize()
    gate = auto_takes_gate_pass(f["kept"], g["mask"], nq, nk, causal)
    if want_gate is not None:
        assert gate == want_gate
    b = g if gate else d
    for n in ("dq", "dk", "dv", "mask", "kept"):
        assert torch.equal(a[n], b[n]), (n, gate)
    kt = f["kept"].cpu().numpy()
    frac = int(kt.sum()) / (fwd_legal_tiles(nq, nk, causal) * kt.shape[0] * kt.shape[1])
    return gate, frac


@pytest.mark.parametrize("preset,tau,want_gate", [("sparse", 1.0, True), ("sparse", 1e-4, True),
                                                  ("calibrated", 1.0, None),
                                                  ("sparse", 0.0, False)])
def test_auto_walk_choice_structured(preset, tau, want_gate):
    """mala_bwd_auto on structured inputs: the sparse preset keeps about a
    quarter of the legal tiles at 1,500 keys (the gate-pass walks), tau = 0
    all of them (the default walk). Both walks are held to the oracle by the
    tests above, on these inputs."""
    x = to_dev(W.make_structured_preset(preset, 1500, hq=8, hkv=2, d=128))
    print(f"[auto] preset={preset} tau={tau}", flush=True)
    assert_auto_is_chosen_walk(x, tau, want_gate=want_gate)


def test_auto_walk_choice_sinks():
    """Mass on the sink keys and the rest of the logits flat: the forward,
    which meets the sinks last, keeps nearly every tile, while the backward
    keeps few. The choice follows the backward's own sampled decisions and
    takes the gate-pass walks."""
    x = to_dev(W.make_structured(1500, hq=8, hkv=2, d=128, window=65536))
    print("[auto] sinks", flush=True)
    gate, frac = assert_auto_is_chosen_walk(x, 1.0, want_gate=True)
    assert frac > 0.7


@pytest.mark.parametrize("shape", SHAPES)
def test_auto_walk_choice_shapes(shape):
    """Ragged shapes, both head sizes, causal and not: whichever walk the
    rule picks, the result is that walk's."""
    b, hq, hkv, nq, nk, d = shape
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=5 + nq)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    print(f"[auto] shape={shape}", flush=True)
    for causal in (True, False):
        for tau in (1e-4, 100.0):
            assert_auto_is_chosen_walk(x, tau, causal=causal)


def test_auto_walk_f32_is_plain_backward():
    """fp32 has one backward walk: mala_bwd_auto reads no counters and equals
    mala_bwd bit for bit, at a tolerance that keeps few tiles and one that
    keeps most."""
    m = lib()
    x = to_dev(W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=64, planted=4))
    for tau in (1e-4, 100.0):
        f = m.mala_fwd(x["q"], x["k"], x["v"], tau, softmax_scale=x["scale"])
        a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau,
                       softmax_scale=x["scale"], want_mask=True, fwd_kept=f["kept"])
        b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau,
                       softmax_scale=x["scale"], want_mask=True)
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "mask", "kept"):
            assert torch.equal(a[n], b[n]), (n, tau)


def random_case(case):
    """Seeded shape and options of one randomized parity case."""
    rng = np.random.default_rng(20260000 + case)
    hkv = int(rng.choice([1, 2]))
    c = dict(d=int(rng.choice([64, 128])), hkv=hkv, hq=hkv * int(rng.choice([1, 2, 4])),
             b=int(rng.choice([1, 2])), nk=int(rng.integers(1, 420)),
             causal=bool(rng.random() < 0.7), tau=float(rng.choice([0.0, 1e-4, 1e-2, 1.0, 100.0])),
             fp32=bool(rng.random() < 0.25), planted=int(rng.integers(0, 7)))
    c["nq"] = c["nk"] if rng.random() < 0.5 else int(rng.integers(1, c["nk"] + 1))
    return c


# case 161: one query row, non-causal, tau = 100: dQ and dK near zero
@pytest.mark.parametrize("case", list(range(48)) + [161])
def test_random_shapes(case):
    """Seeded random problems (batch, GQA group, ragged and chunked lengths,
    both head sizes, causal or not, the tolerance from 0 to 100, bf16 or
    fp32): the forward, and the default, gate-pass and automatic backward,
    each against the oracle at the same bars (the automatic one also against
    the walk it picks, bit for bit)."""
    c = random_case(case)
    print(f"[random] case={case} {c}", flush=True)
    cfg = W.CONFIGS[1] if c["fp32"] else W.CONFIGS[2]
    x = W.make_prefill(cfg, n=c["nk"], hq=c["hq"], hkv=c["hkv"], d=c["d"], batch=c["b"],
                       planted=c["planted"], seed=31 + case)
    if c["nq"] < c["nk"]:
        x["q"] = x["q"][:, :, c["nk"] - c["nq"]:].contiguous()
        x["do"] = x["do"][:, :, c["nk"] - c["nq"]:].contiguous()
    x = to_dev(x)
    tau, causal = c["tau"], c["causal"]
    g, r, _ = check_forward(x, tau, causal=causal, max_ties=4)
    # a random problem can leave dQ and dK near zero (one query row, tau =
    # 100), where their relative Frobenius error is the bf16-O rounding of D
    gb, _, _ = check_backward(x, tau, g, r, causal=causal, fro_o_rounding=True)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())
    check_backward(x, tau, g, r, causal=causal, gate_pass=True, fro_o_rounding=True)
    assert_auto_is_chosen_walk(x, tau, causal=causal)


@pytest.mark.parametrize("case", range(24))
def test_random_structured(case):
    """Seeded random structured-logit problems (sink logits up to 30, band
    widths 16 to 65,536, retrieval keys up to 64 at logits up to 40, peaks up
    to 60, tolerances 1e-4 to 100): the forward, and the default, gate-pass
    and automatic backward, each against the oracle. dQ takes the bf16-O
    rounding term, as on the other structured inputs: where the sink keys
    dominate, dP - D cancels and the stored O's rounding is amplified."""
    rng = np.random.default_rng(20263000 + case)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    n = int(rng.integers(100, 1600))
    window = int(rng.choice([16, 64, 128, 512, 2048, 65536]))
    kw = dict(hq=hq, hkv=hkv, d=128, window=window, seed=900 + case,
              sink_logit=float(rng.choice([0.0, 8.0, 18.0, 30.0])),
              retrieval=int(rng.choice([0, 4, 16, 64])),
              retrieval_logit=float(rng.choice([10.0, 22.0, 40.0])),
              peak=float(rng.choice([5.0, 25.0, 60.0])))
    tau = float(rng.choice([1e-4, 1e-2, 1.0, 100.0]))
    causal = bool(rng.random() < 0.8)
    print(f"[random structured] case={case} n={n} tau={tau} causal={causal} {kw}", flush=True)
    x = to_dev(W.make_structured(n, **kw))
    g, r, _ = check_forward(x, tau, causal=causal, max_ties=12)
    gb, _, _ = check_backward(x, tau, g, r, causal=causal, dq_o_rounding=True,
                              fro_o_rounding=True, max_ties=12)
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())
    check_backward(x, tau, g, r, causal=causal, gate_pass=True, dq_o_rounding=True,
                   fro_o_rounding=True, max_ties=12)
    assert_auto_is_chosen_walk(x, tau, causal=causal)


@pytest.mark.parametrize("case", range(8))
def test_random_long_shapes(case):
    """Seeded random bf16 problems of 1,000-3,000 keys (many phases of the
    forward's and dQ's three-buffer staging, several 128-key dK/dV blocks per
    head): the forward, the default and gate-pass backward, the nested call
    and the single-bf16 dS of MALA_FLAG_FAST_GRAD, each against the oracle,
    and the automatic choice against the walk it returns."""
    rng = np.random.default_rng(20262000 + case)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    nk = int(rng.integers(1000, 3000))
    nq = nk if rng.random() < 0.6 else int(rng.integers(1, nk + 1))
    d = int(rng.choice([64, 128]))
    tau = float(rng.choice([1e-4, 1e-2, 1.0]))
    print(f"[random long] case={case} hq={hq} hkv={hkv} nq={nq} nk={nk} d={d} tau={tau}",
          flush=True)
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=1,
                       planted=int(rng.integers(0, 32)), seed=131 + case)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    g, r, _ = check_forward(x, tau, max_ties=4)
    check_backward(x, tau, g, r)
    check_backward(x, tau, g, r, gate_pass=True)
    check_backward(x, tau, g, r, fwd_mask=g["mask"])
    m = lib()
    a = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                   softmax_scale=x["scale"], want_mask=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True)
    torch.cuda.synchronize()
    # the flag changes only dQ's dS precision: same decisions, dK and dV
    assert torch.equal(a["mask"], b["mask"]) and torch.equal(a["dk"], b["dk"])
    assert torch.equal(a["dv"], b["dv"])
    u, w = np64(b["dq"]), np64(a["dq"])
    assert np.abs(u - w).max() <= 2e-2 * max(1.0, np.abs(w).max())
    # the automatic choice (a sampled gate above 1,984 keys): one of the two
    # walks, bit for bit
    c = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                   softmax_scale=x["scale"], want_mask=True, fwd_kept=g["kept"])
    e = m.mala_bwd(x["q"], x["k"], x["v"], g["o"], g["lse"], x["do"], tau,
                   softmax_scale=x["scale"], want_mask=True, gate_pass=True)
    torch.cuda.synchronize()
    assert any(all(torch.equal(c[n], r_[n]) for n in ("dq", "dk", "dv", "mask", "kept"))
               for r_ in (a, e))


def expand_fwd(fmask, shape):
    """The forward tile mask on the backward partition (each backward tile
    lies in one forward tile)."""
    (fbq, fbk, _), (bbq, bbk, _), _ = tiling()
    up = np.repeat(np.repeat(fmask, fbq // bbq, axis=2), fbk // bbk, axis=3)
    return up[:, :, :shape[2], :shape[3]]


def nested_vs_gate_pass(x, tau, fwd_mask, causal=True):
    """mala_bwd_nested with ``fwd_mask`` against the gate pass on the same
    inputs: its decisions are the gate pass's restricted to the forward's
    kept tiles, bit for bit; returns both results and the expected mask."""
    m = lib()
    f = m.mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, gate_pass=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], tau, causal=causal,
                   softmax_scale=x["scale"], want_mask=True, fwd_mask=fwd_mask)
    torch.cuda.synchronize()
    ma, mb = a["mask"].cpu().numpy(), b["mask"].cpu().numpy()
    up = expand_fwd(fwd_mask.cpu().numpy(), ma.shape)
    want = np.where((ma == O.KEPT) & (up != O.KEPT), O.SKIPPED, ma)
    assert np.array_equal(mb, want), f"{int((mb != want).sum())} decisions differ"
    assert np.array_equal(b["kept"].cpu().numpy(), (mb == O.KEPT).sum(-1))
    return f, a, b, want


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 100.0])
def test_nested_shapes(shape, tau):
    """mala_bwd_nested on the forward's own mask: the oracle's bar, support
    nested in the forward's, and the gate pass's decisions and gradients
    wherever the two agree (exact arithmetic makes them agree everywhere)."""
    b, hq, hkv, nq, nk, d = shape
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=hq, hkv=hkv, d=d, batch=b, planted=4, seed=7 + nq)
    if nq < nk:
        x["q"] = x["q"][:, :, nk - nq:].contiguous()
        x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    print(f"[nested] shape={shape} tau={tau}", flush=True)
    g, r, _ = check_forward(x, tau, max_ties=4)
    gb, _, _ = check_backward(x, tau, g, r, fwd_mask=g["mask"])
    check_nesting(g["mask"].cpu().numpy(), gb["mask"].cpu().numpy())
    _, a, b_, want = nested_vs_gate_pass(x, tau, g["mask"])
    assert_bitwise_where_agree(a["mask"].cpu().numpy(), want, a, b_, hq // hkv)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("density", [0.0, 0.03, 0.5, 1.0])
def test_nested_arbitrary_forward_masks(causal, density):
    """The walk over the forward's kept tiles with masks the forward would not
    write (sparse, dense, empty; more than 64 key tiles, so the look-ahead
    window moves): decisions are exactly the gate pass's on the given tiles,
    and the gradients are the oracle's on that support."""
    nq, nk = 300, 4700
    x = W.make_prefill(W.CONFIGS[2], n=nk, hq=2, hkv=1, d=128, planted=4, seed=11)
    x["q"] = x["q"][:, :, nk - nq:].contiguous()
    x["do"] = x["do"][:, :, nk - nq:].contiguous()
    x = to_dev(x)
    tau = 1e-4
    print(f"[nested mask] causal={causal} density={density}", flush=True)
    fm = lib().mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"],
                        want_mask=True)["mask"].cpu().numpy()
    rng = np.random.default_rng(int(1000 * density) + causal)
    rand = np.where(rng.random(fm.shape) < density, O.KEPT, O.SKIPPED).astype(np.int8)
    fm = np.where(fm == O.NOT_VISITED, fm, rand)
    fmt = torch.from_numpy(fm).to(DEV)
    f, a, b, _ = nested_vs_gate_pass(x, tau, fmt, causal=causal)
    if density == 0.0:
        for n in ("dq", "dk", "dv"):
            assert not b[n].any(), n
    # the oracle's own forward (O, LSE) and its own backward decisions,
    # restricted to the tiles the given forward mask keeps
    (fbq, fbk, _), (bq, bk, _), _ = tiling()
    qn, kn, vn, don = np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(x["do"])
    g = lib().mala_fwd(x["q"], x["k"], x["v"], tau, causal=causal, softmax_scale=x["scale"],
                       want_mask=True)
    torch.cuda.synchronize()
    rf = O.mala_fwd(qn, kn, vn, tau, x["scale"], causal, fbq, fbk,
                    replay=g["mask"].cpu().numpy(), band=BAND["bf16"])
    gm = b["mask"].cpu().numpy()
    rb = O.mala_bwd(qn, kn, vn, rf["o"], rf["lse"], don, tau, x["scale"], causal, bq, bk,
                    replay=gm, band=BAND["bf16"], o_storage="bf16", lse_storage="f32")
    up = expand_fwd(fm, gm.shape)
    want = np.where((up == O.KEPT) | (rb["mask"] == O.NOT_VISITED), rb["mask"], O.SKIPPED)
    assert np.array_equal(gm, want), f"{int((gm != want).sum())} decisions differ"
    ties = int(((up == O.KEPT) & (np.abs(rb["margin"]) < BAND["bf16"])).sum())
    check_ties("nested near ties", ties, 4)
    if density == 0.0:
        assert not (want == O.KEPT).any()
    # gradients on that support (every decision of ``want`` is the oracle's,
    # or a replayed near tie)
    rr = O.mala_bwd(qn, kn, vn, rf["o"], rf["lse"], don, tau, x["scale"], causal, bq, bk,
                    replay=want, band=np.inf, o_storage="bf16", lse_storage="f32")
    bd = add_output_rounding(grad_rounding_bounds(qn, kn, vn, don, x["scale"], causal, rf, want,
                                                  "bf16", lse_gpu=f["lse"].cpu().numpy(),
                                                  o_gpu=np64(f["o"])),
                             rr, "bf16")
    for n in ("dq", "dk", "dv"):
        compare_values(n, np64(b[n]), rr[n], "bf16", bound=bd[n])


def test_backward_modes_are_deterministic():
    """Every backward mode gives the same bits on a second run: the default
    path, the gate pass (whose heavy key blocks sum per-head partials in head
    order) and the nested call."""
    m = lib()
    x = to_dev(W.make_structured(2000, hq=8, hkv=2, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-4, softmax_scale=x["scale"], want_mask=True)
    for kw in (dict(), dict(gate_pass=True), dict(fwd_mask=f["mask"])):
        runs = [m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                           softmax_scale=x["scale"], **kw) for _ in range(2)]
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "kept"):
            assert torch.equal(runs[0][n], runs[1][n]), (n, list(kw))


def test_nested_noncausal_fast_grad_and_f32():
    """The nested call with MALA_FLAG_FAST_GRAD, non-causal, and for fp32
    (where the forward mask is not read and the call is the backward)."""
    m = lib()
    x = to_dev(W.make_structured(900, hq=4, hkv=1, d=128))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-2, softmax_scale=x["scale"], want_mask=True)
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, gate_pass=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-2,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True, fwd_mask=f["mask"])
    torch.cuda.synchronize()
    assert_bitwise_where_agree(a["mask"].cpu().numpy(), b["mask"].cpu().numpy(), a, b, 4)
    assert int((a["mask"] != b["mask"]).sum()) <= 2
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=160, hq=2, hkv=1, d=128, planted=3))
    for tau in (0.0, 0.5, 50.0):
        g, r, _ = check_forward(x, tau, causal=False, max_ties=4)
        check_backward(x, tau, g, r, causal=False, fwd_mask=g["mask"])
    x = to_dev(W.make_prefill(W.CONFIGS[1], n=150, hq=4, hkv=2, d=64, planted=4))
    g, r, _ = check_forward(x, 1.0, max_ties=2)
    check_backward(x, 1.0, g, r, fwd_mask=g["mask"])


# ------------------------------------------------------------- decode

def check_decode(x, lens, tau, steps_q, max_ties=4, split_keys=0):
    m = lib()
    kc, vc = x["k_cache"], x["v_cache"]
    kind = dtype_name(kc)
    _, _, (_, dbk, chunk) = tiling()
    q = steps_q
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    print(f"[decode] {kind} lens={lens} tau={tau} split_keys={split_keys}", flush=True)
    g = m.mala_decode(q, kc, vc, seq, tau, max_n_k=max(lens), softmax_scale=x["scale"],
                      want_mask=True, split_keys=split_keys)
    torch.cuda.synchronize()
    if split_keys == 0:   # 256 keys, capped at max_n_k rounded up to 64 (one split)
        assert g["split"] == min(chunk, -(-max(lens) // 64) * 64)
    chunk = g["split"]
    gmask = g["mask"].cpu().numpy()
    r = O.mala_decode(np64(q), np64(kc), np64(vc), lens, tau, x["scale"], chunk, dbk,
                      replay=gmask, band=BAND[kind])
    assert np.array_equal(gmask, r["mask"]), "decode decisions differ outside the near-tie band"
    assert r["near_ties"] <= max_ties
    kept = g["kept"].cpu().numpy()
    hq = q.shape[1]
    assert np.array_equal(kept[:, :hq], (r["mask"] == O.KEPT).sum((-1, -2)))
    assert np.array_equal(kept[:, hq:], r["v_tiles"].sum((-1, -2)))
    compare_values("decode O", np64(g["o"]), r["o"], kind)
    check_lse("decode LSE", np64(g["lse"]), r["lse"], kind)
    return g, r


@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 50.0])
def test_decode_bf16_small(tau):
    x = W.make_decode(W.CONFIGS[5], cache=1100, steps=3, batch=3, planted=16)
    x = to_dev(x)
    lens = [1103, 1101, 257]
    q = x["q_steps"][2]
    check_decode(x, lens, tau, q.contiguous())


@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0, 50.0])
def test_decode_f32_small(tau):
    x = W.make_decode(W.CONFIGS[5], cache=600, steps=2, batch=2, hq=4, hkv=2, planted=8)
    x = {k: (v.float() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    x = to_dev(x)
    check_decode(x, [602, 65], tau, x["q_steps"][1].contiguous())


# split lengths other than the default: one tile per split, splits that are
# not whole groups of four tiles, several 32-tile decision words per split,
# the automatic rule, and one split per sequence (App. A.1 "Fused decoding
# execution": each split tests its tiles against its own partial normalizer)
@pytest.mark.parametrize("split_keys", [64, 192, 512, 2560, -1, 8192])
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0])
def test_decode_bf16_split_lengths(split_keys, tau):
    x = W.make_decode(W.CONFIGS[5], cache=4100, steps=1, batch=3, planted=24)
    x = to_dev(x)
    g, r = check_decode(x, [4101, 3001, 257], tau, x["q_steps"][0].contiguous(),
                        split_keys=split_keys)
    if split_keys == 8192:
        assert g["split"] == 4160 and g["mask"].shape[2] == 1


# one split per sequence runs as three passes (tile statistics, per-head gate
# replay, P V over kept tiles); other group shapes: 16 query heads per KV head
# (a 1024-thread gate workgroup) and 4 per KV head with two KV heads
@pytest.mark.parametrize("hq,hkv", [(16, 1), (8, 2)])
@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_decode_bf16_unsplit_groups(hq, hkv, tau):
    x = W.make_decode(W.CONFIGS[5], cache=3000, steps=1, batch=2, hq=hq, hkv=hkv, planted=12)
    x = to_dev(x)
    g, r = check_decode(x, [3001, 1500], tau, x["q_steps"][0].contiguous(), split_keys=8192)
    assert g["split"] == 3008 and g["mask"].shape[2] == 1


# many (sequence, KV head) pairs of ragged lengths (splits past the end of
# shorter sequences); with 512-key splits a split is two groups of four tiles
@pytest.mark.parametrize("batch,hq,hkv,split_keys", [(40, 4, 2, 0), (40, 4, 2, 128),
                                                     (80, 2, 2, 512)])
@pytest.mark.parametrize("tau", [0.0, 1e-4, 1.0])
def test_decode_bf16_many_sequences(batch, hq, hkv, split_keys, tau):
    x = W.make_decode(W.CONFIGS[5], cache=4100, steps=1, batch=batch, hq=hq, hkv=hkv, planted=8)
    x = to_dev(x)
    lens = [4101 - (97 * b) % 3900 for b in range(batch)]
    check_decode(x, lens, tau, x["q_steps"][0].contiguous(), split_keys=split_keys)


@pytest.mark.parametrize("split_keys", [64, 320, 2560])
def test_decode_f32_split_lengths(split_keys):
    x = W.make_decode(W.CONFIGS[5], cache=2200, steps=1, batch=2, hq=4, hkv=2, planted=8)
    x = {k: (v.float() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    x = to_dev(x)
    check_decode(x, [2201, 130], 1e-4, x["q_steps"][0].contiguous(), split_keys=split_keys)


def random_decode_case(case):
    """Seeded shape and options of one randomized decode case."""
    rng = np.random.default_rng(20261000 + case)
    hkv = int(rng.choice([1, 2]))
    cache = int(rng.integers(1, 3000))
    c = dict(batch=int(rng.integers(1, 7)), hkv=hkv, hq=hkv * int(rng.choice([1, 2, 4, 8])),
             cache=cache, tau=float(rng.choice([0.0, 1e-4, 1.0, 50.0])),
             fp32=bool(rng.random() < 0.25), planted=int(rng.integers(0, 9)),
             split=str(rng.choice(["default", "auto", "multiple", "unsplit"])),
             mult=64 * int(rng.integers(1, 40)))
    c["lens"] = [int(x) for x in rng.integers(1, cache + 2, size=c["batch"])]
    return c


@pytest.mark.parametrize("case", range(24))
def test_random_decode(case):
    """Seeded random decode batches (ragged lengths from 1 key up, GQA groups
    up to 8, the default, automatic, any-multiple-of-64 and one-per-sequence
    split lengths, the tolerance from 0 to 50, bf16 or fp32) against the
    oracle: decisions, counters, O and LSE."""
    c = random_decode_case(case)
    print(f"[random decode] case={case} {c}", flush=True)
    x = W.make_decode(W.CONFIGS[5], cache=c["cache"], steps=1, batch=c["batch"], hq=c["hq"],
                      hkv=c["hkv"], planted=c["planted"], seed=77 + case)
    if c["fp32"]:
        x = {k: (v.float() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    x = to_dev(x)
    sk = {"default": 0, "auto": lib().DECODE_SPLIT_AUTO, "multiple": c["mult"],
          "unsplit": -(-max(c["lens"]) // 64) * 64}[c["split"]]
    check_decode(x, c["lens"], c["tau"], x["q_steps"][0].contiguous(), split_keys=sk)


@pytest.mark.parametrize("case", range(16))
def test_random_structured_decode(case):
    """Seeded random decode batches over structured-logit caches (sinks up to
    logit 30, band widths 16 to 65,536, retrieval keys), each sequence's query
    its last visible row, every split-length mode: decisions, counters, O and
    LSE against the oracle."""
    rng = np.random.default_rng(20264000 + case)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    n = int(rng.integers(64, 3000))
    b = int(rng.integers(1, 5))
    kw = dict(hq=hq, hkv=hkv, d=128, batch=b, seed=700 + case, with_do=False,
              window=int(rng.choice([16, 128, 1024, 65536])),
              sink_logit=float(rng.choice([0.0, 8.0, 18.0, 30.0])),
              retrieval=int(rng.choice([0, 16, 64])))
    tau = float(rng.choice([1e-4, 1e-2, 1.0, 50.0]))
    split = str(rng.choice(["default", "auto", "multiple", "unsplit"]))
    lens = [int(v) for v in rng.integers(1, n + 1, size=b)]
    print(f"[random structured decode] case={case} n={n} tau={tau} split={split}", flush=True)
    x = W.make_structured(n, **kw)
    q = torch.stack([x["q"][i, :, lens[i] - 1] for i in range(b)]).to(DEV).contiguous()
    y = to_dev({"k_cache": x["k"], "v_cache": x["v"], "scale": x["scale"]})
    sk = {"default": 0, "auto": lib().DECODE_SPLIT_AUTO, "multiple": 64 * int(rng.integers(1, 30)),
          "unsplit": -(-max(lens) // 64) * 64}[split]
    check_decode(y, lens, tau, q, split_keys=sk, max_ties=8)


def test_decode_clamps_out_of_range_lengths():
    """seqlens_k outside [1, max_n_k] is clamped on the device (the header's
    contract): lengths 0 and 5000 with max_n_k = 701 give exactly the results
    of lengths 1 and 701."""
    m = lib()
    x = to_dev(W.make_decode(W.CONFIGS[5], cache=700, steps=1, batch=2, planted=4))
    q = x["q_steps"][0].contiguous()
    outs = []
    for lens in ([0, 5000], [1, 701]):
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        g = m.mala_decode(q, x["k_cache"], x["v_cache"], seq, 1e-4, max_n_k=701,
                          softmax_scale=x["scale"], want_mask=True)
        torch.cuda.synchronize()
        outs.append({k_: g[k_].cpu() for k_ in ("o", "lse", "mask", "kept")})
    for k_ in outs[0]:
        assert torch.equal(outs[0][k_], outs[1][k_]), k_


def test_decode_group16_and_single_key():
    x = W.make_decode(W.CONFIGS[5], cache=300, steps=1, batch=2, hq=16, hkv=1, planted=4)
    x = to_dev(x)
    check_decode(x, [1, 301], 1e-4, x["q_steps"][0].contiguous())


# ------------------------------------------------------------- empty / errors on device

def test_empty_query_rows():
    m = lib()
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.randn((1, 2, 5, 128), device=DEV).to(torch.bfloat16)
    out = m.mala_fwd(q, k, k, 1e-4)
    assert out["o"].shape == (1, 2, 0, 128)
    b = m.mala_bwd(q, k, k, out["o"], out["lse"], q, 1e-4)
    torch.cuda.synchronize()
    assert torch.count_nonzero(b["dk"]) == 0 and torch.count_nonzero(b["dv"]) == 0
    # the gate-pass walks, the nested call and the automatic choice (which
    # takes the gate-pass walks without rows to sample) write the zero dK, dV
    # themselves
    f = m.mala_fwd(q, k, k, 1e-4, want_mask=True)
    for kw in (dict(gate_pass=True), dict(fwd_mask=f["mask"]), dict(fwd_kept=f["kept"])):
        dk = torch.full_like(k, 7.0)
        g = m.mala_bwd(q, k, k, f["o"], f["lse"], q, 1e-4, out=dict(dk=dk), **kw)
        torch.cuda.synchronize()
        assert torch.count_nonzero(g["dk"]) == 0 and torch.count_nonzero(g["dv"]) == 0, kw


def test_fast_grad_flag_same_support():
    """MALA_FLAG_FAST_GRAD changes only the precision of dS in dQ: the
    decisions, dK and dV are identical and dQ stays within tolerance on the
    Gaussian workload."""
    m = lib()
    x = to_dev(W.make_prefill(W.CONFIGS[3], n=600, hq=4, hkv=1, planted=8))
    f = m.mala_fwd(x["q"], x["k"], x["v"], 1e-4, softmax_scale=x["scale"])
    a = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True)
    b = m.mala_bwd(x["q"], x["k"], x["v"], f["o"], f["lse"], x["do"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True, fast_grad=True)
    torch.cuda.synchronize()
    assert torch.equal(a["mask"], b["mask"])
    assert torch.equal(a["dv"], b["dv"])
    assert torch.equal(a["dk"], b["dk"])
    r = O.mala_fwd(np64(x["q"]), np64(x["k"]), np64(x["v"]), 1e-4, x["scale"], True,
                   *tiling()[0][:2], replay=m.mala_fwd(x["q"], x["k"], x["v"], 1e-4,
                   softmax_scale=x["scale"], want_mask=True)["mask"].cpu().numpy(), band=1e-3)
    rb = O.mala_bwd(np64(x["q"]), np64(x["k"]), np64(x["v"]), r["o"], r["lse"], np64(x["do"]),
                    1e-4, x["scale"], True, *tiling()[1][:2], o_storage="bf16", lse_storage="f32")
    bd = {}
    for split in (False, True):
        bd[split] = add_output_rounding(
            grad_rounding_bounds(np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(x["do"]), x["scale"],
                                 True, r, rb["mask"], "bf16", split_dq=split,
                                 lse_gpu=f["lse"].cpu().numpy(), o_gpu=np64(f["o"])), rb, "bf16")
    for name in ("dq", "dk"):
        compare_values(name + " fast", np64(b[name]), rb[name], "bf16", bound=bd[False][name])
        compare_values(name + " split", np64(a[name]), rb[name], "bf16", bound=bd[True][name])


# ------------------------------------------------------------- autograd entry

@pytest.mark.parametrize("mode", ["default", "gate_pass", "nested", "auto"])
def test_autograd_chunked_prefill_matches_direct_calls(mode):
    """mala_attention (torch.autograd) runs the same two C-ABI calls: its
    output and gradients equal mala_fwd / mala_bwd bit for bit, here on a
    chunked prefill (the last 100 of 356 positions query all 356 keys) whose
    inputs come from an upstream torch op, so the gradient flows through it.
    ``gate_pass`` is the backward with the separate score pass; ``nested``
    the backward on the forward's kept tiles (mala_bwd_nested)."""
    m = lib()
    x = to_dev(W.make_prefill(W.CONFIGS[2], n=356, hq=4, hkv=2, planted=4, seed=11))
    scale = x["scale"]
    base = x["q"][:, :, -100:].float().clone().requires_grad_()
    k = x["k"].clone().requires_grad_()
    v = x["v"].clone().requires_grad_()
    do = x["do"][:, :, -100:].contiguous()
    q = (base * 1.0).to(torch.bfloat16).contiguous()        # upstream op
    gp = "auto" if mode == "auto" else mode == "gate_pass"
    o = m.mala_attention(q, k, v, 1e-4, softmax_scale=scale, gate_pass=gp,
                         nested=mode == "nested")
    o.backward(do)
    qd = q.detach()
    f = m.mala_fwd(qd, k.detach(), v.detach(), 1e-4, softmax_scale=scale,
                   want_mask=mode == "nested")
    if mode == "auto":      # the walk the sampled backward decisions choose
        gm = m.mala_bwd(qd, k.detach(), v.detach(), f["o"], f["lse"], do, 1e-4,
                        softmax_scale=scale, gate_pass=True, want_mask=True)["mask"]
        gp = auto_takes_gate_pass(f["kept"], gm, 100, 356, True)
    b = m.mala_bwd(qd, k.detach(), v.detach(), f["o"], f["lse"], do, 1e-4, softmax_scale=scale,
                   gate_pass=gp, fwd_mask=f["mask"])
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), f["o"])
    assert torch.equal(base.grad, b["dq"].float())
    assert torch.equal(k.grad, b["dk"]) and torch.equal(v.grad, b["dv"])


# ------------------------------------------------------------- graph capture

def test_graph_capture_replays_match_eager():
    """The forward, the default and the automatic backward and a decode step
    captured in one HIP graph (torch.cuda.CUDAGraph): a call only launches
    kernels (no allocation, memset or synchronization inside it), so every
    replay gives the eager results bit for bit. Before each replay every
    output and workspace is overwritten with garbage and unrelated eager
    work runs, with synchronizations in between."""
    m = lib()
    x = to_dev(W.make_structured_preset("sparse", 1500, hq=8, hkv=2, d=128))
    q, k, v, do, sc = x["q"], x["k"], x["v"], x["do"], x["scale"]
    y = to_dev(W.make_decode(W.CONFIGS[5], cache=700, steps=1, batch=2, planted=4))
    qd = y["q_steps"][0].contiguous()
    seq = torch.tensor([701, 300], dtype=torch.int32, device=DEV)
    tau = 1e-2

    def step(bufs):
        f = m.mala_fwd(q, k, v, tau, softmax_scale=sc, out=bufs["f"])
        b = m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=sc, want_mask=True,
                       out=bufs["b"])
        a = m.mala_bwd(q, k, v, f["o"], f["lse"], do, tau, softmax_scale=sc, want_mask=True,
                       fwd_kept=f["kept"], out=bufs["a"])
        d = m.mala_decode(qd, y["k_cache"], y["v_cache"], seq, tau, max_n_k=701,
                          softmax_scale=y["scale"], want_mask=True, out=bufs["d"])
        return dict(f=f, b=b, a=a, d=d)

    eager = step({"f": {}, "b": {}, "a": {}, "d": {}})
    torch.cuda.synchronize()
    ref = {s_: {n: t.clone() for n, t in r.items() if isinstance(t, torch.Tensor) and n != "ws"}
           for s_, r in eager.items()}
    bufs = {s_: dict(r) for s_, r in eager.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(bufs)
    other = to_dev(W.make_prefill(W.CONFIGS[2], n=300, hq=2, hkv=2, planted=2, seed=5))
    for rep in range(3):
        for r in outs.values():
            for n, t in r.items():
                if isinstance(t, torch.Tensor):
                    t.fill_(7 if t.is_floating_point() else -3)
        m.mala_fwd(other["q"], other["k"], other["v"], 1e-4, softmax_scale=other["scale"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s_, r in ref.items():
            for n, t in r.items():
                assert torch.equal(outs[s_][n], t), (rep, s_, n)


# ------------------------------------------------------------- staged entry points

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_staged_entry_points_match_single_calls(dtype):
    """mala_bwd_stage (PREP, DKDV, DQ) and mala_decode_stage (SPLIT, COMBINE),
    the calls bench.py times one by one, give bit-identical results to
    mala_bwd and mala_decode, including the decisions and the counters."""
    m = lib()
    cfg = W.CONFIGS[2] if dtype == torch.bfloat16 else W.CONFIGS[1]
    x = W.make_prefill(cfg, n=300, hq=4, hkv=2, d=128 if dtype == torch.bfloat16 else 64,
                       planted=4, seed=21)
    x = to_dev({k: (v.to(dtype) if isinstance(v, torch.Tensor) else v) for k, v in x.items()})
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    f = m.mala_fwd(q, k, v, 1e-2, softmax_scale=x["scale"])
    a = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True)
    b = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True,
                   stages=(m.mala.BWD_PREP, m.mala.BWD_DKDV, m.mala.BWD_DQ))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "mask", "kept"):
        assert torch.equal(a[name], b[name]), name
    # the same with the gate pass, whose main stage is the gate, plan, walks
    # and finalize
    a = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True,
                   gate_pass=True)
    b = m.mala_bwd(q, k, v, f["o"], f["lse"], do, 1e-2, softmax_scale=x["scale"], want_mask=True,
                   gate_pass=True, stages=(m.mala.BWD_PREP, m.mala.BWD_DKDV, m.mala.BWD_DQ))
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "mask", "kept"):
        assert torch.equal(a[name], b[name]), ("gate pass", name)

    y = W.make_decode(W.CONFIGS[5], cache=700, steps=1, batch=2, planted=4)
    y = to_dev({k: (v.to(dtype) if isinstance(v, torch.Tensor) and v.is_floating_point() else v)
                for k, v in y.items()})
    if dtype == torch.float32:
        y["k_cache"], y["v_cache"] = y["k_cache"][..., :64].contiguous(), y["v_cache"][..., :64].contiguous()
        y["q_steps"] = y["q_steps"][..., :64].contiguous()
    qd = y["q_steps"][0].contiguous()
    seq = torch.tensor([701, 300], dtype=torch.int32, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    c = m.mala_decode(qd, y["k_cache"], y["v_cache"], seq, 1e-2, max_n_k=701, want_mask=True)
    e = m.mala_decode(qd, y["k_cache"], y["v_cache"], seq, 1e-2, max_n_k=701, want_mask=True,
                      events=ev)
    torch.cuda.synchronize()
    for name in ("o", "lse", "mask", "kept"):
        assert torch.equal(c[name], e[name]), name
