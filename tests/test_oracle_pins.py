"""Pins of the fp64 CPU oracle to facts it does not compute itself.

Each test checks one oracle function against something fixed outside the
oracle: numbers the pages print (tests/golden/), format specifications,
closed forms, limits that reduce to a textbook function, brute force on tiny
inputs, or invariants of the definition.  Each is chosen so that a plausible
slip (a dropped term, a wrong sign, a transposed operand, a wrong index)
fails it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class Shape:
    def __init__(self, **kw):
        self.beta, self.beta_u, self.rms_eps = 4.0, 25.0, 1e-6
        self.__dict__.update(kw)


def f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- pages' numbers -----------------------------------------------------------------

def test_param_counts_match_pages():
    """K3 layer shapes reproduce every parameter count the pages print."""
    cfg = synth.CONFIGS["k3_prefill_bf16"]
    sp = synth.specs(cfg)
    d, L, E, I = cfg.d, cfg.latent, cfg.n_experts, cfg.expert_inter
    expert = 3 * L * I
    counts = {
        "W_down projection 7168 -> 3584": sp["w_down_proj"].numel,
        "RMSNorm + W_up projection 3584 -> 7168": sp["w_up_proj"].numel,
        "router, 896 scores": sp["w_router"].numel,
        "one routed expert": expert,
        "all 896 routed experts of a layer": sp["w_gate"].numel + sp["w_up"].numel
        + sp["w_down"].numel,
        "16 active routed experts": cfg.top_k * expert,
        "2 shared experts at width 7168": sp["sh_gate"].numel + sp["sh_up"].numel
        + sp["sh_down"].numel,
        "W_down + W_up per layer": sp["w_down_proj"].numel + sp["w_up_proj"].numel,
        "dense layer-1 SiTU-GLU FFN, intermediate 33792": 3 * d * 33792,
        "routers over 92 MoE layers": 92 * sp["w_router"].numel,
        "shared experts over 92 MoE layers": 92 * (3 * d * cfg.shared_inter * cfg.n_shared),
        "W_down + W_up over 92 MoE layers": 92 * 2 * d * L,
        "routed experts over 92 MoE layers": 92 * E * expert,
    }
    items = json.load(open(os.path.join(GOLDEN, "param_counts.json")))["items"]
    assert len(items) == len(counts)
    for it in items:
        n = counts[it["what"]]
        assert round(n / it["unit"]) * it["unit"] == pytest.approx(it["value"], rel=1e-9), it
    # the expert width I = 3072 is the one that reproduces "33.0 M": neighbours do not
    assert round(3 * L * 3072 / 1e5) == 330
    assert round(3 * L * 3072 / 1e5) != round(3 * L * 3200 / 1e5)


# ---- storage decoders ----------------------------------------------------------------

def test_e4m3_decode_matches_ocp_table():
    for line in open(os.path.join(GOLDEN, "e4m3_codes.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = oracle.e4m3_to_double(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_decode_all_codes_monotone_and_exact():
    vals = [oracle.e4m3_to_double(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # 0x00..0x7E strictly increasing
    # every code is a 4-significant-bit dyadic number: v * 2^9 * 2^(e) exact
    for v in vals[1:]:
        m, e = math.frexp(v)
        assert (m * 16) == int(m * 16)


def test_bf16_decode():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x3F81) == 1.0 + 2.0 ** -7
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133


def test_fp8_block_scale_applied_per_block():
    """An fp8 matrix element decodes to code * scale of its own 128x128 block."""
    codes = np.full((256, 384), 0x38, np.uint8)  # every code = 1.0
    scales = f32(np.arange(1, 7).reshape(1, 2, 3))
    m = oracle.Mat(codes, scales)
    for (r, c, s) in [(0, 0, 1), (0, 127, 1), (0, 128, 2), (0, 383, 3), (128, 0, 4),
                      (255, 255, 5), (200, 300, 6)]:
        assert oracle.lib().orc_decode(m.ref, 0, r, c) == s


def _golden(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        out.append((int(code, 16), float(val)))
    return out


def test_e2m1_decode_matches_ocp_table():
    table = _golden("e2m1_codes.txt")
    assert len(table) == 16
    for code, val in table:
        got = oracle.e2m1_to_double(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e8m0_decode_matches_ocp_table():
    for code, val in _golden("e8m0_codes.txt"):
        got = oracle.e8m0_to_double(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val, hex(code)
    # every other code is a power of two, doubling per code
    for c in range(1, 255):
        assert oracle.e8m0_to_double(c) == 2 * oracle.e8m0_to_double(c - 1)


def _mx_table_decode(codes, e8):
    """Independent MXFP4 decode for the pins: the golden E2M1 table and the
    E8M0 doubling rule, element 2i in the low nibble of byte i."""
    table = np.array([v for _, v in _golden("e2m1_codes.txt")])
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[:-1] + (-1,))
    sc = np.ldexp(1.0, e8.astype(np.int64) - 127)
    return table[nib] * np.repeat(sc, 32, axis=-1)


def test_mxfp4_nibble_order_and_block_scale():
    """Element 2i is the low nibble of byte i, 2i+1 the high one; each element
    takes the E8M0 scale of its own row and 32-wide column block."""
    rows, cols = 3, 96
    codes = np.full((rows, cols // 2), 0x72, np.uint8)  # low nibble 1.0, high nibble 6.0
    e8 = np.array([[120, 127, 130], [1, 200, 126], [127, 127, 128]], np.uint8)
    m = oracle.Mat(codes, e8)
    assert m.c.cols == cols and m.c.dtype == oracle.MXFP4
    for r in range(rows):
        for c in (0, 1, 30, 31, 32, 33, 63, 64, 95):
            s = 2.0 ** (int(e8[r, c // 32]) - 127)
            assert oracle.lib().orc_decode(m.ref, 0, r, c) == (6.0 if c % 2 else 1.0) * s


def test_mxfp4_expert_equals_expert_on_decoded_values():
    """An expert with MXFP4 matrices gives exactly the expert on the same values
    written out in fp64-exact fp32 (decoded here from the spec tables)."""
    rng = np.random.default_rng(21)
    E, L, I = 2, 64, 96
    def mx(rows, cols):
        codes = rng.integers(0, 256, size=(E, rows, cols // 2), dtype=np.uint8)
        e8 = rng.integers(118, 124, size=(E, rows, cols // 32), dtype=np.uint8)
        return codes, e8
    (gc, ge), (uc, ue), (dc, de) = mx(I, L), mx(I, L), mx(L, I)
    x = rng.normal(size=L)
    s = Shape(latent=L, expert_inter=I)
    for e in range(E):
        a = oracle.expert(s, oracle.Mat(gc, ge), oracle.Mat(uc, ue), oracle.Mat(dc, de), x,
                          index=e)
        dec = [f32(_mx_table_decode(c[e], sc[e])) for c, sc in ((gc, ge), (uc, ue), (dc, de))]
        assert all((d.astype(np.float64) == _mx_table_decode(c[e], sc[e])).all()
                   for d, (c, sc) in zip(dec, ((gc, ge), (uc, ue), (dc, de))))
        b = oracle.expert(s, *(oracle.Mat(d) for d in dec), x)
        np.testing.assert_array_equal(a, b)


def _mx8_table_decode(codes, e8):
    """MX FP8 decode for the layout pins: the element values from the e4m3
    decoder (pinned above on the OCP table and on every code), the scale from
    the E8M0 doubling rule, placed here per row and 32-wide block."""
    table = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    sc = np.ldexp(1.0, e8.astype(np.int64) - 127)
    return table[codes] * np.repeat(sc, 32, axis=-1)


def test_mxfp8_matrix_element_and_block_scale():
    """An MX FP8 matrix holds one e4m3 code a byte; each element takes the E8M0
    scale of its own row and 32-wide column block (not a neighbour's)."""
    rows, cols = 3, 96
    codes = np.arange(rows * cols, dtype=np.int64).reshape(rows, cols) % 0x7E
    codes = (codes | ((np.arange(cols) % 3 == 0) * 0x80)).astype(np.uint8)  # some negatives
    e8 = np.array([[120, 127, 130], [1, 200, 126], [127, 127, 128]], np.uint8)
    m = oracle.Mat(codes, e8)
    assert m.c.cols == cols and m.c.dtype == oracle.MXFP8
    want = _mx8_table_decode(codes, e8)
    for r in range(rows):
        for c in (0, 1, 30, 31, 32, 33, 63, 64, 95):
            assert oracle.lib().orc_decode(m.ref, 0, r, c) == want[r, c]
    with pytest.raises(ValueError):
        oracle.Mat(codes[:, :80], e8)  # scales of a different row length


def test_mxfp8_expert_equals_expert_on_decoded_values():
    """An expert with MX FP8 matrices gives exactly the expert on the same values
    written out in fp64-exact fp32 (decoded here from the spec tables)."""
    rng = np.random.default_rng(23)
    E, L, I = 2, 64, 96
    def mx(rows, cols):
        codes = rng.integers(0, 256, size=(E, rows, cols), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x00  # no NaN codes
        e8 = rng.integers(110, 118, size=(E, rows, cols // 32), dtype=np.uint8)
        return codes, e8
    (gc, ge), (uc, ue), (dc, de) = mx(I, L), mx(I, L), mx(L, I)
    x = rng.normal(size=L)
    s = Shape(latent=L, expert_inter=I)
    for e in range(E):
        a = oracle.expert(s, oracle.Mat(gc, ge), oracle.Mat(uc, ue), oracle.Mat(dc, de), x,
                          index=e)
        dec = [f32(_mx8_table_decode(c[e], sc[e])) for c, sc in ((gc, ge), (uc, ue), (dc, de))]
        assert all((d.astype(np.float64) == _mx8_table_decode(c[e], sc[e])).all()
                   for d, (c, sc) in zip(dec, ((gc, ge), (uc, ue), (dc, de))))
        b = oracle.expert(s, *(oracle.Mat(d) for d in dec), x)
        np.testing.assert_array_equal(a, b)


# ---- scalar functions -----------------------------------------------------------------

def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, abs=1e-15)
    for z in (-7.5, -1.0, 0.3, 2.0, 11.0):
        assert oracle.sigmoid(z) + oracle.sigmoid(-z) == pytest.approx(1.0, abs=1e-15)


def test_situ_phi_pins():
    b = 4.0
    assert oracle.phi(0.0, b) == 0.0
    # slope at 0 is sigma(0) * beta * (1/beta) = 1/2, like SiLU
    h = 1e-6
    assert (oracle.phi(h, b) - oracle.phi(-h, b)) / (2 * h) == pytest.approx(0.5, rel=1e-8)
    # bounded above by beta, approached from below
    assert oracle.phi(60.0, b) == pytest.approx(b, rel=1e-12)
    assert all(oracle.phi(g, b) < b for g in np.linspace(-50, 50, 1001))
    # beta -> infinity reduces to SiLU g * sigmoid(g)
    for g in (-6.0, -1.3, 0.7, 2.5, 8.0):
        silu = g / (1.0 + math.exp(-g))
        assert oracle.phi(g, 1e7) == pytest.approx(silu, rel=1e-9)
    # below: |beta tanh(g/beta)| <= |g|, so phi >= min SiLU = -0.27846
    assert min(oracle.phi(g, b) for g in np.linspace(-20, 0, 4001)) >= -0.2785
    # the tanh cap bites: at g = beta*atanh(1/2) the capped factor is beta/2, not g
    g = b * math.atanh(0.5)
    assert oracle.phi(g, b) == pytest.approx((b / 2) / (1 + math.exp(-g)), rel=1e-14)


def test_situ_psi_pins():
    bu = 25.0
    assert oracle.psi(0.0, bu) == 0.0
    h = 1e-6
    assert (oracle.psi(h, bu) - oracle.psi(-h, bu)) / (2 * h) == pytest.approx(1.0, rel=1e-9)
    assert oracle.psi(1e4, bu) == pytest.approx(bu, rel=1e-15)
    for u in (0.5, 3.0, 40.0):
        assert oracle.psi(-u, bu) == -oracle.psi(u, bu)
        assert oracle.psi(u, 1e8) == pytest.approx(u, rel=1e-12)  # beta_u -> inf: identity
    assert oracle.psi(bu * math.atanh(0.5), bu) == pytest.approx(bu / 2, rel=1e-14)


# ---- step 1: router logits --------------------------------------------------------------

def test_router_logits_one_hot_weights_select_columns():
    """W_r with one 1 per row (expert e reads feature pi(e)) gives z = x[pi(e)] + b."""
    rng = np.random.default_rng(1)
    E, d, bt = 5, 9, 7
    pi = np.array([6, 0, 3, 8, 2])
    W = np.zeros((E, d), np.float32)
    W[np.arange(E), pi] = 1.0
    b = f32(rng.normal(size=E))
    x = f32(rng.normal(size=(bt, d)))
    w = oracle.Weights({"w_router": W, "router_bias": b})
    z = oracle.router_logits(Shape(d=d, n_experts=E), w, x)
    np.testing.assert_array_equal(z, x[:, pi].astype(np.float64) + b.astype(np.float64))
    # selected rows only
    z2 = oracle.router_logits(Shape(d=d, n_experts=E), w, x, rows=[4, 1])
    np.testing.assert_array_equal(z2, z[[4, 1]])


def test_router_logits_linear_in_x():
    rng = np.random.default_rng(2)
    E, d = 6, 32
    W = f32(rng.normal(size=(E, d)))
    a, c = f32(rng.integers(-3, 4, (3, d))), f32(rng.integers(-3, 4, (3, d)))
    w = oracle.Weights({"w_router": W, "router_bias": None})
    s = Shape(d=d, n_experts=E)
    za, zc = oracle.router_logits(s, w, a), oracle.router_logits(s, w, c)
    zs = oracle.router_logits(s, w, a + c)
    np.testing.assert_allclose(zs, za + zc, rtol=0, atol=1e-12)


def test_router_logits_bf16_exact_on_integers():
    """bf16 integers: the fp64 dot product is exact, equal to the integer dot."""
    rng = np.random.default_rng(3)
    E, d = 4, 64
    Wi = rng.integers(-8, 9, (E, d))
    xi = rng.integers(-2, 3, (2, d))
    bits = lambda a: ((a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    w = oracle.Weights({"w_router": bits(Wi), "router_bias": None})
    z = oracle.router_logits(Shape(d=d, n_experts=E), w, bits(xi))
    np.testing.assert_array_equal(z, (xi @ Wi.T).astype(np.float64))


# ---- step 2: batch quantile cutoff -------------------------------------------------------

def test_quantile_hand_example():
    col = None
    rows = []
    for line in open(os.path.join(GOLDEN, "quantile_tiny.txt")):
        if line.startswith("# column:"):
            col = [float(v) for v in line.split(":")[1].split()]
        elif line.strip() and not line.startswith("#"):
            rows.append(tuple(float(v) for v in line.split()))
    z = f32(np.array(col)[:, None])
    for m, v in rows:
        assert oracle.quantile(z, int(m))[0] == v


def test_quantile_order_statistic_definition_brute_force():
    """zeta is the value v of the column with #{z >= v} >= m > #{z > v}."""
    rng = np.random.default_rng(4)
    z = f32(rng.integers(-5, 6, (40, 6)))  # many duplicates
    for m in range(1, 41):
        zeta = oracle.quantile(z, m)
        for e in range(6):
            col = z[:, e]
            assert zeta[e] in col
            assert (col >= zeta[e]).sum() >= m > (col > zeta[e]).sum()


def test_quantile_rejects_bad_rank():
    z = f32(np.zeros((4, 2)))
    for m in (0, 5):
        with pytest.raises(ValueError):
            oracle.quantile(z, m)


# ---- step 3: top-k ---------------------------------------------------------------------

def _brute_topk(r, k):
    """The unique k-subset S with (r_a > r_b) or (r_a == r_b and a < b) for all a in S, b not in S."""
    E = len(r)
    found = []
    for S in itertools.combinations(range(E), k):
        out = [b for b in range(E) if b not in S]
        if all((r[a] > r[b]) or (r[a] == r[b] and a < b) for a in S for b in out):
            found.append(S)
    assert len(found) == 1
    return list(found[0])


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for E, k in ((6, 2), (7, 3), (5, 5), (8, 1)):
        z = f32(rng.integers(-3, 4, (30, E)))       # frequent ties
        alpha = f32(rng.integers(-1, 2, E))
        idx, w = oracle.topk(z, k, alpha=alpha)
        for t in range(z.shape[0]):
            r = (z[t] - alpha).astype(np.float32)
            assert list(idx[t]) == _brute_topk(r, k)


def test_topk_all_selected_when_k_equals_E():
    z = f32(np.random.default_rng(6).normal(size=(5, 4)))
    idx, _ = oracle.topk(z, 4)
    assert (idx == np.arange(4)).all()


def test_topk_weights_are_raw_scores_independent_of_cutoff():
    """w = sigmoid(z) at the chosen expert; a cutoff shift common to all experts
    keeps the choice and must not change w (w is not sigmoid(z - alpha))."""
    rng = np.random.default_rng(7)
    z = f32(rng.normal(size=(20, 9)))
    i0, w0 = oracle.topk(z, 3, alpha=f32(np.zeros(9)))
    i1, w1 = oracle.topk(z, 3, alpha=f32(np.full(9, 0.75)))
    np.testing.assert_array_equal(i0, i1)
    np.testing.assert_array_equal(w0, w1)
    assert oracle.topk(f32(np.zeros((1, 3))), 1)[1][0, 0] == 0.5


def test_topk_cutoff_moves_selection():
    """Raising one expert's cutoff can only remove it from tokens' choices."""
    rng = np.random.default_rng(8)
    z = f32(rng.normal(size=(200, 6)))
    base, _ = oracle.topk(z, 2)
    alpha = f32(np.zeros(6))
    alpha[2] = 1.0
    moved, _ = oracle.topk(z, 2, alpha=alpha)
    assert (moved == 2).sum() < (base == 2).sum()
    assert ((moved == 2) & ~(base == 2).any(1, keepdims=True)).sum() == 0


# ---- step 4: dispatch -----------------------------------------------------------------

def test_running_cutoff_step():
    """rate 1 follows the batch quantile, rate 0 keeps alpha; with dyadic values
    every step is exact: from alpha 0 toward zeta 1 at rate 1/2, alpha_n =
    1 - 2^-n (the geometric closed form of the moving average)."""
    z = np.array([1.0, -3.0, 0.25], np.float32)
    a = np.array([0.5, 2.0, -1.0], np.float32)
    np.testing.assert_array_equal(oracle.cutoff_update(a, z, 1.0), z)
    np.testing.assert_array_equal(oracle.cutoff_update(a, z, 0.0), a)
    alpha = np.zeros(1, np.float32)
    for n in range(1, 20):
        alpha = oracle.cutoff_update(alpha, np.ones(1, np.float32), 0.5)
        assert alpha[0] == 1.0 - 2.0 ** -n
    # a constant zeta is a fixed point
    np.testing.assert_array_equal(oracle.cutoff_update(z, z, 0.3), z)


def test_dispatch_invariants():
    for hot in (0, 5):
        idx = synth.routing_fixture(300, 4, 24, seed=3, hot=hot)
        counts, offsets, perm, inv = oracle.dispatch(idx, 24)
        flat = idx.reshape(-1)
        np.testing.assert_array_equal(counts, np.bincount(flat, minlength=24))
        assert counts.sum() == idx.size
        assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
        assert sorted(perm) == list(range(idx.size))
        np.testing.assert_array_equal(inv[perm], np.arange(idx.size))
        experts = flat[perm]
        assert (np.diff(experts) >= 0).all()
        tokens = perm // 4
        for e in range(24):
            seg = tokens[offsets[e]:offsets[e + 1]]
            assert (np.diff(seg) > 0).all()
        if hot:
            assert (counts == 0).sum() == 0 or counts[:hot].min() > counts[hot:].max() // 4


def test_dispatch_tiny_hand_example():
    idx = np.array([[0, 2], [1, 2], [0, 1]], np.int32)  # pairs p = 0..5
    counts, offsets, perm, inv = oracle.dispatch(idx, 4)
    assert list(counts) == [2, 2, 2, 0]
    assert list(offsets) == [0, 2, 4, 6, 6]
    assert list(perm) == [0, 4, 2, 5, 1, 3]
    assert list(inv) == [0, 4, 2, 5, 1, 3]


def test_dispatch_rejects_out_of_range_ids():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 9]], np.int32), 4)


# ---- step 6: expert SiTU-GLU -------------------------------------------------------------

def test_expert_reduces_to_swiglu_when_caps_vanish():
    """beta, beta_u -> inf: o = W_d (SiLU(W_g x) * (W_u x)), the textbook SwiGLU."""
    rng = np.random.default_rng(9)
    L, I = 6, 10
    Wg, Wu, Wd = (f32(rng.normal(size=s)) for s in ((I, L), (I, L), (L, I)))
    x = rng.normal(size=L)
    s = Shape(latent=L, expert_inter=I, beta=1e8, beta_u=1e8)
    o = oracle.expert(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x)
    g, u = Wg.astype(np.float64) @ x, Wu.astype(np.float64) @ x
    ref = Wd.astype(np.float64) @ (g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(o, ref, rtol=1e-9, atol=1e-12)


def test_expert_output_bounded():
    """|phi| < beta, |psi| < beta_u => |o_l| <= beta*beta_u*sum_i |W_d[l][i]|, even for huge inputs."""
    rng = np.random.default_rng(10)
    L, I = 8, 12
    Wg, Wu, Wd = (f32(rng.normal(size=s)) for s in ((I, L), (I, L), (L, I)))
    x = 1e4 * rng.normal(size=L)
    s = Shape(latent=L, expert_inter=I)
    o = oracle.expert(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x)
    bound = 4.0 * 25.0 * np.abs(Wd.astype(np.float64)).sum(1)
    assert (np.abs(o) <= bound).all() and np.abs(o).max() > 0.5 * bound.min()


def test_expert_picks_matrix_by_index():
    rng = np.random.default_rng(11)
    L, I, E = 4, 5, 3
    Wg, Wu = f32(rng.normal(size=(E, I, L))), f32(rng.normal(size=(E, I, L)))
    Wd = f32(rng.normal(size=(E, L, I)))
    x = rng.normal(size=L)
    s = Shape(latent=L, expert_inter=I)
    for e in range(E):
        a = oracle.expert(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x, index=e)
        b = oracle.expert(s, oracle.Mat(Wg[e]), oracle.Mat(Wu[e]), oracle.Mat(Wd[e]), x)
        np.testing.assert_array_equal(a, b)


# ---- dense layer-1 FFN ---------------------------------------------------------------------

def test_rmsnorm_closed_forms():
    # a constant row c: every element becomes c / sqrt(c^2 + eps) * gamma
    for c, eps in ((3.0, 0.0), (-0.5, 1e-6), (2.0, 0.25)):
        x = np.full(8, c)
        g = f32(np.arange(1, 9) / 4)
        np.testing.assert_allclose(oracle.rmsnorm(x, g, eps),
                                   c / math.sqrt(c * c + eps) * g.astype(np.float64),
                                   rtol=1e-15)
    # with eps = 0 the result has unit RMS and is exactly invariant to a power-of-two scale
    rng = np.random.default_rng(30)
    x = rng.normal(size=97)
    n = oracle.rmsnorm(x, None, 0.0)
    assert abs(np.sqrt(np.mean(n * n)) - 1.0) < 1e-14
    np.testing.assert_array_equal(oracle.rmsnorm(4.0 * x, None, 0.0), n)


def test_dense_ffn_structure():
    rng = np.random.default_rng(31)
    d, I = 24, 40
    Wg, Wu = f32(rng.normal(size=(I, d))), f32(rng.normal(size=(I, d)))
    Wd = f32(rng.normal(size=(d, I)))
    x, r = rng.normal(size=d), rng.normal(size=d)
    s = oracle.FfnShape(d, I, rms_eps=0.0)
    M = oracle.Mat
    y = oracle.dense_ffn(s, M(Wg), M(Wu), M(Wd), x, r)
    # the residual enters additively, exactly: y(r) - y(0) = r
    y0 = oracle.dense_ffn(s, M(Wg), M(Wu), M(Wd), x)
    np.testing.assert_array_equal(y - y0, (y0 + r) - y0)
    # gamma = 0 zeroes the FFN (phi(0) = psi(0) = 0): y = r
    np.testing.assert_array_equal(
        oracle.dense_ffn(s, M(Wg), M(Wu), M(Wd), x, r, gamma=np.zeros(d, np.float32)), r)
    # pre-norm: the output does not depend on the input's scale (eps = 0)
    np.testing.assert_array_equal(oracle.dense_ffn(s, M(Wg), M(Wu), M(Wd), 8.0 * x, r), y)
    # it is the expert GLU on the normalised row
    n = oracle.rmsnorm(x, None, 0.0)
    np.testing.assert_array_equal(y0, oracle.expert(s, M(Wg), M(Wu), M(Wd), n))


def test_dense_ffn_reduces_to_swiglu_when_caps_vanish():
    """beta, beta_u -> inf and a plain RMSNorm: the textbook pre-norm SwiGLU block."""
    rng = np.random.default_rng(32)
    d, I = 16, 28
    Wg, Wu = f32(rng.normal(size=(I, d))), f32(rng.normal(size=(I, d)))
    Wd = f32(rng.normal(size=(d, I)))
    x, r = rng.normal(size=d), rng.normal(size=d)
    s = oracle.FfnShape(d, I, beta=1e8, beta_u=1e8, rms_eps=1e-6)
    y = oracle.dense_ffn(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x, r)
    n = x / np.sqrt(np.mean(x * x) + 1e-6)
    g, u = Wg.astype(np.float64) @ n, Wu.astype(np.float64) @ n
    ref = r + Wd.astype(np.float64) @ (g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-12)


def test_dense_ffn_rejects_mismatched_shapes():
    d, I = 8, 12
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.dense_ffn(oracle.FfnShape(d, I), oracle.Mat(z((I, d), np.float32)),
                         oracle.Mat(z((I, d), np.float32)), oracle.Mat(z((I, d), np.float32)),
                         np.ones(d))


# ---- step 7: combine + latent RMSNorm ----------------------------------------------------

def test_combine_is_score_weighted_sum():
    L, k = 5, 3
    s = Shape(latent=L, top_k=k)
    o = np.zeros((k, L))
    o[0, 1], o[1, 3], o[2, 1] = 1.0, 1.0, 1.0
    ylat, _ = oracle.combine_norm(s, o, [0.25, 0.5, 0.125])
    np.testing.assert_array_equal(ylat, [0, 0.375, 0, 0.5, 0])


def test_rmsnorm_closed_form_and_unit_rms():
    L, k = 16, 2
    s = Shape(latent=L, top_k=k)
    c = 0.003
    o = np.full((k, L), c)
    _, n = oracle.combine_norm(s, o, [1.0, 0.0])
    np.testing.assert_allclose(n, c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    rng = np.random.default_rng(12)
    o = rng.normal(size=(k, L))
    ylat, n = oracle.combine_norm(s, o, [0.3, 0.6])
    ms = np.mean(ylat ** 2)
    assert math.sqrt(np.mean(n ** 2)) == pytest.approx(math.sqrt(ms / (ms + 1e-6)), rel=1e-13)
    # scale invariance and per-channel gamma
    _, n2 = oracle.combine_norm(s, 50 * o, [0.3, 0.6])
    np.testing.assert_allclose(n2, n * math.sqrt((ms + 1e-6) / (ms + 1e-6 / 2500)), rtol=1e-13)
    g = f32(np.linspace(0.5, 2, L))
    _, n3 = oracle.combine_norm(s, o, [0.3, 0.6], gamma=g)
    np.testing.assert_allclose(n3, n * g, rtol=1e-14)
    _, n0 = oracle.combine_norm(s, np.zeros((k, L)), [1.0, 1.0])
    assert (n0 == 0).all()


# ---- shared experts ----------------------------------------------------------------------

def test_two_shared_experts_equal_one_concatenated_glu():
    rng = np.random.default_rng(13)
    d, Is = 12, 7
    G, U = f32(rng.normal(size=(2, Is, d))), f32(rng.normal(size=(2, Is, d)))
    D = f32(rng.normal(size=(2, d, Is)))
    x = rng.normal(size=d)
    two = oracle.shared(Shape(d=d, n_shared=2, shared_inter=Is),
                        oracle.Weights({"sh_gate": G, "sh_up": U, "sh_down": D}), x)
    one = oracle.shared(Shape(d=d, n_shared=1, shared_inter=2 * Is),
                        oracle.Weights({"sh_gate": G.reshape(1, 2 * Is, d),
                                        "sh_up": U.reshape(1, 2 * Is, d),
                                        "sh_down": np.concatenate([D[0], D[1]], 1)[None]}), x)
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-12)
    zero = oracle.shared(Shape(d=d, n_shared=2, shared_inter=Is),
                         oracle.Weights({"sh_gate": G, "sh_up": U, "sh_down": D}),
                         np.zeros(d))
    assert (zero == 0).all()


# ---- whole layer ---------------------------------------------------------------------------

def _layer(cfg, seed=0, routing="normal"):
    return synth.host_layer(cfg, seed, routing)


TINY = synth.CONFIGS["tiny_fp32"]


def test_forward_zero_input_gives_zero_output():
    lay = _layer(TINY)
    lay["x"] = np.zeros_like(lay["x"])
    out = oracle.forward(TINY, lay, cutoff=oracle.GIVEN)
    assert (out["y"] == 0).all()
    # all logits tie at 0: the k lowest expert ids are chosen
    assert (out["idx"] == np.arange(TINY.top_k)).all()


def test_forward_invariant_to_expert_down_scale():
    """RMSNorm before W_up: scaling every W_d by c > 0 leaves y unchanged
    (exactly up to rounding when eps = 0)."""
    cfg = TINY.with_(rms_eps=0.0)
    lay = _layer(cfg)
    a = oracle.forward(cfg, lay)["y"]
    lay["w_down"] = f32(lay["w_down"] * 8.0)
    b = oracle.forward(cfg, lay)["y"]
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)


def test_forward_token_permutation_equivariant():
    lay = _layer(TINY)
    a = oracle.forward(TINY, lay)
    p = np.random.default_rng(14).permutation(TINY.bt)
    lay["x"] = np.ascontiguousarray(lay["x"][p])
    b = oracle.forward(TINY, lay)
    np.testing.assert_allclose(b["y"], a["y"][p], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(b["idx"], a["idx"][p])
    np.testing.assert_array_equal(b["zeta"], a["zeta"])


def test_forward_expert_relabel_invariant():
    lay = _layer(TINY)
    a = oracle.forward(TINY, lay)
    q = np.random.default_rng(15).permutation(TINY.n_experts)
    for n in ("w_router", "w_gate", "w_up", "w_down"):
        lay[n] = np.ascontiguousarray(lay[n][q])
    b = oracle.forward(TINY, lay)
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.sort(q[b["idx"]], 1), a["idx"])


def test_forward_equals_its_steps():
    """The whole-layer call and the per-token step functions agree (the large
    parity cases use the step functions)."""
    cfg = TINY
    lay = _layer(cfg)
    out = oracle.forward(cfg, lay)
    w = oracle.Weights(lay)
    z = oracle.router_logits(cfg, w, lay["x"])
    np.testing.assert_array_equal(z.astype(np.float32), out["z32"])
    zeta = oracle.quantile(z.astype(np.float32), cfg.quantile_rank)
    np.testing.assert_array_equal(zeta, out["zeta"])
    idx, wt = oracle.topk(z.astype(np.float32), cfg.top_k, alpha=zeta, z64=z)
    np.testing.assert_array_equal(idx, out["idx"])
    for t in (0, 17, 63):
        xt = lay["x"][t].astype(np.float64)
        xl = oracle.matvec(w.mats["w_down_proj"], xt)
        o = np.stack([oracle.expert(cfg, w.mats["w_gate"], w.mats["w_up"], w.mats["w_down"],
                                    xl, index=e) for e in idx[t]])
        _, n = oracle.combine_norm(cfg, o, wt[t], lay["gamma"])
        y = oracle.output(cfg, w, n, xt)
        np.testing.assert_allclose(y, out["y"][t], rtol=1e-13, atol=1e-13)


def test_batch_quantile_balances_zipf_skewed_load():
    """Quantile balancing drives each expert's count toward bt*k/E: under Zipf
    logit offsets plain top-k piles tokens on the first experts, the batch
    cutoffs do not."""
    cfg = synth.CONFIGS["tiny_fp32"].with_(bt=512, bias="zipf1.1")
    lay = _layer(cfg)
    given = oracle.forward(cfg, lay, cutoff=oracle.GIVEN)["counts"]
    batch = oracle.forward(cfg, lay, cutoff=oracle.BATCH)["counts"]
    mean = cfg.bt * cfg.top_k / cfg.n_experts
    assert given.max() > 3 * mean
    assert batch.max() < 1.6 * mean and batch.min() > 0.4 * mean


# ---- MX FP8 activations (the expert GEMMs' inputs in the block-scaled MFMA path) ---------

def test_e4m3_encode_round_trips_every_code_and_rounds_to_even():
    for code in list(range(0x7F)) + list(range(0x81, 0xFF)):
        assert oracle.double_to_e4m3(oracle.e4m3_to_double(code)) == code, hex(code)
    assert oracle.double_to_e4m3(-0.0) == 0x80
    assert oracle.double_to_e4m3(1.0625) == 0x38      # tie 1.0 / 1.125 -> even (1.0)
    assert oracle.double_to_e4m3(1.1875) == 0x3A      # tie 1.125 / 1.25 -> even (1.25)
    assert oracle.double_to_e4m3(2.0 ** -10) == 0x00  # subnormal tie 0 / 2^-9 -> 0
    assert oracle.double_to_e4m3(3 * 2.0 ** -10) == 0x02
    assert oracle.double_to_e4m3(447.0) == 0x7E and oracle.double_to_e4m3(1e6) == 0x7E
    assert oracle.double_to_e4m3(-1e6) == 0xFE


def test_e4m3_encode_is_nearest_by_brute_force():
    grid = np.array([oracle.e4m3_to_double(c) for c in range(0x7F)])  # 0 .. 448
    rng = np.random.default_rng(40)
    for v in np.concatenate([rng.normal(0, 30, 3000), rng.normal(0, 0.01, 1000)]):
        c = oracle.double_to_e4m3(v)
        d = np.abs(grid - min(abs(v), 448.0))
        assert abs(oracle.e4m3_to_double(c & 0x7F) - abs(v)) <= d.min() + 1e-300
        assert (c >> 7) == (v < 0)


def test_mx8_block_rules():
    rng = np.random.default_rng(41)
    x = rng.normal(0, 3, 32 * 20) * np.repeat(2.0 ** rng.integers(-20, 20, 20), 32)
    x[64:96] = 0.0  # an all-zero block
    codes, sc = oracle.mx8_quantize(x, 32)
    for b in range(20):
        blk = x[32 * b:32 * (b + 1)]
        amax = np.abs(blk).max()
        if amax == 0:
            assert sc[b] == 0 and not codes[32 * b:32 * (b + 1)].any()
            continue
        assert sc[b] == int(np.floor(np.log2(amax))) - 8 + 127
        top = codes[32 * b + int(np.argmax(np.abs(blk)))] & 0x7F
        assert 0x78 <= top <= 0x7E  # the block maximum lands in [256, 448]
        deq = np.array([oracle.e4m3_to_double(c) for c in codes[32 * b:32 * (b + 1)]]) * \
            2.0 ** (int(sc[b]) - 127)
        step = 2.0 ** (int(sc[b]) - 127)
        # within half an E4M3 ulp (relative 2^-4 for normals, 2^-10 * scale below them)
        assert np.all(np.abs(deq - blk) <= np.maximum(np.abs(blk) * 2.0 ** -4, step * 2.0 ** -10)
                      + np.where(np.abs(blk) > 448 * step, np.abs(blk) - 448 * step, 0))
    # a power-of-two scaling of a block only moves its shared exponent
    c2, s2 = oracle.mx8_quantize(x * 2.0 ** 5, 32)
    np.testing.assert_array_equal(c2, codes)
    nz = sc > 0
    np.testing.assert_array_equal(s2[nz], sc[nz] + 5)


def _bf16_rne(v):
    """bf16 rounding (ties to even) of normal doubles on their bit patterns:
    keep the top 7 of the 52 fraction bits."""
    u = np.asarray(v, np.float64).view(np.uint64)
    low = u & np.uint64((1 << 45) - 1)
    keep = u >> np.uint64(45)
    half = np.uint64(1 << 44)
    up = (low > half) | ((low == half) & ((keep & np.uint64(1)) == 1))
    return ((keep + up.astype(np.uint64)) << np.uint64(45)).view(np.float64)


def test_round_bf16():
    """The oracle's bf16 rounding: ties to even at 8 significant bits, carries
    into the exponent, subnormal steps of 2^-133, and agreement with torch's
    fp32 -> bf16 conversion (RNE) on fp32-exact values."""
    r = oracle.round_bf16
    assert r(1.0 + 2.0 ** -8) == 1.0                     # tie, even below
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie, even above
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert r(-(2.0 - 2.0 ** -9)) == -2.0                 # carry into the exponent
    assert r(3 * 2.0 ** -134) == 2.0 ** -132             # subnormal tie, even above
    assert r(2.0 ** -134) == 0.0                         # subnormal tie, even below
    assert r(0.0) == 0.0 and math.copysign(1.0, r(-0.0)) == -1.0
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(5).normal(size=4000).astype(np.float32) * \
        np.float32(2.0) ** np.random.default_rng(6).integers(-30, 30, 4000).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([r(float(a)) for a in v])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(_bf16_rne(v.astype(np.float64)), want)


def test_expert_with_mx8_inputs_is_the_quantised_composition():
    """act_mx_block = 32: gate/up read MX FP8 x_lat, down reads MX FP8 h (each
    rounded to bf16, then quantised in blocks of 32), composed from the pinned
    pieces."""
    rng = np.random.default_rng(42)
    L, I = 64, 96
    Wg, Wu = f32(rng.normal(size=(I, L)) / 8), f32(rng.normal(size=(I, L)) / 8)
    Wd = f32(rng.normal(size=(L, I)) / 10)
    x = rng.normal(size=L)

    def q(v):
        c, s = oracle.mx8_quantize(_bf16_rne(v), 32)
        return np.array([oracle.e4m3_to_double(k) for k in c]) * np.repeat(
            2.0 ** (s.astype(np.int64) - 127), 32)

    s = Shape(latent=L, expert_inter=I)
    s.act_quant = "mxfp8"
    o = oracle.expert(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x)
    xq = q(x)
    g, u = Wg.astype(np.float64) @ xq, Wu.astype(np.float64) @ xq
    h = np.array([oracle.phi(a) * oracle.psi(b) for a, b in zip(g, u)])
    np.testing.assert_allclose(o, Wd.astype(np.float64) @ q(h), rtol=1e-12, atol=1e-12)
    # and it differs from the exact expert by the quantisation only (a few per cent)
    s.act_quant = "none"
    o_exact = oracle.expert(s, oracle.Mat(Wg), oracle.Mat(Wu), oracle.Mat(Wd), x)
    rel = np.abs(o - o_exact).max() / np.abs(o_exact).max()
    assert 1e-4 < rel < 0.1


# ---- step 8: output projection plus the shared experts -----------------------------------
#
# y = W_up n + sum_j W_ds,j (phi(W_gs,j x) psi(W_us,j x)).  At g = u = +-1000 the
# SiTU factors sit exactly on their caps in fp64 (sigmoid(1000) = 1, tanh(250) =
# tanh(40) = 1, sigmoid(-1000) = 0), so every hidden value is exactly
# beta * beta_u = 100, -100 or 0, and with dyadic weights the whole output is an
# exact dyadic number: the expected values below are exact sums.

def _output_case(S=2):
    d, L, Is = 6, 4, 3
    # shared gate/up rows read x[0] only, with weight +1 or -1: g, u = +-1000
    sg = np.zeros((S, Is, d), np.float32)
    su = np.zeros((S, Is, d), np.float32)
    signs_g = np.array([[1, 1, -1], [1, -1, 1], [-1, 1, 1]][:S], np.float32)
    signs_u = np.array([[1, -1, 1], [-1, 1, 1], [1, 1, -1]][:S], np.float32)
    sg[:, :, 0], su[:, :, 0] = signs_g, signs_u
    # the hidden values those signs give at the caps: phi(+1000) = 4, phi(-1000) = 0,
    # psi(+-1000) = +-25
    h = np.where(signs_g > 0, 4.0, 0.0) * 25.0 * signs_u
    rng = np.random.default_rng(50)
    sd = (rng.integers(-8, 9, (S, d, Is)) / 8.0).astype(np.float32)   # dyadic
    wup = (rng.integers(-8, 9, (d, L)) / 16.0).astype(np.float32)     # dyadic
    n = rng.integers(-6, 7, L) / 4.0                                   # dyadic
    x = np.zeros(d)
    x[0], x[3] = 1000.0, 7.0  # x[3] meets only zero weights
    shp = Shape(d=d, latent=L, n_shared=S, shared_inter=Is)
    mats = {"w_up_proj": wup, "sh_gate": sg, "sh_up": su, "sh_down": sd}
    return shp, mats, x, n, h


def test_output_at_the_situ_caps_is_exact():
    """y equals W_up n plus every shared expert's W_ds h, bit for bit: a dropped
    routed term, a dropped or single shared expert, swapped gate/up, or a
    transposed W_ds or W_up all change y."""
    shp, mats, x, n, h = _output_case()
    y = oracle.output(shp, oracle.Weights(mats), n, x)
    routed = mats["w_up_proj"].astype(np.float64) @ n
    shared = sum(mats["sh_down"][j].astype(np.float64) @ h[j] for j in range(2))
    np.testing.assert_array_equal(y, routed + shared)
    assert np.abs(routed).max() > 0 and np.abs(shared).max() > 0
    assert not np.array_equal(y, routed) and not np.array_equal(y, shared)
    assert not np.array_equal(y, routed + mats["sh_down"][0].astype(np.float64) @ h[0])
    # the shared term alone (W_up = 0) is orc_shared, exactly
    z = dict(mats, w_up_proj=np.zeros_like(mats["w_up_proj"]))
    np.testing.assert_array_equal(oracle.output(shp, oracle.Weights(z), n, x), shared)
    np.testing.assert_array_equal(oracle.shared(shp, oracle.Weights(mats), x), shared)


def test_output_without_shared_experts_selects_latent_entries():
    """S = 0 and a one-hot W_up (row r picks entry p(r) of n): y is those entries
    of n, exactly."""
    d, L = 5, 4
    pick = [2, 0, 3, 3, 1]
    wup = np.zeros((d, L), np.float32)
    wup[np.arange(d), pick] = 1.0
    n = np.array([0.5, -1.25, 3.0, -0.75])
    shp = Shape(d=d, latent=L, n_shared=0, shared_inter=8)
    y = oracle.output(shp, oracle.Weights({"w_up_proj": wup}), n, np.ones(d))
    np.testing.assert_array_equal(y, n[pick])


def test_output_is_linear_in_w_up_only_through_the_routed_term():
    """Doubling W_up adds exactly W_up n: the shared term does not move."""
    shp, mats, x, n, _ = _output_case()
    y1 = oracle.output(shp, oracle.Weights(mats), n, x)
    y2 = oracle.output(shp, oracle.Weights(dict(mats, w_up_proj=2 * mats["w_up_proj"])), n, x)
    np.testing.assert_array_equal(y2 - y1, mats["w_up_proj"].astype(np.float64) @ n)
