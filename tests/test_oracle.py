"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-derived
closed forms (tests/golden/), a scalar brute force over every small tree, a
library attention routine (torch SDPA in float64) for the special cases the
pages name, high-precision mpmath for RoPE, and invariants of the mask.
The mutation tests at the end plant plausible mistakes into the oracle and
check that a pin catches each one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import bruteforce
from oracle import tv_oracle as O
from tree_verify_mla_tv_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _closed(s: str) -> float:
    """Evaluate the tiny closed-form vocabulary used by the golden files."""
    s = s.strip()
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    if s == "ln2":
        return math.log(2.0)
    for fn in ("cos", "sin"):
        for sign in ("", "-"):
            if s.startswith(f"{sign}{fn} "):
                v = getattr(math, fn)(float(s[len(sign) + 4:]))
                return -v if sign else v
    return float(Fraction(s))


def _rand_inputs(rng, B, q, H, P, d_c, d_r):
    kv = P + q
    return (rng.standard_normal((B, q, H, d_c)), rng.standard_normal((B, q, H, d_r)),
            rng.standard_normal((B, kv, d_c)), rng.standard_normal((B, kv, d_r)))


def _sdpa(q_lat, q_rope, c_kv, k_rope, mask, sm_scale):
    """torch SDPA in float64: q_cat = [q_lat, q_rope], k_cat = [c_kv, k_rope], v = c_kv.

    q_* [q,H,*], kv [kv,*], mask [q,kv] bool or None.  Returns out [q,H,d_c].
    """
    qc = torch.from_numpy(np.concatenate([q_lat, q_rope], -1)).permute(1, 0, 2)  # [H,q,E]
    kc = torch.from_numpy(np.concatenate([c_kv, k_rope], -1))[None].expand(qc.shape[0], -1, -1)
    v = torch.from_numpy(c_kv)[None].expand(qc.shape[0], -1, -1)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qc, kc.contiguous(), v.contiguous(),
                                                         attn_mask=m, scale=sm_scale)
    return o.permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# Trees and visibility
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bad", [[0, 0], [-1, 1], [-1, 0, 2], [-1, -1], [-1, 0, 5], [3]])
def test_invalid_trees_raise(bad):
    with pytest.raises(ValueError):
        O.validate_tree(np.array([bad]))


def test_depths_and_positions():
    parent = np.array([[-1, 0, 0, 1, 3, 2], [-1, 0, 1, 2, 3, 4]])
    assert O.tree_depths(parent).tolist() == [[0, 1, 1, 2, 3, 2], [0, 1, 2, 3, 4, 5]]
    assert O.node_positions(parent, 7).tolist() == [[7, 8, 8, 9, 10, 9], [7, 8, 9, 10, 11, 12]]
    kp = O.key_positions(parent, 3)
    assert kp.tolist() == [[0, 1, 2, 3, 4, 4, 5, 6, 5], [0, 1, 2, 3, 4, 5, 6, 7, 8]]


@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("P", [0, 1, 3])
def test_visibility_matches_transitive_closure(q_len, P):
    for tree in bruteforce.all_recursive_trees(q_len):
        vis = O.visibility(np.array([tree]), P)[0]
        for i, j in itertools.product(range(q_len), range(P + q_len)):
            assert vis[i, j] == bruteforce.visible_scalar(tree, P, i, j)


# ---------------------------------------------------------------------------
# Golden closed forms
# ---------------------------------------------------------------------------
def test_golden_sibling_tree():
    g = json.load(open(os.path.join(GOLDEN, "sibling_tree_closed_form.json")))
    B, H, P, q, d_c, d_r = (g[k] for k in ("B", "H", "prefix_len", "q_len", "d_c", "d_r"))
    q_lat = np.zeros((B, q, H, d_c))
    q_lat[0, :, 0, :] = [_closed(v) for v in g["q_lat_head0"]]
    q_lat[0, :, 1, :] = [_closed(v) for v in g["q_lat_head1"]]
    q_rope = np.zeros((B, q, H, d_r))
    c_kv = np.array([g["c_kv"]], dtype=np.float64)
    k_rope = np.array([g["k_rope"]], dtype=np.float64)
    out, lse = O.verify_attn(q_lat, q_rope, c_kv, k_rope, np.array(g["parent"]), P, g["sm_scale"])
    for h in (0, 1):
        exp_out = np.array([[_closed(v) for v in row] for row in g[f"expected_out_head{h}"]])
        exp_lse = np.array([_closed(v) for v in g[f"expected_lse_head{h}"]])
        np.testing.assert_allclose(out[0, :, h, :], exp_out, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, h], exp_lse, rtol=1e-14, atol=1e-14)


def test_golden_rope():
    g = json.load(open(os.path.join(GOLDEN, "rope_neox_closed_form.json")))
    for case in g["cases"]:
        y = O.rope_neox(np.array(case["x"], dtype=np.float64), np.array(case["pos"]), g["theta"])
        exp = np.array([_closed(v) for v in case["expected"]])
        np.testing.assert_allclose(y, exp, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# RoPE against high-precision complex rotation
# ---------------------------------------------------------------------------
def test_rope_matches_mpmath_complex_form():
    mpmath.mp.dps = 40
    rng = np.random.default_rng(11)
    for d_r, theta in ((4, 10000.0), (32, 10000.0), (64, 10000.0), (64, 500000.0)):
        x = rng.standard_normal((6, d_r))
        pos = np.array([0, 1, 7, 513, 2064, 8224])
        y = O.rope_neox(x, pos, theta)
        half = d_r // 2
        for r in range(x.shape[0]):
            for k in range(half):
                # Textbook complex form: (x1 + i x2) * exp(i * pos * theta^(-2k/d)).
                ang = mpmath.mpf(int(pos[r])) * mpmath.power(mpmath.mpf(theta), -mpmath.mpf(2 * k) / d_r)
                z = mpmath.mpc(x[r, k], x[r, k + half]) * mpmath.expjpi(ang / mpmath.pi)
                assert abs(float(z.real) - y[r, k]) <= 1e-12 * (1 + abs(float(z.real)))
                assert abs(float(z.imag) - y[r, k + half]) <= 1e-12 * (1 + abs(float(z.imag)))


def test_rope_invariants():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 64))
    a = rng.standard_normal(64)
    b = rng.standard_normal(64)
    # Identity at position 0, exactly.
    assert np.array_equal(O.rope_neox(x, np.zeros(5), 10000.0), x)
    # Each (k, k + d/2) pair keeps its norm.
    y = O.rope_neox(x, np.array([1, 10, 100, 1000, 8000]), 10000.0)
    np.testing.assert_allclose(y[:, :32] ** 2 + y[:, 32:] ** 2, x[:, :32] ** 2 + x[:, 32:] ** 2, rtol=1e-13)
    # Relative-position property: <R(p+t)a, R(p'+t)b> depends on p - p' only.
    for p, pp, t in ((5, 2, 100), (8192, 8100, 33), (0, 40, 7)):
        lhs = O.rope_neox(a, np.array(p + t), 1e4) @ O.rope_neox(b, np.array(pp + t), 1e4)
        rhs = O.rope_neox(a, np.array(p), 1e4) @ O.rope_neox(b, np.array(pp), 1e4)
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(rhs))


def test_rope_single_rounding_f32():
    """Stored result = exact rotation (float64 cos/sin) rounded once to fp32."""
    mpmath.mp.dps = 50
    rng = np.random.default_rng(13)
    x = rng.standard_normal((400, 64)).astype(np.float32).astype(np.float64)
    pos = rng.integers(0, 9000, size=400)
    got = O.rope_neox_stored(x, pos, 10000.0, "f32")
    inv = O.rope_inv_freq(64, 10000.0)
    mism = 0
    for r in range(0, 400, 7):
        ang = float(pos[r]) * inv
        c, s = np.cos(ang), np.sin(ang)
        for k in range(32):
            e1 = mpmath.mpf(x[r, k]) * mpmath.mpf(c[k]) - mpmath.mpf(x[r, k + 32]) * mpmath.mpf(s[k])
            e2 = mpmath.mpf(x[r, k + 32]) * mpmath.mpf(c[k]) + mpmath.mpf(x[r, k]) * mpmath.mpf(s[k])
            for e, g in ((e1, got[r, k]), (e2, got[r, k + 32])):
                f = np.float32(float(e))  # float(mpf) is one correct rounding to float64
                mism += int(float(f) != g)
    assert mism == 0


def _bf16_rne_fraction(x: float) -> float:
    """Nearest bf16 to x (ties to even), by exact rational comparison."""
    if x == 0:
        return 0.0
    fx = Fraction(x)
    e = math.frexp(abs(x))[1]  # |x| in [2^(e-1), 2^e)
    ulp = Fraction(2) ** (e - 8)
    lo = (abs(fx) // ulp) * ulp
    hi = lo + ulp
    d_lo, d_hi = abs(fx) - lo, hi - abs(fx)
    if d_lo < d_hi or (d_lo == d_hi and (lo / ulp) % 2 == 0):
        r = lo
    else:
        r = hi
    return float(r) if x > 0 else -float(r)


def test_round_to_bf16_single_rounding():
    rng = np.random.default_rng(14)
    vals = list(rng.standard_normal(2000) * 3.0)
    # Exact ties, and float64 values one ulp either side of a bf16 midpoint: a
    # detour through fp32 would round these to the midpoint and then tie to even.
    for base in (1.0, 1.5, -2.25, 0.3):
        bits = np.float32(base).view(np.uint32) & np.uint32(0xFFFF0000)
        lo = float(np.uint32(bits).view(np.float32))
        mid = lo + math.ldexp(1.0, math.frexp(abs(lo))[1] - 9) * (1 if lo > 0 else -1)
        vals += [mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)]
    got = O.round_to_bf16(np.array(vals))
    for v, g in zip(vals, got):
        assert g == _bf16_rne_fraction(float(v)), v


def test_bf16_bits_roundtrip():
    rng = np.random.default_rng(15)
    x = rng.standard_normal(1000)
    r = O.round_to_bf16(x)
    assert np.array_equal(O.bf16_bits_to_f64(O.f64_to_bf16_bits(r)), r)
    # The generator's fp32->bf16 rounding agrees with the oracle's float64->bf16 one
    # on fp32 inputs (both are a single round-to-nearest-even).
    x32 = x.astype(np.float32)
    assert np.array_equal(O.bf16_bits_to_f64(W.f32_to_bf16_bits(x32)), O.round_to_bf16(x32.astype(np.float64)))


# ---------------------------------------------------------------------------
# Attention: brute force over every small tree
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("P", [0, 1, 3])
def test_attention_brute_force_all_trees(q_len, P):
    rng = np.random.default_rng(100 * q_len + P)
    H, d_c, d_r = 2, 3, 2
    for tree in bruteforce.all_recursive_trees(q_len):
        ql, qr, ck, kr = _rand_inputs(rng, 1, q_len, H, P, d_c, d_r)
        out, lse, probs = O.verify_attn(ql, qr, ck, kr, np.array([tree]), P, 0.37, return_probs=True)
        so, sl = bruteforce.verify_attn_scalar(ql, qr, ck, kr, [tree], P, 0.37)
        np.testing.assert_allclose(out, np.array(so), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(sl), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-12)


def test_attention_vs_sdpa_random_tree_mask():
    rng = np.random.default_rng(21)
    B, q, H, P, d_c, d_r = 2, 17, 4, 40, 32, 16
    ql, qr, ck, kr = _rand_inputs(rng, B, q, H, P, d_c, d_r)
    parent = np.stack([W.tree_rrt(q, rng), W.tree_branch(q, rng)])
    out, lse = O.verify_attn(ql, qr, ck, kr, parent, P, 0.11)
    for b in range(B):
        A = np.array(bruteforce.ancestor_closure(list(parent[b])))
        mask = np.concatenate([np.ones((q, P), bool), A], axis=1)
        ref = _sdpa(ql[b], qr[b], ck[b], kr[b], mask, 0.11)
        np.testing.assert_allclose(out[b], ref, rtol=1e-11, atol=1e-12)
        s = 0.11 * (np.einsum("qhd,kd->qhk", ql[b], ck[b]) + np.einsum("qhd,kd->qhk", qr[b], kr[b]))
        s = np.where(mask[:, None, :], s, -np.inf)
        np.testing.assert_allclose(lse[b], logsumexp(s, axis=-1), rtol=1e-12)


@pytest.mark.parametrize("P", [0, 1, 64])
def test_chain_tree_equals_causal(P):
    """A pure chain is ordinary causal attention (the greedy-equivalence case)."""
    rng = np.random.default_rng(22 + P)
    q, H, d_c, d_r = 9, 3, 16, 8
    ql, qr, ck, kr = _rand_inputs(rng, 1, q, H, P, d_c, d_r)
    out, _ = O.verify_attn(ql, qr, ck, kr, W.tree_chain(q)[None], P, 0.2)
    if P == 0:
        qc = torch.from_numpy(np.concatenate([ql[0], qr[0]], -1)).permute(1, 0, 2)
        kc = torch.from_numpy(np.concatenate([ck[0], kr[0]], -1))[None].expand(H, -1, -1).contiguous()
        v = torch.from_numpy(ck[0])[None].expand(H, -1, -1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qc, kc, v, is_causal=True, scale=0.2)
        ref = ref.permute(1, 0, 2).numpy()
    else:
        mask = np.arange(P + q)[None, :] <= (P + np.arange(q))[:, None]
        ref = _sdpa(ql[0], qr[0], ck[0], kr[0], mask, 0.2)
    np.testing.assert_allclose(out[0], ref, rtol=1e-11, atol=1e-12)


def test_single_node_is_full_attention():
    """q_len = 1 (autoregressive decode, budget 0) attends to every kv row."""
    rng = np.random.default_rng(23)
    ql, qr, ck, kr = _rand_inputs(rng, 1, 1, 4, 50, 16, 8)
    out, _ = O.verify_attn(ql, qr, ck, kr, np.array([[-1]]), 50, 0.3)
    ref = _sdpa(ql[0], qr[0], ck[0], kr[0], None, 0.3)
    np.testing.assert_allclose(out[0], ref, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Mask invariants
# ---------------------------------------------------------------------------
def test_non_ancestors_do_not_matter():
    rng = np.random.default_rng(24)
    B, q, H, P, d_c, d_r = 1, 12, 3, 5, 8, 4
    ql, qr, ck, kr = _rand_inputs(rng, B, q, H, P, d_c, d_r)
    parent = W.tree_rrt(q, rng)[None]
    out, lse = O.verify_attn(ql, qr, ck, kr, parent, P, 0.5)
    for i in range(q):
        anc = set(O.ancestors_of(parent[0], i))
        ck2, kr2 = ck.copy(), kr.copy()
        for m in range(q):
            if m not in anc:
                ck2[0, P + m] += 1e4 * rng.standard_normal(d_c)
                kr2[0, P + m] -= 1e4
        out2, lse2 = O.verify_attn(ql, qr, ck2, kr2, parent, P, 0.5)
        assert np.array_equal(out2[0, i], out[0, i]) and np.array_equal(lse2[0, i], lse[0, i])


def test_zero_queries_give_visible_mean():
    rng = np.random.default_rng(25)
    B, q, H, P, d_c, d_r = 2, 9, 2, 6, 8, 4
    _, _, ck, kr = _rand_inputs(rng, B, q, H, P, d_c, d_r)
    parent = np.stack([W.tree_rrt(q, rng) for _ in range(B)])
    out, lse = O.verify_attn(np.zeros((B, q, H, d_c)), np.zeros((B, q, H, d_r)), ck, kr, parent, P, 1.0)
    depth = O.tree_depths(parent)
    for b in range(B):
        for i in range(q):
            rows = list(range(P)) + [P + m for m in O.ancestors_of(parent[b], i)]
            assert len(rows) == P + depth[b, i] + 1
            np.testing.assert_allclose(out[b, i], np.broadcast_to(ck[b, rows].mean(0), (H, d_c)), rtol=1e-13)
            np.testing.assert_allclose(lse[b, i], math.log(len(rows)), rtol=1e-14)


def test_constant_latent_gives_ones():
    rng = np.random.default_rng(26)
    ql, qr, _, kr = _rand_inputs(rng, 2, 7, 3, 4, 8, 4)
    parent = np.stack([W.tree_rrt(7, rng) for _ in range(2)])
    out, _ = O.verify_attn(ql, qr, np.ones((2, 11, 8)), kr, parent, 4, 0.4)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-15)


def test_root_without_prefix_copies_its_row():
    rng = np.random.default_rng(27)
    ql, qr, ck, kr = _rand_inputs(rng, 2, 6, 3, 0, 8, 4)
    parent = np.stack([W.tree_rrt(6, rng) for _ in range(2)])
    out, lse = O.verify_attn(ql, qr, ck, kr, parent, 0, 0.4)
    for b in range(2):
        assert np.array_equal(out[b, 0], np.broadcast_to(ck[b, 0], (3, 8)))


def test_relabelling_permutes_outputs():
    """Another topological numbering of the same tree permutes the outputs."""
    rng = np.random.default_rng(28)
    q, H, P, d_c, d_r = 8, 2, 3, 6, 4
    ql, qr, ck, kr = _rand_inputs(rng, 1, q, H, P, d_c, d_r)
    parent = W.tree_rrt(q, rng)
    # Relabel by a breadth-first order (root first), which is topological.
    order = [0]
    for n in order:
        order += [c for c in range(q) if parent[c] == n]
    new_of = {old: new for new, old in enumerate(order)}
    parent2 = np.array([-1 if parent[old] < 0 else new_of[int(parent[old])] for old in order])
    perm = np.array(order)
    ck2 = np.concatenate([ck[:, :P], ck[:, P + perm]], axis=1)
    kr2 = np.concatenate([kr[:, :P], kr[:, P + perm]], axis=1)
    out, lse = O.verify_attn(ql, qr, ck, kr, parent[None], P, 0.3)
    out2, lse2 = O.verify_attn(ql[:, perm], qr[:, perm], ck2, kr2, parent2[None], P, 0.3)
    np.testing.assert_allclose(out2[0], out[0, perm], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2[0], lse[0, perm], rtol=1e-13)


# ---------------------------------------------------------------------------
# The whole step (RoPE at tree positions + attention)
# ---------------------------------------------------------------------------
def _complex_rope(x, pos, theta):
    """Independent rotation: complex multiply of (x1 + i x2) by exp(i ang)."""
    d = x.shape[-1]
    k = np.arange(d // 2)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * np.power(theta, -2.0 * k / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], -1)


def test_step_chain_equals_causal_with_rope():
    """A chain tree: every node turns at prefix+i, keys at their own index."""
    w = W.WORKLOADS["b2_h8_p0_q9_chain"]
    inp = W.make_inputs(w)
    P = 6
    rng = np.random.default_rng(29)
    q, H = w.q_len, w.H
    ql = rng.standard_normal((1, q, H, 16)).astype(np.float32)
    qr = rng.standard_normal((1, q, H, 8)).astype(np.float32)
    ck = rng.standard_normal((1, P + q, 16)).astype(np.float32)
    kr = rng.standard_normal((1, P + q, 8)).astype(np.float32)
    res = O.verify_step(ql, qr, ck, kr, W.tree_chain(q)[None], P, 10000.0, 0.25, "f32")
    qrot = _complex_rope(qr[0].astype(np.float64), (P + np.arange(q))[:, None], 10000.0)
    krot = _complex_rope(kr[0].astype(np.float64), np.arange(P + q), 10000.0)
    np.testing.assert_allclose(res["q_rope"][0], qrot, rtol=0, atol=4e-7)  # one fp32 rounding
    np.testing.assert_allclose(res["k_rope"][0], krot, rtol=0, atol=4e-7)
    mask = np.arange(P + q)[None, :] <= (P + np.arange(q))[:, None]
    ref = _sdpa(ql[0].astype(np.float64), res["q_rope"][0], ck[0].astype(np.float64), res["k_rope"][0],
                mask, 0.25)
    np.testing.assert_allclose(res["out"][0], ref, rtol=1e-11, atol=1e-12)
    assert inp["parent"].tolist() == [list(range(-1, q - 1))] * w.B


def test_step_bf16_cache_rounding():
    w = W.WORKLOADS["tiny_b3_h8_p1_q5"]
    inp = W.make_inputs(w)
    ck = W.f32_to_bf16_bits(inp["c_kv"])
    kr = W.f32_to_bf16_bits(inp["k_rope"])
    res = O.verify_step(inp["q_lat"], inp["q_rope"], ck, kr, inp["parent"], w.prefix_len, w.theta,
                        w.sm_scale, "bf16")
    # Rotated keys are exact bf16 values: re-rounding changes nothing.
    assert np.array_equal(O.round_to_bf16(res["k_rope"]), res["k_rope"])
    pos_k = O.key_positions(inp["parent"], w.prefix_len)
    exact = _complex_rope(O.bf16_bits_to_f64(kr), pos_k, w.theta)
    assert np.max(np.abs(res["k_rope"] - exact) / np.maximum(np.abs(exact), 1e-3)) <= 2.0 ** -8


# ---------------------------------------------------------------------------
# Mutation checks: plausible mistakes planted in the oracle fail a pin.
# ---------------------------------------------------------------------------
def _brute_small_fails():
    try:
        test_attention_brute_force_all_trees(4, 1)
    except AssertionError:
        return True
    return False


def test_mutation_self_not_visible(monkeypatch):
    monkeypatch.setattr(O, "ancestors_of", lambda row, i: [n for n in _walk(row, i) if n != i])
    assert _brute_small_fails()


def test_mutation_sibling_visible(monkeypatch):
    def leaky(row, i):
        a = _walk(row, i)
        return a + [n for n in range(len(row)) if n not in a and n < i]
    monkeypatch.setattr(O, "ancestors_of", leaky)
    assert _brute_small_fails()


def test_mutation_dropped_rope_term(monkeypatch):
    real = O.verify_attn

    def dropped(q_lat, q_rope, c_kv, k_rope, *a, **k):
        return real(q_lat, np.zeros_like(np.asarray(q_rope, float)), c_kv, k_rope, *a, **k)
    monkeypatch.setattr(O, "verify_attn", dropped)
    with pytest.raises(AssertionError):
        test_attention_vs_sdpa_random_tree_mask()


def test_mutation_rope_sign_and_pairing(monkeypatch):
    real = O.rope_neox
    monkeypatch.setattr(O, "rope_neox", lambda x, pos, theta: real(x, -np.asarray(pos), theta))
    with pytest.raises(AssertionError):
        test_rope_matches_mpmath_complex_form()
    with pytest.raises(AssertionError):
        test_golden_rope()

    def interleaved(x, pos, theta):
        x = np.asarray(x, float)
        d = x.shape[-1]
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        inv = np.argsort(perm)
        return real(x[..., perm], pos, theta)[..., inv]
    monkeypatch.setattr(O, "rope_neox", interleaved)
    with pytest.raises(AssertionError):
        test_golden_rope()


def test_mutation_inv_freq_exponent(monkeypatch):
    monkeypatch.setattr(O, "rope_inv_freq", lambda d, theta: 1.0 / theta ** (np.arange(d // 2) / d))
    with pytest.raises(AssertionError):
        test_golden_rope()


def test_mutation_positions_off_by_one(monkeypatch):
    real = O.node_positions
    monkeypatch.setattr(O, "node_positions", lambda p, P: real(p, P) + 1)
    with pytest.raises(AssertionError):
        test_step_chain_equals_causal_with_rope()


def _walk(row, i):
    out, n = [], int(i)
    while n != -1:
        out.append(n)
        n = int(row[n])
    return out
