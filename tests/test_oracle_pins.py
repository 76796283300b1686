"""Pins for the CPU oracle: every check compares the oracle with something
other than itself -- a closed form, a hand-computed value, a worked example
from the pages, brute force with exact rationals, or a library routine.

All of these run on the CPU (no GPU marker)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
T24 = np.float32(2.0 ** 24)  # 2^24 + 1 is not a float32; it is a tie that rounds to 2^24


def seg_bounds(N, R, c):
    S = -(-N // R)
    return min(c * S, N), min((c + 1) * S, N)


# ---------------------------------------------------------------- pages' examples

def test_pages_worked_examples(orc):
    g = json.load(open(os.path.join(GOLDEN, "collectives_4gpu.json")))
    x = np.array(g["allreduce"]["input"], dtype=np.int32)
    want = np.array(g["allreduce"]["every_rank"], dtype=np.int32)
    for y in (orc.ring_allreduce(x), orc.tree_allreduce(x)):
        assert (y == want[None, :]).all()
        assert y.shape == (4, 4)
    x = np.array(g["reduce_scatter"]["input"], dtype=np.int32)
    assert (orc.ring_reduce_scatter(x) == np.array(g["reduce_scatter"]["shards"])).all()
    x = np.array(g["all_gather"]["input"], dtype=np.int32)
    want = np.array(g["all_gather"]["every_rank"], dtype=np.int32)
    assert (orc.ring_all_gather(x) == want[None, :]).all()


def test_tree_shape_r8_matches_worked_listing(orc):
    g = json.load(open(os.path.join(GOLDEN, "double_binary_tree_r8.json")))
    for t, key in ((0, "tree_a_children"), (1, "tree_b_children")):
        par = orc.tree_parents(8, t)
        kids = {}
        for r, p in enumerate(par):
            if p >= 0:
                kids.setdefault(p, []).append(r)
        assert {str(k): sorted(v) for k, v in kids.items()} == g[key]


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("R", [2, 3, 4, 5, 7, 8, 16])
@pytest.mark.parametrize("N", [0, 1, 3, 7, 64, 1000, 4097])
def test_int32_equals_integer_sum(orc, R, N):
    rng = np.random.default_rng(R * 1000 + N)
    x = rng.integers(-(2 ** 31), 2 ** 31, size=(R, N), dtype=np.int64).astype(np.int32)
    want = (x.astype(np.int64).sum(axis=0) % (2 ** 32)).astype(np.uint32).view(np.int32)
    for y in (orc.ring_allreduce(x), orc.tree_allreduce(x)):
        assert y.shape == (R, N)
        assert (y == want[None, :]).all()
    if N % R == 0:
        rs = orc.ring_reduce_scatter(x)
        assert (rs.reshape(-1) == want).all()


@pytest.mark.parametrize("R", [2, 3, 8, 16])
@pytest.mark.parametrize("N", [1, 5, 33, 1024])
def test_rank_id_pattern(orc, R, N):
    # x_r[e] = r + R*e  =>  sum = R(R-1)/2 + R^2 e   (mod 2^32)
    e = np.arange(N, dtype=np.int64)
    x = np.stack([(r + R * e) for r in range(R)]).astype(np.int32)
    want = ((R * (R - 1) // 2 + R * R * e) % (2 ** 32)).astype(np.uint32).view(np.int32)
    assert (orc.ring_allreduce(x) == want).all()
    assert (orc.tree_allreduce(x) == want).all()


@pytest.mark.parametrize("dtype", ["int32", "float32", "bf16"])
@pytest.mark.parametrize("R", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("N", [0, 1, 2, 7, 8, 13, 100])
def test_all_ones_give_R(orc, dtype, R, N):
    if dtype == "int32":
        x = np.ones((R, N), np.int32)
        want = np.full(N, R, np.int32)
    elif dtype == "float32":
        x = np.ones((R, N), np.float32)
        want = np.full(N, R, np.float32)
    else:
        x = np.full((R, N), 0x3F80, np.uint16)  # bf16 1.0
        # R is a small integer, exactly representable: its bf16 pattern is
        # the top half of the float32 pattern.
        want = np.full(N, np.float32(R).view(np.uint32) >> 16, np.uint16)
    for y in (orc.ring_allreduce(x, dtype), orc.tree_allreduce(x, dtype)):
        assert (y == want[None, :]).all()
    if dtype == "bf16" and R == 16 and N:
        assert orc.ring_allreduce(x, dtype)[0, 0] == 0x4180  # bf16 16.0


@pytest.mark.parametrize("R", [2, 4, 8, 16])
def test_integer_valued_floats_are_order_free(orc, R):
    # |partial| <= 16 * 1000 < 2^24: every float32 partial is exact, so any
    # order gives the exact integer sum.
    rng = np.random.default_rng(R)
    x = rng.integers(-1000, 1001, size=(R, 999)).astype(np.float32)
    want = x.astype(np.int64).sum(axis=0).astype(np.float32)
    assert (orc.ring_allreduce(x) == want).all()
    assert (orc.tree_allreduce(x) == want).all()


def test_bf16_integer_inputs_round_once(orc):
    # bf16 integers in [-128, 128] are exact; fp32 partials are exact; the one
    # rounding of the exact sum must equal torch's float32 -> bf16 of it.
    import torch
    R, N = 16, 2000
    rng = np.random.default_rng(7)
    xi = rng.integers(-128, 129, size=(R, N))
    x = torch.tensor(xi, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    exact = torch.tensor(xi.sum(axis=0), dtype=torch.float32)
    want = exact.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (orc.ring_allreduce(x, "bf16") == want).all()
    assert (orc.tree_allreduce(x, "bf16") == want).all()
    assert (orc.ring_reduce_scatter(x, "bf16").reshape(-1) == want).all()


# ---------------------------------------------------------------- structure

@pytest.mark.parametrize("R", [2, 3, 4, 5, 6, 8, 9, 16])
def test_every_rank_identical_and_rs_ag_is_ar(orc, R):
    rng = np.random.default_rng(100 + R)
    for dtype in ("float32", "bf16", "int32"):
        N = R * 37
        if dtype == "int32":
            x = rng.integers(-1000, 1001, size=(R, N)).astype(np.int32)
        elif dtype == "float32":
            x = rng.standard_normal((R, N)).astype(np.float32)
        else:
            x = orc.bf16_from_f32(rng.standard_normal((R, N)).astype(np.float32) * 0.02)
        ar = orc.ring_allreduce(x, dtype)
        assert (ar == ar[0:1]).all()
        tr = orc.tree_allreduce(x, dtype)
        assert (tr == tr[0:1]).all()
        rs = orc.ring_reduce_scatter(x, dtype)
        ag = orc.ring_all_gather(rs, dtype)
        assert ag.tobytes() == ar.tobytes()
        for q in range(R):  # shard q is segment q of the all-reduce
            lo, hi = seg_bounds(N, R, q)
            assert rs[q].tobytes() == ar[0, lo:hi].tobytes()


def test_all_gather_is_concatenation(orc):
    rng = np.random.default_rng(3)
    for R in (2, 3, 8):
        for n in (0, 1, 5, 64):
            s = rng.standard_normal((R, n)).astype(np.float32)
            y = orc.ring_all_gather(s)
            assert y.tobytes() == np.tile(s.reshape(-1), (R, 1)).tobytes()


# ---------------------------------------------------------------- summation order

def test_ring_order_pin_r4_every_segment(orc):
    # Element of segment c: ring fold is x_{c+1} + x_{c+2} + x_{c+3} + x_c.
    # With x_c = -T, x_{c+1} = T, x_{c+2} = x_{c+3} = 1 (T = 2^24):
    #   T + 1 -> T (tie to even), T + 1 -> T, T + (-T) = 0.
    # Exact sum is 2; a fold started at the owner gives 2; the reverse
    # direction gives 2 as well.
    R, N = 4, 8
    x = np.zeros((R, N), np.float32)
    for c in range(R):
        lo, hi = seg_bounds(N, R, c)
        for e in range(lo, hi):
            x[c, e] = -T24
            x[(c + 1) % R, e] = T24
            x[(c + 2) % R, e] = 1
            x[(c + 3) % R, e] = 1
    y = orc.ring_allreduce(x)
    assert (y == 0.0).all()
    assert (orc.exact_sum(x) == 2.0).all()


def test_ring_and_tree_order_pin_r8(orc):
    # Element 0 (ring segment 0, tree A's half).  x1 = T, x3 = 1, x5 = 1,
    # x7 = -T, others 0.
    # Ring: x1 + x2 + ... + x7 + x0 = T, T, T+1 -> T, T, T+1 -> T, T, 0, 0.
    # Tree A (0->4, 4->{2,6}, 2->{1,3}, 6->{5,7}):
    #   P(2) = x2 + x1 + x3 = 0 + T + 1 -> T
    #   P(6) = x6 + x5 + x7 = 0 + 1 - T = 1 - T (exact)
    #   P(4) = x4 + P(2) + P(6) = T + (1 - T) = 1;  P(0) = x0 + P(4) = 1.
    R, N = 8, 16
    x = np.zeros((R, N), np.float32)
    x[1, 0], x[3, 0], x[5, 0], x[7, 0] = T24, 1, 1, -T24
    assert orc.ring_allreduce(x)[:, 0].tolist() == [0.0] * R
    assert orc.tree_allreduce(x)[:, 0].tolist() == [1.0] * R
    assert orc.exact_sum(x)[0] == 2.0


def test_tree_children_ascending_own_first_pin(orc):
    # Tree A at R = 8: node 2 has leaf children 1 and 3.  x2 = T, x1 = 1,
    # x3 = -T, all else 0 (element 0 is in tree A's half).
    #   own first, children ascending: (T + 1) -> T, T + (-T) = 0   -> 0
    #   children descending: (T - T) + 1 = 1;  own last: (1 - T) + T = 1.
    R, N = 8, 4
    x = np.zeros((R, N), np.float32)
    x[2, 0], x[1, 0], x[3, 0] = T24, 1, -T24
    assert orc.tree_allreduce(x)[:, 0].tolist() == [0.0] * R
    # Same pattern in tree B's half (element N-1): B is A mirrored, so node
    # 5 has children 4 and 6: x5 = T, x4 = 1, x6 = -T -> 0.
    x[:, :] = 0
    x[5, N - 1], x[4, N - 1], x[6, N - 1] = T24, 1, -T24
    assert orc.tree_allreduce(x)[:, N - 1].tolist() == [0.0] * R


def test_tree_half_split(orc):
    # Elements [0, ceil(N/2)) go through tree A, the rest through tree B.
    # Pattern that gives 0 through tree A and 1 through tree B: use the
    # tree-A pin (node 2 with children 1, 3) everywhere.  In tree B, rank 2
    # is a leaf (child of 1) and the sum folds differently.
    R = 8
    for N in (1, 2, 3, 9, 10):
        x = np.zeros((R, N), np.float32)
        x[2, :], x[1, :], x[3, :] = T24, 1, -T24
        y = orc.tree_allreduce(x)[0]
        H = (N + 1) // 2
        # Tree B: 7->{3}, 3->{1,5}, 1->{0,2}, 5->{4,6}
        #   P(1) = x1 + x0 + x2 = 1 + 0 + T -> T (tie)
        #   P(5) = 0;  P(3) = x3 + P(1) + P(5) = -T + T + 0 = 0;  P(7) = 0
        assert y[:H].tolist() == [0.0] * H
        assert y[H:].tolist() == [0.0] * (N - H)
        # and a pattern that separates the two trees: x1 = T, x0 = 1, x2 = -T
        x[:, :] = 0
        x[1, :], x[0, :], x[2, :] = T24, 1, -T24
        y = orc.tree_allreduce(x)[0]
        # Tree A: P(2) = x2 + x1 + x3 = -T + T + 0 = 0; P(4) = 0; P(0) = x0 + P(4) = 1.
        # Tree B: P(1) = x1 + x0 + x2 = (T + 1) -> T, T - T = 0; P(3) = 0 ... = 0.
        assert y[:H].tolist() == [1.0] * H
        assert y[H:].tolist() == [0.0] * (N - H)


# ---------------------------------------------------------------- brute force

def _tree_children_from_parents(par):
    kids = {r: [] for r in range(len(par))}
    for r, p in enumerate(par):
        if p >= 0:
            kids[p].append(r)
    return {k: sorted(v) for k, v in kids.items()}


def _closed_form_ring(x):
    """Closed form, not a step replay: y[e] in segment c is the float32 left
    fold x_{c+1} + x_{c+2} + ... + x_c along the ring."""
    R, N = x.shape
    y = np.empty(N, np.float32)
    for c in range(R):
        lo, hi = seg_bounds(N, R, c)
        for e in range(lo, hi):
            acc = np.float32(x[(c + 1) % R, e])
            for k in range(2, R + 1):
                acc = np.float32(acc + x[(c + k) % R, e])
            y[e] = acc
    return y


def _closed_form_tree(x, orc):
    R, N = x.shape
    H = (N + 1) // 2
    y = np.empty(N, np.float32)
    for t in (0, 1):
        par = orc.tree_parents(R, t)
        kids = _tree_children_from_parents(par)
        root = par.index(-1)

        def fold(v, e):
            acc = np.float32(x[v, e])
            for ch in kids[v]:
                acc = np.float32(acc + fold(ch, e))
            return acc
        for e in (range(0, H) if t == 0 else range(H, N)):
            y[e] = fold(root, e)
    return y


@pytest.mark.parametrize("R", [2, 3, 4, 5, 6])
def test_brute_force_tiny(orc, R):
    rng = np.random.default_rng(R)
    for N in range(0, 14):
        for trial in range(3):
            # small-magnitude values with widely different exponents, so that
            # the order of additions matters
            x = (rng.standard_normal((R, N)) * 10.0 ** rng.integers(-3, 4, size=(R, N))).astype(np.float32)
            ring = orc.ring_allreduce(x)
            tree = orc.tree_allreduce(x)
            assert ring.tobytes() == np.tile(_closed_form_ring(x), (R, 1)).tobytes()
            assert tree.tobytes() == np.tile(_closed_form_tree(x, orc), (R, 1)).tobytes()
            for e in range(N):
                exact = sum(Fraction(float(v)) for v in x[:, e])
                bound = Fraction(1, 10 ** 6) * abs(exact) + Fraction(R, 10 ** 6) * max(
                    1, max(abs(Fraction(float(v))) for v in x[:, e]))
                for y in (ring[0, e], tree[0, e]):
                    assert abs(Fraction(float(y)) - exact) <= bound


# ---------------------------------------------------------------- tolerance at size

@pytest.mark.parametrize("R", [8, 16])
def test_fp32_within_stated_tolerance(orc, R):
    rng = np.random.default_rng(R)
    x = rng.standard_normal((R, 50_000)).astype(np.float32)
    ex = orc.exact_sum(x)
    # the float64 sum is the plain definition; check it with numpy too
    assert np.array_equal(ex, x.astype(np.float64).sum(axis=0)) or np.allclose(
        ex, x.astype(np.float64).sum(axis=0), rtol=1e-15, atol=1e-12)
    for y in (orc.ring_allreduce(x)[0], orc.tree_allreduce(x)[0]):
        err = np.abs(y.astype(np.float64) - ex)
        assert (err <= 1e-6 * np.abs(ex) + 1e-6 * R).all()


def test_bf16_within_stated_tolerance(orc):
    R = 16
    rng = np.random.default_rng(5)
    x = orc.bf16_from_f32(rng.standard_normal((R, 50_000)).astype(np.float32) * 0.02)
    ex = orc.exact_sum(x, "bf16")
    y = orc.f32_from_bf16(orc.ring_allreduce(x, "bf16")[0]).astype(np.float64)
    assert (np.abs(y - ex) <= 1e-2 * np.abs(ex) + 1e-6 * R).all()


# ---------------------------------------------------------------- tree construction

@pytest.mark.parametrize("R", list(range(2, 65)))
def test_tree_invariants(orc, R):
    for t in (0, 1):
        par = orc.tree_parents(R, t)
        assert par.count(-1) == 1
        root = par.index(-1)
        kids = _tree_children_from_parents(par)
        assert sum(len(v) for v in kids.values()) == R - 1
        assert all(len(v) <= 2 for v in kids.values())
        seen, stack = set(), [root]      # spans every rank
        while stack:
            v = stack.pop()
            seen.add(v)
            stack.extend(kids[v])
        assert seen == set(range(R))
        depth = {root: 0}
        order = [root]
        for v in order:
            for ch in kids[v]:
                depth[ch] = depth[v] + 1
                order.append(ch)
        assert max(depth.values()) <= int(np.ceil(np.log2(R))) + 1
    # tree A is an in-order binary tree: left subtree < node < right subtree
    parA = orc.tree_parents(R, 0)
    kidsA = _tree_children_from_parents(parA)

    def inorder(v):
        small = [c for c in kidsA[v] if c < v]
        large = [c for c in kidsA[v] if c > v]
        assert len(small) <= 1 and len(large) <= 1
        out = []
        for c in small:
            out += inorder(c)
        out.append(v)
        for c in large:
            out += inorder(c)
        return out
    assert inorder(0) == list(range(R))
    # complementary: for even R no rank is interior in both trees
    if R % 2 == 0:
        kidsB = _tree_children_from_parents(orc.tree_parents(R, 1))
        assert not any(kidsA[r] and kidsB[r] for r in range(R))


# ---------------------------------------------------------------- bf16 and LL

def test_bf16_rounding_table(orc):
    cases = {
        0x3F808000: 0x3F80,  # tie, even neighbour below
        0x3F818000: 0x3F82,  # tie, odd below -> up
        0x3F808001: 0x3F81,  # above half
        0x3F807FFF: 0x3F80,  # below half
        0x00000000: 0x0000,
        0x80000000: 0x8000,
        0x7F800000: 0x7F80,  # +inf
        0xFF800000: 0xFF80,  # -inf
        0x7F7FFFFF: 0x7F80,  # largest float32 rounds to +inf in bf16
        0x7F7F0000: 0x7F7F,  # largest bf16 stays
        0x00000001: 0x0000,  # smallest denormal rounds to +0
        0x00008000: 0x0000,  # tie at zero -> even (0)
        0x00018000: 0x0002,  # denormal tie, odd -> up
    }
    for u, want in cases.items():
        f = np.array([u], np.uint32).view(np.float32)[0]
        assert orc.lib().orc_bf16_from_f32(float(f)) == want, hex(u)


def test_bf16_matches_torch(orc):
    import torch
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    f = np.concatenate([f, (rng.standard_normal(100_000) * 0.02).astype(np.float32)])
    mine = orc.bf16_from_f32(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    nan = orc.bf16_from_f32(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# ---------------------------------------------------------------- max / min / avg

@pytest.mark.parametrize("R", [2, 3, 5, 8, 16])
def test_max_min_equal_elementwise_extremes(orc, R):
    rng = np.random.default_rng(40 + R)
    N = R * 23 + 5
    xi = rng.integers(-(2 ** 31), 2 ** 31, size=(R, N), dtype=np.int64).astype(np.int32)
    xf = rng.standard_normal((R, N)).astype(np.float32)
    for x in (xi, xf):
        for op, ref in (("max", x.max(axis=0)), ("min", x.min(axis=0))):
            assert (orc.ring_allreduce(x, op=op) == ref[None, :]).all()
            assert (orc.tree_allreduce(x, op=op) == ref[None, :]).all()
    xb = orc.bf16_from_f32(xf)
    yb = orc.ring_allreduce(xb, "bf16", op="max")[0]
    assert (orc.f32_from_bf16(yb) == orc.f32_from_bf16(xb).max(axis=0)).all()
    NR = (N // R) * R
    assert (orc.ring_reduce_scatter(xi[:, :NR], op="min").reshape(-1) == xi[:, :NR].min(axis=0)).all()


def test_max_signed_zero_follows_the_fold_order(orc):
    # max keeps the running value only when it is strictly larger, so for
    # {+0, -0} the value folded last wins.  R = 2, N = 2: element 0 is in
    # segment 0 (fold x1 then x0), element 1 in segment 1 (fold x0 then x1).
    x = np.array([[0.0, 0.0], [-0.0, -0.0]], np.float32)
    y = orc.ring_allreduce(x, op="max")[0]
    assert np.signbit(y[0]) == False and np.signbit(y[1]) == True  # noqa: E712
    y = orc.ring_allreduce(x, op="min")[0]
    assert np.signbit(y[0]) == False and np.signbit(y[1]) == True  # noqa: E712


@pytest.mark.parametrize("R", [2, 3, 8, 16])
def test_avg_is_the_sum_divided_once(orc, R):
    rng = np.random.default_rng(60 + R)
    N = 1000
    x = rng.standard_normal((R, N)).astype(np.float32)
    want = orc.ring_allreduce(x) / np.float32(R)          # numpy float32 division
    assert orc.ring_allreduce(x, op="avg").tobytes() == want.astype(np.float32).tobytes()
    want_t = orc.tree_allreduce(x) / np.float32(R)
    assert orc.tree_allreduce(x, op="avg").tobytes() == want_t.astype(np.float32).tobytes()
    ex = orc.exact_sum(x) / R
    y = orc.ring_allreduce(x, op="avg")[0].astype(np.float64)
    assert (np.abs(y - ex) <= 1e-6 * np.abs(ex) + 1e-6).all()
    # integer multiples of R: the average is exact
    k = rng.integers(-1000, 1001, size=(R, N))
    xi = (k * R).astype(np.float32)
    assert (orc.ring_allreduce(xi, op="avg")[0] == k.sum(axis=0).astype(np.float32)).all()


def test_bf16_avg_rounds_once_after_dividing(orc):
    import torch
    R, N = 16, 3000
    rng = np.random.default_rng(9)
    xb = orc.bf16_from_f32(rng.standard_normal((R, N)).astype(np.float32) * 0.02)
    # the same fold in float32 on the widened inputs, divided, rounded once
    s32 = orc.ring_allreduce(orc.f32_from_bf16(xb))[0]
    want = torch.from_numpy(s32 / np.float32(R)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (orc.ring_allreduce(xb, "bf16", op="avg")[0] == want).all()
    assert (orc.ring_reduce_scatter(xb[:, :N - N % R], "bf16", op="avg").reshape(-1) ==
            orc.ring_allreduce(xb[:, :N - N % R], "bf16", op="avg")[0]).all()


def test_int32_avg_is_refused(orc):
    x = np.ones((4, 8), np.int32)
    with pytest.raises(RuntimeError):
        orc.ring_allreduce(x, op="avg")


# ---------------------------------------------------------------- multi-channel rings

def _channel_bounds(N, R, K, c, k):
    S = -(-N // R)
    Sk = -(-(-(-S // K)) // 8) * 8
    a, b = min(c * S, N), min((c + 1) * S, N)
    return min(a + k * Sk, b), min(a + (k + 1) * Sk, b)


def test_reverse_stride_folds_the_other_way(orc):
    # Stride 3 at R = 4 is the ring q -> q-1: segment c folds x_{c+3},
    # x_{c+2}, x_{c+1}, x_c.  With x_c = -T, x_{c+1} = T, x_{c+2} = x_{c+3} = 1:
    #   1 + 1 = 2, 2 + T = T + 2 (exact: even), T + 2 - T = 2.
    # Stride 1 (x_{c+1} first) gives 0, see test_ring_order_pin_r4_every_segment.
    R, N = 4, 8
    x = np.zeros((R, N), np.float32)
    for c in range(R):
        lo, hi = seg_bounds(N, R, c)
        for e in range(lo, hi):
            x[c, e], x[(c + 1) % R, e] = -T24, T24
            x[(c + 2) % R, e] = x[(c + 3) % R, e] = 1
    assert (orc.ring_allreduce(x, strides=[3]) == 2.0).all()
    assert (orc.ring_allreduce(x, strides=[1]) == 0.0).all()


def test_channel_split_of_each_segment(orc):
    # R = 4, N = 64: S = 16, two channels of Sk = 8 -> channel 0 takes the
    # first 8 elements of every segment (stride 1 -> 0.0), channel 1 the last
    # 8 (stride 3 -> 2.0), with the pattern above in every element.
    R, N = 4, 64
    x = np.zeros((R, N), np.float32)
    for c in range(R):
        x[c, c * 16:(c + 1) * 16] = -T24
        x[(c + 1) % R, c * 16:(c + 1) * 16] = T24
        x[(c + 2) % R, c * 16:(c + 1) * 16] = 1
        x[(c + 3) % R, c * 16:(c + 1) * 16] = 1
    y = orc.ring_allreduce(x, strides=[1, 3])[0].reshape(R, 16)
    assert (y[:, :8] == 0.0).all() and (y[:, 8:] == 2.0).all()


def _closed_form_channels(x, strides):
    R, N = x.shape
    K = len(strides)
    y = np.empty(N, np.float32)
    for c in range(R):
        for k, m in enumerate(strides):
            lo, hi = _channel_bounds(N, R, K, c, k)
            for e in range(lo, hi):
                acc = np.float32(x[(c + m) % R, e])
                for j in range(2, R + 1):
                    acc = np.float32(acc + x[(c + j * m) % R, e])
                y[e] = acc
    return y


@pytest.mark.parametrize("R,strides", [(4, [1, 3]), (5, [1, 4, 2, 3]), (8, [1, 7, 3, 5]),
                                       (8, [3]), (7, [1, 6, 2])])
def test_channels_brute_force_and_identities(orc, R, strides):
    rng = np.random.default_rng(R + len(strides))
    for N in (1, 5, 37, 200, 1000):
        x = (rng.standard_normal((R, N)) * 10.0 ** rng.integers(-3, 4, size=(R, N))).astype(np.float32)
        y = orc.ring_allreduce(x, strides=strides)
        assert y.tobytes() == np.tile(_closed_form_channels(x, strides), (R, 1)).tobytes()
        xi = rng.integers(-1000, 1001, size=(R, N)).astype(np.int32)
        assert (orc.ring_allreduce(xi, strides=strides) == xi.sum(axis=0)[None, :]).all()
    N = R * 53
    x = rng.standard_normal((R, N)).astype(np.float32)
    ar = orc.ring_allreduce(x, strides=strides)
    rs = orc.ring_reduce_scatter(x, strides=strides)
    assert orc.ring_all_gather(rs, strides=strides).tobytes() == ar.tobytes()
    assert orc.ring_all_gather(rs).tobytes() == ar.tobytes()  # all-gather is a copy


def test_channel_strides_must_visit_every_rank(orc):
    x = np.ones((4, 8), np.float32)
    with pytest.raises(RuntimeError):
        orc.ring_allreduce(x, strides=[2])     # gcd(2, 4) = 2
    with pytest.raises(RuntimeError):
        orc.ring_allreduce(x, strides=[4])


# ---------------------------------------------------------------- all-cores build

@pytest.mark.parametrize("R,N", [(2, 1), (3, 1000), (8, 4097), (16, 16 * 333)])
def test_openmp_build_gives_the_same_bits(orc, R, N):
    """The OpenMP build parallelises only over elements (or ranks) within a
    step, so every element keeps its fold order: the same bits as one
    thread, for every collective and operator."""
    rng = np.random.default_rng(R * 1000 + N)
    x = rng.standard_normal((R, N)).astype(np.float32)
    xi = rng.integers(-1000, 1000, size=(R, N), endpoint=True).astype(np.int32)
    xb = orc.bf16_from_f32(x * 0.02)
    n = N - N % R
    want = [orc.ring_allreduce(x), orc.ring_allreduce(xi), orc.ring_allreduce(xb, "bf16"),
            orc.ring_allreduce(x, op="max"), orc.ring_allreduce(x, op="avg"),
            orc.tree_allreduce(x), orc.tree_allreduce(xb, "bf16"), orc.exact_sum(x),
            orc.ring_reduce_scatter(x[:, :n]), orc.ring_all_gather(xb, "bf16"),
            orc.ring_allreduce(x, strides=[1, R - 1] if R > 2 else [1])]
    with orc.parallel(4) as threads:
        assert threads == 4
        got = [orc.ring_allreduce(x), orc.ring_allreduce(xi), orc.ring_allreduce(xb, "bf16"),
               orc.ring_allreduce(x, op="max"), orc.ring_allreduce(x, op="avg"),
               orc.tree_allreduce(x), orc.tree_allreduce(xb, "bf16"), orc.exact_sum(x),
               orc.ring_reduce_scatter(x[:, :n]), orc.ring_all_gather(xb, "bf16"),
               orc.ring_allreduce(x, strides=[1, R - 1] if R > 2 else [1])]
    for w, g in zip(want, got):
        assert w.tobytes() == g.tobytes()
