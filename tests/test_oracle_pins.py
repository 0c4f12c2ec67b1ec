"""Pins for the CPU oracle: checks against things other than the oracle itself.

Kinds of pin used here (the pages print no worked numeric example):
  * hand-derived closed forms stored under tests/golden/;
  * a library routine that reduces to the same definition:
    torch.nn.functional.scaled_dot_product_attention and torch.logsumexp in
    fp64 on the CPU;
  * invariants of the definition: constant keys give the mean of V, a single
    key gives that key's value, V = 1 gives 1, a dominant key selects its
    value, joint permutation of keys and values changes nothing, masked keys
    contribute nothing, and the Split operator's result does not depend on s.
Together these fail on a dropped scale, a wrong sign, a wrong GQA index, a
transposed operand, an off-by-one causal bound, a wrong log base or a wrong
merge weight (tests/test_oracle_mutations.py plants each of these).
"""
import json
import math
import os

import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa_reference(q, k, v, qo_indptr, kv_indptr, scale, mask_kind, mask=None):
    """Per-request fp64 torch SDPA (+ torch.logsumexp for the LSE) on CPU."""
    q, k, v = q.double(), k.double(), v.double()
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    outs, lses = [], []
    for b in range(len(qo_indptr) - 1):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
        nq, nk = q1 - q0, k1 - k0
        qb = q[q0:q1].transpose(0, 1)  # [Hq, nq, D]
        kb = k[k0:k1].transpose(0, 1).repeat_interleave(G, dim=0)
        vb = v[k0:k1].transpose(0, 1).repeat_interleave(G, dim=0)
        if mask_kind == oracle.MASK_NONE:
            allowed = torch.ones(nq, nk, dtype=torch.bool)
        elif mask_kind == oracle.MASK_CAUSAL:
            allowed = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
        else:
            allowed = mask[:nq, :nk].bool()
        o = torch.nn.functional.scaled_dot_product_attention(
            qb, kb, vb, attn_mask=allowed, scale=scale)
        scores = torch.matmul(qb, kb.transpose(1, 2).contiguous()) * scale
        scores = scores.masked_fill(~allowed, float("-inf"))
        lse = torch.logsumexp(scores, dim=-1)
        outs.append(o.transpose(0, 1))
        lses.append(lse.transpose(0, 1))
    return torch.cat(outs), torch.cat(lses)


def rand(shape, seed, dtype=torch.float64):
    return synth.randn(shape, dtype, synth.gen(seed))


# ---- hand-derived closed forms -------------------------------------------

def test_golden_two_keys():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_two_keys.json")))
    q = torch.tensor(g["q"], dtype=torch.float64).view(1, 1, -1)
    k = torch.tensor(g["k"], dtype=torch.float64).view(2, 1, -1)
    v = torch.tensor(g["v"], dtype=torch.float64).view(2, 1, -1)
    o, lse = oracle.attention(q, k, v, [0, 1], [0, 2], g["scale"])
    assert torch.allclose(o.view(-1), torch.tensor(g["o"], dtype=torch.float64), atol=1e-14)
    assert abs(float(lse) - g["lse"]) < 1e-14
    assert abs(g["lse"] - math.log(4.0)) < 1e-15


def test_golden_causal_row0():
    g = json.load(open(os.path.join(GOLDEN, "closed_form_causal_row0.json")))
    L, D = 5, 2
    q = rand((L, 1, D), 11)
    k = rand((L, 1, D), 12)
    v = rand((L, 1, D), 13)
    q[0, 0] = torch.tensor(g["q0"], dtype=torch.float64)
    k[0, 0] = torch.tensor(g["k0"], dtype=torch.float64)
    v[0, 0] = torch.tensor(g["v0"], dtype=torch.float64)
    o, lse = oracle.attention(q, k, v, [0, L], [0, L], g["scale"], oracle.MASK_CAUSAL)
    assert torch.equal(o[0, 0], v[0, 0])
    assert float(lse[0, 0]) == g["lse0"]


# ---- library routine: fp64 torch SDPA --------------------------------------

@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (4, 2), (6, 3)])
@pytest.mark.parametrize("mask_kind", [oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_DENSE])
def test_matches_sdpa(Hq, Hkv, mask_kind):
    lens_q, lens_k, D = [3, 7, 1], [5, 7, 9], 16
    if mask_kind == oracle.MASK_DENSE:
        lens_q, lens_k = [6, 6], [6, 6]
    qo, kv = synth.indptr(lens_q), synth.indptr(lens_k)
    q = rand((sum(lens_q), Hq, D), 1)
    k = rand((sum(lens_k), Hkv, D), 2)
    v = rand((sum(lens_k), Hkv, D), 3)
    mask = None
    if mask_kind == oracle.MASK_DENSE:
        mask = (torch.rand((6, 6), generator=synth.gen(4)) < 0.5).to(torch.uint8)
        mask[torch.arange(6), torch.arange(6)] = 1  # every row keeps a key
    scale = 0.3
    o, lse = oracle.attention(q, k, v, qo, kv, scale, mask_kind, mask)
    o_ref, lse_ref = sdpa_reference(q, k, v, qo, kv, scale, mask_kind, mask)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0)


@settings(max_examples=40, deadline=None)
@given(B=st.integers(1, 3), G=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 2),
       D=st.sampled_from([1, 4, 8]), causal=st.booleans(), seed=st.integers(0, 10_000),
       data=st.data())
def test_random_tiny_shapes_match_sdpa(B, G, Hkv, D, causal, seed, data):
    lens_k = [data.draw(st.integers(1, 12)) for _ in range(B)]
    lens_q = [data.draw(st.integers(1, n)) for n in lens_k]
    Hq = G * Hkv
    qo, kv = synth.indptr(lens_q), synth.indptr(lens_k)
    q = rand((sum(lens_q), Hq, D), seed)
    k = rand((sum(lens_k), Hkv, D), seed + 1)
    v = rand((sum(lens_k), Hkv, D), seed + 2)
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    o, lse = oracle.attention(q, k, v, qo, kv, 0.7, mk)
    o_ref, lse_ref = sdpa_reference(q, k, v, qo, kv, 0.7, mk)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0)


# ---- invariants and closed forms of the definition -------------------------

@pytest.mark.parametrize("mask_kind", [oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_DENSE])
def test_constant_keys_give_mean_of_v(mask_kind):
    L, Hq, Hkv, D, scale = 9, 4, 2, 8, 0.25
    q = rand((L, Hq, D), 5)
    kc = rand((1, Hkv, D), 6)
    k = kc.expand(L, Hkv, D).contiguous()
    v = rand((L, Hkv, D), 7)
    mask = None
    if mask_kind == oracle.MASK_DENSE:
        mask = synth.window_mask(L, 3)
        allowed = mask.bool()
    elif mask_kind == oracle.MASK_CAUSAL:
        allowed = torch.ones(L, L, dtype=torch.bool).tril()
    else:
        allowed = torch.ones(L, L, dtype=torch.bool)
    o, lse = oracle.attention(q, k, v, [0, L], [0, L], scale, mask_kind, mask)
    for i in range(L):
        J = allowed[i].nonzero().view(-1)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            mean_v = v[J, g].mean(0)
            assert torch.allclose(o[i, h], mean_v, atol=1e-13)
            expect = scale * float((q[i, h] * kc[0, g]).sum()) + math.log(len(J))
            assert abs(float(lse[i, h]) - expect) < 1e-12


def test_single_key_returns_its_value():
    Hq, D = 3, 5
    q = rand((1, Hq, D), 8)
    k = rand((1, 1, D), 9)
    v = rand((1, 1, D), 10)
    o, lse = oracle.attention(q, k, v, [0, 1], [0, 1], 0.4)
    for h in range(Hq):
        assert torch.equal(o[0, h], v[0, 0])
        assert abs(float(lse[0, h]) - 0.4 * float((q[0, h] * k[0, 0]).sum())) < 1e-14


def test_unit_values_give_unit_output():
    L, Hq, D = 11, 2, 6
    q, k = rand((L, Hq, D), 14), rand((L, 1, D), 15)
    v = torch.ones((L, 1, D), dtype=torch.float64)
    o, _ = oracle.attention(q, k, v, [0, L], [0, L], 0.5, oracle.MASK_CAUSAL)
    assert torch.allclose(o, torch.ones_like(o), atol=1e-14)


def test_dominant_key_selects_its_value():
    L, D = 16, 8
    q = rand((1, 1, D), 16)
    k = rand((L, 1, D), 17)
    v = rand((L, 1, D), 18)
    k[5, 0] = 50.0 * q[0, 0]  # score far above the rest
    o, lse = oracle.attention(q, k, v, [0, 1], [0, L], 1.0)
    assert torch.allclose(o[0, 0], v[5, 0], atol=1e-12)
    smax = float((q[0, 0] * k[5, 0]).sum())
    assert abs(float(lse[0, 0]) - smax) < 1e-9  # the other terms are below e^-300


def test_joint_permutation_of_keys_and_values():
    L, Hq, D = 20, 4, 8
    q, k, v = rand((1, Hq, D), 19), rand((L, 2, D), 20), rand((L, 2, D), 21)
    perm = torch.randperm(L, generator=synth.gen(22))
    o1, l1 = oracle.attention(q, k, v, [0, 1], [0, L], 0.3)
    o2, l2 = oracle.attention(q, k[perm], v[perm], [0, 1], [0, L], 0.3)
    assert torch.allclose(o1, o2, atol=1e-13)
    assert torch.allclose(l1, l2, atol=1e-13)


def test_masked_keys_contribute_nothing():
    """Poisoning every masked-out K/V entry with NaN or 1e30 changes nothing."""
    L, D = 64, 8
    g = synth.gen(23)
    mask = synth.sparse_mask(L, g, window=8, block=16, globals_per_block=1, random_blocks=1)
    mask[:, 16:32] = 0  # a whole key block that no query may see
    mask[torch.arange(L), torch.arange(L)] = 1
    mask[:, 16:32] = 0
    q, k, v = rand((L, 2, D), 24), rand((L, 2, D), 25), rand((L, 2, D), 26)
    o1, l1 = oracle.attention(q, k, v, [0, L], [0, L], 0.35, oracle.MASK_DENSE, mask)
    unseen = mask.sum(0) == 0
    assert bool(unseen[16:32].all())
    for poison in (float("nan"), 1e30):
        k2, v2 = k.clone(), v.clone()
        k2[unseen] = poison
        v2[unseen] = poison
        o2, l2 = oracle.attention(q, k2, v2, [0, L], [0, L], 0.35, oracle.MASK_DENSE, mask)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # causal, bottom-right aligned: the last key is visible to the last query only
    Lq, Lk = 4, 10
    qq = rand((Lq, 1, D), 27)
    kk, vv = rand((Lk, 1, D), 28), rand((Lk, 1, D), 29)
    o3, l3 = oracle.attention(qq, kk, vv, [0, Lq], [0, Lk], 0.5, oracle.MASK_CAUSAL)
    kk[Lk - 1], vv[Lk - 1] = float("nan"), float("nan")
    o4, l4 = oracle.attention(qq, kk, vv, [0, Lq], [0, Lk], 0.5, oracle.MASK_CAUSAL)
    assert torch.equal(o3[:Lq - 1], o4[:Lq - 1]) and torch.equal(l3[:Lq - 1], l4[:Lq - 1])
    assert bool(torch.isnan(o4[Lq - 1]).all())


def test_row_without_valid_key():
    L, D = 4, 3
    q, k, v = rand((L, 1, D), 30), rand((L, 1, D), 31), rand((L, 1, D), 32)
    mask = torch.ones(L, L, dtype=torch.uint8)
    mask[2] = 0
    o, lse = oracle.attention(q, k, v, [0, L], [0, L], 1.0, oracle.MASK_DENSE, mask)
    assert torch.equal(o[2, 0], torch.zeros(D, dtype=torch.float64))
    assert lse[2, 0] == float("-inf")
    # and a causal request with fewer keys than queries
    o2, lse2 = oracle.attention(rand((3, 1, D), 33), k[:1], v[:1], [0, 3], [0, 1], 1.0,
                                oracle.MASK_CAUSAL)
    assert lse2[0, 0] == float("-inf") and lse2[1, 0] == float("-inf")
    assert torch.equal(o2[2, 0], v[0, 0])


def test_row_subset_matches_full():
    lens = [5, 8]
    q, k, v = rand((13, 4, 8), 34), rand((13, 2, 8), 35), rand((13, 2, 8), 36)
    qo = kv = synth.indptr(lens)
    o, lse = oracle.attention(q, k, v, qo, kv, 0.5, oracle.MASK_CAUSAL)
    rows = torch.tensor([[0, 0], [12, 3], [7, 1], [5, 2]])
    os_, ls_ = oracle.attention(q, k, v, qo, kv, 0.5, oracle.MASK_CAUSAL, rows=rows)
    for n, (t, h) in enumerate(rows.tolist()):
        assert torch.equal(os_[n], o[t, h]) and ls_[n] == lse[t, h]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_storage_dtypes_widen_exactly(dtype):
    """The oracle's element widening equals torch's own exact upcast."""
    L, D = 12, 16
    q, k, v = (synth.randn((L, 2, D), dtype, synth.gen(s)) for s in (37, 38, 39))
    k[0, 0, 0] = torch.tensor(6e-8 if dtype == torch.float16 else 1e-38, dtype=dtype)  # subnormal
    o1, l1 = oracle.attention(q, k, v, [0, L], [0, L], 0.25, oracle.MASK_CAUSAL)
    o2, l2 = oracle.attention(q.double(), k.double(), v.double(), [0, L], [0, L], 0.25,
                              oracle.MASK_CAUSAL)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- the Split operator ----------------------------------------------------

@pytest.mark.parametrize("lengths", [[256], [7, 64, 1, 33], [1000, 3]])
@pytest.mark.parametrize("s", [1, 2, 3, 4, 7, 16])
def test_split_ranges_partition_each_request(lengths, s):
    kv = synth.indptr(lengths)
    maxlen = max(lengths)
    c = oracle.chunk_len(maxlen, s)
    assert c == -(-maxlen // s)
    r = oracle.split_ranges(kv, maxlen, s)
    for b, n in enumerate(lengths):
        used = [tuple(x) for x in r[b].tolist() if x[0] >= 0]
        assert len(used) == -(-n // c)
        covered = []
        for lo, hi in used:
            assert 0 < hi - lo <= c and lo % c == 0
            covered.extend(range(lo, hi))
        assert covered == list(range(n))  # disjoint, ordered, complete
        assert all(x == [-1, -1] for x in r[b].tolist()[len(used):])


def flat_ranges_brute(lengths, total, P, s):
    """The flat plan by enumeration: walk every packed key row, tag it with
    (request, piece) and cut a request's rows wherever the tag changes."""
    c = -(-total // P) if total else 0
    owner = {}
    pos = 0
    for b, n in enumerate(lengths):
        for j in range(n):
            owner[pos + j] = (b, j)
        pos += n
    out = [[[-1, -1] for _ in range(s)] for _ in lengths]
    last = {}
    for t in range(total):
        if t not in owner:
            continue
        b, j = owner[t]
        key = (b, t // c)
        if b not in last or last[b][0] != key:
            i = 0 if b not in last else last[b][1] + 1
            out[b][i] = [j, j + 1]
            last[b] = (key, i)
        else:
            out[b][last[b][1]][1] = j + 1
    return torch.tensor(out, dtype=torch.int64).reshape(len(lengths), s, 2)


@pytest.mark.parametrize("lengths", [[256], [7, 64, 1, 33], [1000, 3], [0, 5, 0, 9, 0],
                                     [13] * 9])
@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 64])
def test_flat_ranges_match_enumeration(lengths, P):
    total = sum(lengths)
    n = max(lengths)
    s = oracle.flat_max_splits(total, n, P)
    c = oracle.flat_piece_len(total, P)
    assert c == (-(-total // P) if total else 0)
    r = oracle.flat_ranges(synth.indptr(lengths), total, P, s)
    assert torch.equal(r, flat_ranges_brute(lengths, total, P, s))
    # every request is partitioned in order; no request needs more slots than
    # the bound, and the bound is reached by some placement of a request of
    # length n (checked on the worst offset below)
    for b, nb in enumerate(lengths):
        used = [tuple(x) for x in r[b].tolist() if x[0] >= 0]
        cov = []
        for lo, hi in used:
            assert 0 < hi - lo <= c
            cov.extend(range(lo, hi))
        assert cov == list(range(nb))


def test_flat_max_splits_is_tight():
    # pieces of 4 rows; request 1 holds rows [3, 12): one row before the
    # first boundary, so its 9 keys touch pieces 0, 1 and 2
    lengths = [3, 9, 4]
    assert oracle.flat_piece_len(16, 4) == 4
    assert oracle.flat_max_splits(16, 9, 4) == 3
    r = oracle.flat_ranges(synth.indptr(lengths), 16, 4, 3)
    assert r[1].tolist() == [[0, 1], [1, 5], [5, 9]]
    assert r[0].tolist() == [[0, 3], [-1, -1], [-1, -1]]
    assert r[2].tolist() == [[0, 4], [-1, -1], [-1, -1]]
    assert oracle.flat_max_splits(16, 9, 2) == 2  # never more than P


def test_flat_ranges_reject_too_few_slots():
    with pytest.raises(ValueError):
        oracle.flat_ranges(synth.indptr([10, 10]), 20, 4, 1)


@pytest.mark.parametrize("P", [1, 3, 7, 50])
def test_split_decode_flat_plan_equals_attention(P):
    lengths = [256, 37, 0, 1, 129]
    B, Hq, Hkv, D = len(lengths), 8, 2, 16
    q, k, v, kv = synth.decode_inputs(B, Hq, Hkv, D, lengths, torch.bfloat16, seed=41)
    o_ref, lse_ref = oracle.attention(q, k, v, list(range(B + 1)), kv, 0.25)
    rg = oracle.flat_ranges(kv, sum(lengths), P)
    o, lse, op, mp, lp = oracle.split_decode(q, k, v, kv, max(lengths), 0.25, 0, ranges=rg)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.equal(lse[2], torch.full((Hq,), -math.inf, dtype=torch.float64))
    ok = torch.isfinite(lse_ref)
    assert torch.allclose(lse[ok], lse_ref[ok], atol=1e-12, rtol=0)


@pytest.mark.parametrize("dtype", [torch.float64, torch.bfloat16])
def test_split_decode_is_invariant_to_s(dtype):
    lengths = [256, 37, 1, 129]
    B, Hq, Hkv, D = len(lengths), 8, 2, 16
    q, k, v, kv = synth.decode_inputs(B, Hq, Hkv, D, lengths, dtype, seed=40)
    qo = list(range(B + 1))
    o_ref, lse_ref = oracle.attention(q, k, v, qo, kv, 0.25)
    for s in (1, 2, 3, 4, 8, 300):
        o, lse, op, mp, lp = oracle.split_decode(q, k, v, kv, max(lengths), 0.25, s)
        assert torch.allclose(o, o_ref, atol=1e-12, rtol=0), s
        assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0), s
        if s == 1:  # one split is the identity
            assert torch.allclose(op[0].view(B, Hq, D), o_ref, atol=1e-13)


def test_merge_properties():
    s, rows, D = 5, 7, 4
    g = synth.gen(41)
    op = torch.randn((s, rows, D), generator=g, dtype=torch.float64)
    mp = torch.randn((s, rows), generator=g, dtype=torch.float64) * 3
    lp = torch.rand((s, rows), generator=g, dtype=torch.float64) * 5 + 0.1
    o, lse = oracle.merge(op, mp, lp)
    # permutation of the partials
    perm = torch.randperm(s, generator=g)
    o2, lse2 = oracle.merge(op[perm], mp[perm], lp[perm])
    assert torch.allclose(o, o2, atol=1e-13) and torch.allclose(lse, lse2, atol=1e-13)
    # associativity: merging two pre-merged groups
    oa, la = oracle.merge(op[:2], mp[:2], lp[:2])
    ob, lb = oracle.merge(op[2:], mp[2:], lp[2:])
    o3, lse3 = oracle.merge(torch.stack([oa, ob]), torch.stack([la, lb]),
                            torch.ones((2, rows), dtype=torch.float64))
    assert torch.allclose(o, o3, atol=1e-12) and torch.allclose(lse, lse3, atol=1e-12)
    # an empty partial (m = -inf, l = 0) is ignored
    op4 = torch.cat([op, torch.full((1, rows, D), float("nan"), dtype=torch.float64)])
    mp4 = torch.cat([mp, torch.full((1, rows), float("-inf"), dtype=torch.float64)])
    lp4 = torch.cat([lp, torch.zeros((1, rows), dtype=torch.float64)])
    o4, lse4 = oracle.merge(op4, mp4, lp4)
    assert torch.equal(o4, o) and torch.equal(lse4, lse)
    # all partials empty: O = 0, LSE = -inf
    o5, lse5 = oracle.merge(op4[-1:], mp4[-1:], lp4[-1:])
    assert torch.equal(o5, torch.zeros_like(o5)) and bool((lse5 == float("-inf")).all())
    # closed form with two partials: LSE adds in probability space
    o6, lse6 = oracle.merge(op[:2], mp[:2], lp[:2])
    expect = torch.logaddexp(mp[0] + lp[0].log(), mp[1] + lp[1].log())
    assert torch.allclose(lse6, expect, atol=1e-13)


# ---- values narrower than keys (MLA's absorbed form) -----------------------

@pytest.mark.parametrize("causal", [False, True])
def test_value_width_differs_matches_sdpa(causal):
    """Keys/queries of D elements, values of Dv: fp64 torch SDPA takes the
    value width from V, so it pins the separate value head dim."""
    lens_q, lens_k, D, Dv = [2, 5], [6, 5], 12, 5
    qo, kv = synth.indptr(lens_q), synth.indptr(lens_k)
    q = rand((sum(lens_q), 4, D), 31)
    k = rand((sum(lens_k), 2, D), 32)
    v = rand((sum(lens_k), 2, Dv), 33)
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    o, lse = oracle.attention(q, k, v, qo, kv, 0.45, mk)
    o_ref, lse_ref = sdpa_reference(q, k, v, qo, kv, 0.45, mk)
    assert o.shape == (sum(lens_q), 4, Dv)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_mla_absorbed_decode_by_loops():
    """MLA decode in its absorbed form, written out with plain loops: every
    head scores the whole cache row (latent + rotary part), the output
    averages the latent part of the rows."""
    H, T, Dc, Dr, scale = 3, 7, 6, 2, 0.37
    q = rand((1, H, Dc + Dr), 34)
    cache = rand((T, 1, Dc + Dr), 35)
    o, lse = oracle.attention(q, cache, cache[:, :, :Dc].contiguous(), [0, 1], [0, T], scale)
    for h in range(H):
        s = [scale * sum(float(q[0, h, d]) * float(cache[t, 0, d]) for d in range(Dc + Dr))
             for t in range(T)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for d in range(Dc):
            want = sum(w[t] * float(cache[t, 0, d]) for t in range(T)) / z
            assert abs(float(o[0, h, d]) - want) < 1e-13
        assert abs(float(lse[0, h]) - (m + math.log(z))) < 1e-13


def test_constant_keys_mean_of_narrow_values():
    L, Hq, D, Dv = 7, 2, 9, 4
    q = rand((1, Hq, D), 36)
    k = rand((1, 1, D), 37).expand(L, 1, D).contiguous()
    v = rand((L, 1, Dv), 38)
    o, lse = oracle.attention(q, k, v, [0, 1], [0, L], 0.6)
    for h in range(Hq):
        assert torch.allclose(o[0, h], v[:, 0].mean(0), atol=1e-13)
        assert abs(float(lse[0, h]) - (0.6 * float((q[0, h] * k[0, 0]).sum()) + math.log(L))) < 1e-12
