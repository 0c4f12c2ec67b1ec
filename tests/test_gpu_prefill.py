"""GPU parity of dense / causal prefill against the fp64 oracle."""
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, TOL_O, check

pytestmark = pytest.mark.gpu


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


def prefill(q, k, v, qo, kv, causal, scale=None):
    lq = (qo[1:] - qo[:-1]).max().item()
    lk = (kv[1:] - kv[:-1]).max().item()
    o, lse = ra().attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), qo.to(DEV), kv.to(DEV), lq, lk,
                               scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G", [1, 4])
def test_ragged_small(dtype, D, causal, G):
    # lengths span several 128-row / 64-key tiles with ragged tails, n_q != n_kv
    lens_q = [300, 1, 129, 64]
    lens_k = [300, 77, 200, 64]
    Hkv = 2
    qo, kv = synth.indptr(lens_q), synth.indptr(lens_k)
    g = synth.gen(D + G + causal)
    q = synth.randn((sum(lens_q), G * Hkv, D), dtype, g)
    k = synth.randn((sum(lens_k), Hkv, D), dtype, g)
    v = synth.randn((sum(lens_k), Hkv, D), dtype, g)
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    o_ref, lse_ref = oracle.attention(q, k, v, qo, kv, 1 / D ** 0.5, mk)
    o, lse = prefill(q, k, v, qo, kv, causal)
    check(f"prefill {dtype} D={D} causal={causal} G={G}", o, o_ref, lse, lse_ref, dtype)


def test_rows_without_keys():
    """Causal with fewer keys than queries: the first rows see nothing."""
    qo, kv = synth.indptr([130]), synth.indptr([5])
    g = synth.gen(21)
    q = synth.randn((130, 2, 64), torch.bfloat16, g)
    k = synth.randn((5, 1, 64), torch.bfloat16, g)
    v = synth.randn((5, 1, 64), torch.bfloat16, g)
    o_ref, lse_ref = oracle.attention(q, k, v, qo, kv, 0.125, oracle.MASK_CAUSAL)
    o, lse = prefill(q, k, v, qo, kv, True)
    check("prefill empty rows", o, o_ref, lse, lse_ref, torch.bfloat16)
    assert bool((o[:125] == 0).all()) and bool(torch.isinf(lse[:125]).all())


def test_causal_prefill_workload_every_row():
    """B 2, L 4096, 32/8 heads, D 128, bf16, causal: every (token, head) row
    of O and LSE against the fp64 oracle."""
    w = synth.workload("causal_prefill_bf16")
    inp = w.make(DEV)
    print(f"causal prefill {w.B}x{w.L}: oracle over every row ...", flush=True)
    o, lse = prefill(inp["q"], inp["k"], inp["v"], inp["qo_indptr"], inp["kv_indptr"], True)
    o_ref, lse_ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["qo_indptr"],
                                      inp["kv_indptr"], w.scale, oracle.MASK_CAUSAL)
    check("causal prefill 2x4096 every row", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_decode_equals_last_prefill_row():
    """Decode of the last query over the whole sequence = last row of causal prefill."""
    L, Hq, Hkv, D = 777, 8, 2, 128
    g = synth.gen(22)
    q = synth.randn((L, Hq, D), torch.bfloat16, g)
    k = synth.randn((L, Hkv, D), torch.bfloat16, g)
    v = synth.randn((L, Hkv, D), torch.bfloat16, g)
    ind = synth.indptr([L])
    o_p, lse_p = prefill(q, k, v, ind, ind, True)
    o_d, lse_d = ra().attn_decode_splitkv(q[L - 1:L].contiguous().to(DEV), k.to(DEV), v.to(DEV),
                                          ind.to(DEV), L, num_splits=5)
    torch.cuda.synchronize()
    assert (o_p[L - 1].float() - o_d[0].float()).abs().max().item() <= 2 * TOL_O[torch.bfloat16]
    assert (lse_p[L - 1] - lse_d[0]).abs().max().item() <= 2e-3


def test_two_runs_bit_identical():
    qo = kv = synth.indptr([1000, 513])
    g = synth.gen(23)
    q = synth.randn((1513, 8, 128), torch.bfloat16, g)
    k = synth.randn((1513, 2, 128), torch.bfloat16, g)
    v = synth.randn((1513, 2, 128), torch.bfloat16, g)
    o1, l1 = prefill(q, k, v, qo, kv, True)
    o2, l2 = prefill(q, k, v, qo, kv, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---- split-KV prefill / append ---------------------------------------------

def prefill_split(q, k, v, qo, kv, causal, s, scale=None):
    lq = (qo[1:] - qo[:-1]).max().item()
    lk = (kv[1:] - kv[:-1]).max().item()
    o, lse = ra().attn_prefill_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), qo.to(DEV), kv.to(DEV),
                                       lq, lk, scale=scale, causal=causal, num_splits=s)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float16, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_splitkv_append_ragged(dtype, D, causal):
    """Few new tokens against long, ragged key histories (bottom-right causal);
    every split count agrees with the oracle, and with the others."""
    lens_q = [1, 7, 64, 130, 0]
    lens_k = [300, 1000, 2049, 5000, 70]
    Hkv, G = 2, 4
    qo, kv = synth.indptr(lens_q), synth.indptr(lens_k)
    g = synth.gen(60 + D + causal)
    q = synth.randn((sum(lens_q), G * Hkv, D), dtype, g)
    k = synth.randn((sum(lens_k), Hkv, D), dtype, g)
    v = synth.randn((sum(lens_k), Hkv, D), dtype, g)
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    o_ref, lse_ref = oracle.attention(q, k, v, qo, kv, 1 / D ** 0.5, mk)
    outs = []
    for s in (0, 1, 2, 3, 7, 40):
        o, lse = prefill_split(q, k, v, qo, kv, causal, s)
        check(f"splitkv {dtype} D={D} causal={causal} s={s}", o, o_ref, lse, lse_ref, dtype)
        outs.append(o.double().cpu())
    for x in outs[1:]:
        assert (x - outs[0]).abs().max().item() <= 2 * TOL_O[dtype]


def test_splitkv_equals_prefill_when_one_split():
    """s = 1 is attn_prefill itself: bit-identical output."""
    lens = [200, 65]
    qo, kv = synth.indptr(lens), synth.indptr(lens)
    g = synth.gen(77)
    q = synth.randn((sum(lens), 4, 128), torch.bfloat16, g)
    k = synth.randn((sum(lens), 2, 128), torch.bfloat16, g)
    v = synth.randn((sum(lens), 2, 128), torch.bfloat16, g)
    o1, l1 = prefill(q, k, v, qo, kv, True)
    o2, l2 = prefill_split(q, k, v, qo, kv, True, 1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_append_workload_every_row():
    """4 requests x 128 new tokens against 16,384 cached keys, 32/8 heads,
    D 128, bf16, bottom-right causal, automatic split count: every row."""
    w = synth.workload("append_prefill_bf16")
    inp = w.make(DEV)
    qo, kv = inp["qo_indptr"], inp["kv_indptr"]
    lq = (qo[1:] - qo[:-1]).max().item()
    lk = (kv[1:] - kv[:-1]).max().item()
    s = ra().attn_prefill_choose_splits(w.B, w.Hq, w.Hkv, w.D, lq, lk)
    assert s > 1
    o, lse = prefill_split(inp["q"], inp["k"], inp["v"], qo, kv, True, 0)
    o_ref, lse_ref = oracle.attention(inp["q"], inp["k"], inp["v"], qo, kv, w.scale,
                                      oracle.MASK_CAUSAL)
    check(f"append 4x128 vs 16384, s={s}, every row", o, o_ref, lse, lse_ref, torch.bfloat16)
