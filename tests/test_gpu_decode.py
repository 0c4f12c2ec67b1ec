"""GPU parity of split-KV decode and the LSE merge against the fp64 oracle."""
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, TOL_O, check, report

pytestmark = pytest.mark.gpu


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


def run_decode(w_inputs, max_len, s, **kw):
    q, k, v, kv = (w_inputs[x].to(DEV) for x in ("q", "k", "v", "kv_indptr"))
    o, lse = ra().attn_decode_splitkv(q, k, v, kv, max_len, num_splits=s, **kw)
    torch.cuda.synchronize()
    return o, lse


def oracle_decode(inp, scale):
    B = inp["q"].shape[0]
    return oracle.attention(inp["q"], inp["k"], inp["v"], list(range(B + 1)), inp["kv_indptr"],
                            scale)


def test_tiny_fp32_split_counts_agree():
    """Tiny GQA decode, fp32: 4 query heads on 1 KV head, D 64, 256 keys, s in {1, 2, 4}."""
    w = synth.workload("tiny_decode_fp32")
    inp = w.make()
    o_ref, lse_ref = oracle_decode(inp, w.scale)
    outs = []
    for s in w.splits:
        o, lse = run_decode(inp, w.L, s)
        check(f"tiny fp32 s={s}", o, o_ref, lse, lse_ref, torch.float32)
        outs.append(o.double().cpu())
    for a in outs[1:]:
        assert (a - outs[0]).abs().max().item() <= 2 * TOL_O[torch.float32]


def test_llama3_8b_decode_full_parity():
    """B 16, 32/8 heads, D 128, 4096 keys each, bf16, automatic s (every row checked)."""
    w = synth.workload("llama3_8b_decode_bf16")
    inp = w.make(DEV)
    o_ref, lse_ref = oracle_decode(inp, w.scale)
    s_auto = ra().attn_decode_choose_splits(w.B, w.Hq, w.Hkv, w.D, w.B * w.L, w.L)
    print(f"automatic split count s={s_auto}", flush=True)
    o, lse = run_decode(inp, w.L, 0)
    check("llama3-8b decode auto-s", o, o_ref, lse, lse_ref, torch.bfloat16)
    o1, lse1 = run_decode(inp, w.L, 1)
    check("llama3-8b decode s=1", o1, o_ref, lse1, lse_ref, torch.bfloat16)


@pytest.mark.parametrize("kind", ["one_shorter", "jittered"])
def test_nearly_equal_lengths_take_the_equal_length_shape(kind):
    """Lengths that differ a little (mean at least 15/16 of the longest) take
    the equal-length decode shape and its batched merge; with s = 16 the
    shorter request has fewer splits than s, so the merge's batch holds
    slots the request never wrote.  Every row."""
    if kind == "one_shorter":
        lengths = [4096] * 15 + [3840]
    else:
        g = torch.Generator().manual_seed(12)
        lengths = torch.randint(4090, 4097, (16,), generator=g).tolist()
    assert 16 * sum(lengths) >= 15 * 16 * max(lengths)
    q, k, v, kv = synth.decode_inputs(16, 32, 8, 128, lengths, torch.bfloat16, seed=13)
    scale = 128 ** -0.5
    o_ref, lse_ref = oracle.attention(q, k, v, list(range(17)), kv, scale)
    qd, kd, vd, kvd = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    for s in (0, 3, 8, 16):
        print(f"nearly equal lengths ({kind}) s={s}", flush=True)
        o, lse = ra().attn_decode_splitkv(qd, kd, vd, kvd, max(lengths), num_splits=s)
        torch.cuda.synchronize()
        check(f"nearly equal lengths {kind} s={s}", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_ragged_serving_decode_full_parity():
    """64 requests, 64/8 heads, D 128, log-uniform lengths in [128, 32768], bf16."""
    w = synth.workload("ragged_decode_bf16")
    inp = w.make(DEV)
    lengths = inp["lengths"]
    print(f"ragged lengths: total={sum(lengths)} min={min(lengths)} max={max(lengths)}", flush=True)
    o_ref, lse_ref = oracle_decode(inp, w.scale)
    o, lse = run_decode(inp, max(lengths), 0)
    check("ragged decode auto-s", o, o_ref, lse, lse_ref, torch.bfloat16)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
def test_small_ragged_shapes(dtype, D, G):
    lengths = [1, 31, 32, 33, 0, 300, 64, 517]
    Hkv = 2
    q, k, v, kv = synth.decode_inputs(len(lengths), G * Hkv, Hkv, D, lengths, dtype, seed=D + G)
    inp = dict(q=q, k=k, v=v, kv_indptr=kv)
    scale = 1.0 / D ** 0.5
    o_ref, lse_ref = oracle_decode(inp, scale)
    for s in (1, 3, 8, 64):
        o, lse = run_decode(inp, max(lengths), s)
        check(f"decode {dtype} D={D} G={G} s={s}", o, o_ref, lse, lse_ref, dtype)
    # the empty request: O = 0, LSE = -inf
    assert bool((o[4] == 0).all()) and bool(torch.isinf(lse[4]).all())


@pytest.mark.parametrize("Hkv", [1, 2, 6])
def test_equal_lengths_head_groups(Hkv):
    """Equal request lengths take the multi-head workgroup shape (up to four KV
    heads per workgroup; Hkv = 6 leaves idle head slots in the last one)."""
    lengths = [300] * 5
    G = 4
    q, k, v, kv = synth.decode_inputs(len(lengths), G * Hkv, Hkv, 128, lengths, torch.bfloat16,
                                      seed=40 + Hkv)
    inp = dict(q=q, k=k, v=v, kv_indptr=kv)
    o_ref, lse_ref = oracle_decode(inp, 128 ** -0.5)
    for s in (0, 1, 2, 5, 19):
        o, lse = run_decode(inp, max(lengths), s)
        check(f"equal lengths Hkv={Hkv} s={s}", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_split_ranges_bit_exact():
    import reduction_attention_amd as r
    lengths = [1, 31, 32, 33, 0, 300, 4096, 517, 7]
    kv = synth.indptr(lengths)
    for s in (1, 2, 3, 8, 17, 256):
        got = r.attn_debug_split_ranges(kv.to(DEV), max(lengths), s).cpu().to(torch.int64)
        want = oracle.split_ranges(kv, max(lengths), s)
        assert torch.equal(got, want), s


def test_merge_kernel_matches_oracle_merge():
    s, rows, D = 6, 50, 128
    g = synth.gen(11)
    op = torch.randn((s, rows, D), generator=g)
    mp = torch.randn((s, rows), generator=g) * 4
    lp = torch.rand((s, rows), generator=g) * 10 + 0.01
    # unused partials: m = -inf, l = 0, o = NaN (must not be read)
    lp[2, :10] = 0
    mp[2, :10] = float("-inf")
    op[2, :10] = float("nan")
    lp[:, 20] = 0
    mp[:, 20] = float("-inf")  # a row with no partial at all
    o_ref, lse_ref = oracle.merge(op, mp, lp)
    for dt in (torch.float32, torch.bfloat16):
        o, lse = ra().attn_merge_lse(op.to(DEV), mp.to(DEV), lp.to(DEV), o_dtype=dt)
        torch.cuda.synchronize()
        check(f"merge -> {dt}", o, o_ref, lse, lse_ref, dt)


def test_constant_keys_give_mean_of_v():
    lengths = [200, 1000]
    q, k, v, kv = synth.decode_inputs(2, 8, 2, 128, lengths, torch.bfloat16, seed=12)
    k[:] = k[0:1]  # one key vector everywhere (per KV head)
    o, lse = run_decode(dict(q=q, k=k, v=v, kv_indptr=kv), 1000, 4)
    for b, (lo, hi) in enumerate([(0, 200), (200, 1200)]):
        mean_v = v[lo:hi].double().mean(0)  # [Hkv, D]
        want = mean_v.repeat_interleave(4, dim=0)
        assert (o[b].double().cpu() - want).abs().max().item() <= TOL_O[torch.bfloat16]


def test_two_runs_bit_identical():
    w = synth.workload("llama3_8b_decode_bf16")
    inp = w.make(DEV)
    o1, l1 = run_decode(inp, w.L, 8)
    o2, l2 = run_decode(inp, w.L, 8)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_outputs_only_where_expected():
    """NaN canaries around o and lse stay untouched."""
    lengths = [100, 40]
    q, k, v, kv = synth.decode_inputs(2, 8, 2, 128, lengths, torch.bfloat16, seed=13)
    o_buf = torch.full((3 * 2 * 8 * 128,), float("nan"), dtype=torch.bfloat16, device=DEV)
    l_buf = torch.full((3 * 16,), float("nan"), dtype=torch.float32, device=DEV)
    o = o_buf[2 * 8 * 128: 2 * 2 * 8 * 128].view(2, 8, 128)
    lse = l_buf[16:32].view(2, 8)
    ra().attn_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV), 100, num_splits=3,
                             o=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o_buf[:2048]).all()) and bool(torch.isnan(o_buf[4096:]).all())
    assert bool(torch.isnan(l_buf[:16]).all()) and bool(torch.isnan(l_buf[32:]).all())
    o_ref, lse_ref = oracle_decode(dict(q=q, k=k, v=v, kv_indptr=kv), 1 / 128 ** 0.5)
    report("canary decode", o, o_ref, lse, lse_ref)


def test_workspace_reused_across_calls():
    """One workspace (with stale contents) serves calls of other shapes."""
    ws = torch.full((1 << 22,), 255, dtype=torch.uint8, device=DEV)
    for lengths, Hq, s in [([900, 5, 64, 2000], 8, 8), ([33, 1500], 16, 3), ([900, 5, 64, 2000], 8, 8)]:
        q, k, v, kv = synth.decode_inputs(len(lengths), Hq, 2, 128, lengths, torch.bfloat16,
                                          seed=len(lengths) + Hq)
        o, lse = ra().attn_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV),
                                          max(lengths), num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_decode(dict(q=q, k=k, v=v, kv_indptr=kv), 1 / 128 ** 0.5)
        check(f"reuse B={len(lengths)} s={s}", o, o_ref, lse, lse_ref, torch.bfloat16)


@pytest.mark.parametrize("s", [1, 3, 8])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_partials_match_oracle_split(s, dtype, D):
    """attn_decode_partials against the oracle's per-split partials, then merged
    (bf16 on the MFMA kernel, fp32 on the four-wave VALU kernel)."""
    lengths = [700, 1, 64, 0, 513]
    q, k, v, kv = synth.decode_inputs(len(lengths), 8, 2, D, lengths, dtype, seed=s)
    o_ref, lse_ref, op_ref, mp_ref, lp_ref = oracle.split_decode(q, k, v, kv, max(lengths),
                                                                 1 / D ** 0.5, s)
    op, mp, lp = ra().attn_decode_partials(q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV),
                                           max(lengths), s)
    torch.cuda.synchronize()
    used = lp_ref > 0
    assert torch.equal(lp.cpu() > 0, used)
    assert bool(torch.isinf(mp.cpu()[~used]).all())
    do = (op.cpu().double() - op_ref)[used].abs().max().item()
    dm = (mp.cpu().double() - mp_ref)[used].abs().max().item()
    dl = ((lp.cpu().double() - lp_ref) / lp_ref)[used].abs().max().item()
    print(f"partials {dtype} s={s}: max|do|={do:.2e} max|dm|={dm:.2e} max rel dl={dl:.2e}",
          flush=True)
    assert do <= TOL_O[dtype] and dm <= 1e-3 and dl <= 1e-3
    o, lse = ra().attn_merge_lse(op, mp, lp, o_dtype=torch.float32)
    torch.cuda.synchronize()
    check(f"partials+merge {dtype} s={s}", o.view(len(lengths), 8, D), o_ref,
          lse.view(len(lengths), 8), lse_ref, dtype)


# ---- flat split plan (packed key array cut into equal pieces) -------------

def run_flat(inp, max_len, P, **kw):
    q, k, v, kv = (inp[x].to(DEV) for x in ("q", "k", "v", "kv_indptr"))
    o, lse = ra().attn_decode_splitkv_flat(q, k, v, kv, max_len, num_pieces=P, **kw)
    torch.cuda.synchronize()
    return o, lse


def test_flat_ranges_bit_exact():
    lengths = [1, 31, 32, 33, 0, 300, 4096, 517, 7, 0]
    kv = synth.indptr(lengths)
    total = sum(lengths)
    for P in (1, 2, 3, 7, 64, 256, 5117):
        got = ra().attn_debug_flat_ranges(kv.to(DEV), max(lengths), total, P).cpu().to(torch.int64)
        want = oracle.flat_ranges(kv, total, P, got.shape[1])
        assert got.shape[1] == oracle.flat_max_splits(total, max(lengths), P)
        assert torch.equal(got, want), P


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hkv,G", [(1, 8), (2, 16), (3, 4), (8, 8), (12, 1)])
def test_flat_small_ragged(dtype, D, Hkv, G):
    """Pieces spanning several requests, requests spanning several pieces,
    empty requests, and head groups that leave idle wave slots (Hkv 3, 12)."""
    lengths = [1, 31, 32, 33, 0, 300, 64, 517, 0]
    q, k, v, kv = synth.decode_inputs(len(lengths), G * Hkv, Hkv, D, lengths, dtype,
                                      seed=D + G + Hkv)
    inp = dict(q=q, k=k, v=v, kv_indptr=kv)
    o_ref, lse_ref = oracle_decode(inp, 1.0 / D ** 0.5)
    for P in (0, 1, 2, 5, 31, 978):
        o, lse = run_flat(inp, max(lengths), P)
        check(f"flat {dtype} D={D} Hkv={Hkv} G={G} P={P}", o, o_ref, lse, lse_ref, dtype)
    assert bool((o[4] == 0).all()) and bool(torch.isinf(lse[8]).all())


def test_flat_all_requests_empty():
    lengths = [0, 0, 0]
    q, k, v, kv = synth.decode_inputs(3, 8, 2, 128, lengths, torch.bfloat16, seed=3)
    k = torch.zeros((16, 2, 128), dtype=torch.bfloat16)  # rows no request owns
    v = k.clone()
    o = torch.full((3, 8, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    o, lse = ra().attn_decode_splitkv_flat(q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV), 0, o=o)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isinf(lse).all()) and bool((lse < 0).all())


def test_flat_ragged_serving_full_parity():
    """The ragged serving-like workload through the flat plan, every row."""
    w = synth.workload("ragged_decode_bf16")
    inp = w.make(DEV)
    L = inp["lengths"]
    P = ra().attn_decode_flat_pieces(w.B, w.Hq, w.Hkv, w.D, sum(L))
    print(f"flat plan: P={P} piece={-(-sum(L) // P)} "
          f"slots={ra().attn_decode_flat_max_splits(max(L), sum(L), P)}", flush=True)
    o_ref, lse_ref = oracle_decode(inp, w.scale)
    o, lse = run_flat(inp, max(L), 0)
    check("ragged decode, flat plan", o, o_ref, lse, lse_ref, torch.bfloat16)
    o2, lse2 = run_flat(inp, max(L), 0)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_flat_equals_oracle_split_partials():
    """The flat plan's merged result against the oracle's split decode over
    the same ranges, and the Llama-shaped batch (equal lengths)."""
    lengths = [700, 1, 64, 0, 513, 2048]
    q, k, v, kv = synth.decode_inputs(len(lengths), 8, 2, 128, lengths, torch.bfloat16, seed=9)
    P = 6
    rg = oracle.flat_ranges(kv, sum(lengths), P)
    o_ref, lse_ref, *_ = oracle.split_decode(q, k, v, kv, max(lengths), 1 / 128 ** 0.5, 0,
                                             ranges=rg)
    o, lse = run_flat(dict(q=q, k=k, v=v, kv_indptr=kv), max(lengths), P)
    check("flat P=6 vs oracle split decode", o, o_ref, lse, lse_ref, torch.bfloat16)
    w = synth.workload("llama3_8b_decode_bf16")
    inp = w.make(DEV)
    o_ref, lse_ref = oracle_decode(inp, w.scale)
    o, lse = run_flat(inp, w.L, 0)
    check("llama3-8b decode, flat plan", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_flat_rows_outside_requests_not_read():
    """Key rows before kv_indptr[0] and after kv_indptr[B] hold NaN; the
    flat plan's pieces cover them but no request owns them, so they are
    never read."""
    q, k, v, _ = synth.decode_inputs(2, 8, 2, 128, [300, 200], torch.bfloat16, seed=21)
    kk = torch.full((700, 2, 128), float("nan"), dtype=torch.bfloat16)
    vv = kk.clone()
    kk[50:550], vv[50:550] = k, v
    kv = torch.tensor([50, 350, 550], dtype=torch.int32)
    o_ref, lse_ref = oracle.attention(q, kk, vv, [0, 1, 2], kv, 1 / 128 ** 0.5)
    assert torch.isfinite(o_ref).all()
    for P in (1, 3, 7, 700):
        o, lse = ra().attn_decode_splitkv_flat(q.to(DEV), kk.to(DEV), vv.to(DEV), kv.to(DEV),
                                               300, num_pieces=P)
        torch.cuda.synchronize()
        check(f"flat outside rows P={P}", o, o_ref, lse, lse_ref, torch.bfloat16)
