"""GPU parity of block-sparse prefill (BSR outer tiles + 8x8 bitmaps)."""
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, TOL_O, check

pytestmark = pytest.mark.gpu


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


def bsr(q, k, v, dense, kernel="block"):
    m = ra().attn_bsr_encode_host(dense).to(DEV)
    o, lse = ra().attn_prefill_bsr(q.to(DEV), k.to(DEV), v.to(DEV), m, kernel=kernel)
    torch.cuda.synchronize()
    return o, lse, m


def qkv(B, L, Hq, Hkv, D, dtype, seed):
    g = synth.gen(seed)
    return (synth.randn((B, L, Hq, D), dtype, g), synth.randn((B, L, Hkv, D), dtype, g),
            synth.randn((B, L, Hkv, D), dtype, g))


def oracle_bsr(q, k, v, dense, scale):
    B, L = q.shape[:2]
    outs, lses = [], []
    for b in range(B):
        o, lse = oracle.attention(q[b], k[b], v[b], [0, L], [0, L], scale, oracle.MASK_DENSE, dense)
        outs.append(o)
        lses.append(lse)
    return torch.stack(outs), torch.stack(lses)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["sparse", "window", "random", "causal"])
def test_small_masks(dtype, D, kind):
    L, B, Hq, Hkv = 384, 2, 4, 2
    if kind == "sparse":
        dense = synth.sparse_mask(L, synth.gen(31), window=96, block=64, globals_per_block=2,
                                  random_blocks=1)
    elif kind == "window":
        dense = synth.window_mask(L, 100)
    elif kind == "random":
        dense = (torch.rand(L, L, generator=synth.gen(32)) < 0.2).to(torch.uint8)
        dense[:, 128:256] = 0
        dense[70] = 0  # a query row with no valid key
    else:
        dense = torch.ones(L, L, dtype=torch.uint8).tril()
    q, k, v = qkv(B, L, Hq, Hkv, D, dtype, 33 + D)
    o_ref, lse_ref = oracle_bsr(q, k, v, dense, 1 / D ** 0.5)
    o, lse, _ = bsr(q, k, v, dense)
    check(f"bsr {dtype} D={D} {kind}", o, o_ref, lse, lse_ref, dtype)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_part_tiles_by_quadrant(dtype, D):
    """Part tiles whose valid elements sit in chosen 32x32 quadrants: every
    subset of the four (query half, key half) quadrants occurs once, so each
    wave meets tiles where both, one or neither of its 32-key halves hold a
    valid element."""
    L, B, Hq, Hkv = 256, 2, 4, 2
    g = synth.gen(41)
    dense = torch.zeros(L, L, dtype=torch.uint8)
    for qb in range(4):
        for kb in range(4):
            combo = 4 * qb + kb
            for quad in range(4):
                if not (combo >> quad) & 1:
                    continue
                w, kh = quad >> 1, quad & 1
                r0, c0 = 64 * qb + 32 * w, 64 * kb + 32 * kh
                bits = (torch.rand(32, 32, generator=g) < 0.3).to(torch.uint8)
                bits[int(torch.randint(0, 32, (1,), generator=g))][
                    int(torch.randint(0, 32, (1,), generator=g))] = 1
                dense[r0:r0 + 32, c0:c0 + 32] = bits
    q, k, v = qkv(B, L, Hq, Hkv, D, dtype, 43 + D)
    o_ref, lse_ref = oracle_bsr(q, k, v, dense, 1 / D ** 0.5)
    o, lse, m = bsr(q, k, v, dense)
    assert m.nnz_full == 0 and m.nnz_part == 15
    check(f"bsr quadrants {dtype} D={D}", o, o_ref, lse, lse_ref, dtype)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_large_grid(dtype):
    """D 64 on a grid of more workgroups than fit at once (16 block rows x
    64 heads x 2 = 2048), rows with up to 16 stored tiles split in halves."""
    L, B, Hq, Hkv, D = 1024, 2, 64, 8, 64
    dense = synth.sparse_mask(L, synth.gen(51), window=128, block=64, globals_per_block=2,
                              random_blocks=2)
    q, k, v = qkv(B, L, Hq, Hkv, D, dtype, 53)
    o_ref, lse_ref = oracle_bsr(q, k, v, dense, 1 / D ** 0.5)
    o, lse, _ = bsr(q, k, v, dense)
    check(f"bsr large grid {dtype}", o, o_ref, lse, lse_ref, dtype)


def oracle_workload(w, inp):
    """Every (token, head) row of a block-sparse workload by the oracle, one
    call per stacked mask over the query heads it serves (MHA: KV head h
    serves query head h)."""
    assert w.Hkv == w.Hq and w.B == 1
    M = w.num_masks
    masks = inp["mask"] if M > 1 else inp["mask"].unsqueeze(0)
    hpm = w.Hq // M
    q, k, v = (inp[x][0].cpu() for x in ("q", "k", "v"))
    o = torch.empty((w.L, w.Hq, w.D), dtype=torch.float64)
    lse = torch.empty((w.L, w.Hq), dtype=torch.float64)
    for mi in range(M):
        hs = slice(mi * hpm, (mi + 1) * hpm)
        o[:, hs], lse[:, hs] = oracle.attention(q[:, hs], k[:, hs], v[:, hs], [0, w.L],
                                                [0, w.L], w.scale, oracle.MASK_DENSE, masks[mi])
    return o.unsqueeze(0), lse.unsqueeze(0)


@pytest.mark.parametrize("name", ["bsr_prefill_fp16", "bsr_window_prefill_fp16",
                                  "bsr_cols_prefill_fp16", "bsr_heads_prefill_fp16",
                                  "bsr_long_prefill_fp16"])
def test_workload_every_row(name):
    """The block-sparse workloads (L 4096 with the sparse recipe, with its
    window alone and with column globals over a narrow window; L 8192 and
    16384 with one mask per 4 heads), fp16, D 64: every row of both kernels
    against the oracle."""
    w = synth.workload(name)
    inp = w.make(DEV)
    m = ra().attn_bsr_encode_host(inp["mask"])
    print(f"{name}: L={w.L} masks={m.num_masks} full={m.nnz_full} part={m.nnz_part}; "
          "oracle over every row ...", flush=True)
    o_ref, lse_ref = oracle_workload(w, inp)
    md = m.to(DEV)
    for kernel in ("block", "row"):
        o, lse = ra().attn_prefill_bsr(inp["q"], inp["k"], inp["v"], md, kernel=kernel)
        torch.cuda.synchronize()
        check(f"{name} {kernel}-wise every row", o, o_ref, lse, lse_ref, torch.float16)


def test_unstored_tiles_never_read():
    """NaN in K/V of every key block no query row may see leaves the output bit-identical."""
    L, D = 512, 64
    dense = synth.window_mask(L, 100)
    dense[:, 192:256] = 0  # key block 3 is empty in every row
    q, k, v = qkv(1, L, 2, 2, D, torch.float16, 41)
    o1, l1, m = bsr(q, k, v, dense)
    k2, v2 = k.clone(), v.clone()
    # poison key block 3, which no query block row stores
    k2[:, 192:256] = float("nan")
    v2[:, 192:256] = float("nan")
    o2, l2, _ = bsr(q, k2, v2, dense)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_mask_equals_causal_prefill():
    L, Hq, Hkv, D = 512, 4, 2, 128
    q, k, v = qkv(1, L, Hq, Hkv, D, torch.bfloat16, 42)
    dense = torch.ones(L, L, dtype=torch.uint8).tril()
    o_b, lse_b, _ = bsr(q, k, v, dense)
    ind = synth.indptr([L]).to(DEV)
    o_p, lse_p = ra().attn_prefill(q[0].to(DEV), k[0].to(DEV), v[0].to(DEV), ind, ind, L, L,
                                   causal=True)
    torch.cuda.synchronize()
    assert (o_b[0].float() - o_p.float()).abs().max().item() <= 2 * TOL_O[torch.bfloat16]
    assert (lse_b[0] - lse_p).abs().max().item() <= 2e-3


@pytest.mark.parametrize("kind", ["sparse", "random", "workload"])
def test_device_decode_bit_exact(kind):
    if kind == "workload":
        dense = synth.workload("bsr_prefill_fp16").mask()
    elif kind == "sparse":
        dense = synth.sparse_mask(512, synth.gen(51), window=100, block=64, globals_per_block=2,
                                  random_blocks=2)
    else:
        dense = (torch.rand(256, 256, generator=synth.gen(52)) < 0.5).to(torch.uint8)
    m = ra().attn_bsr_encode_host(dense).to(DEV)
    got = ra().attn_debug_bsr_decode(m).cpu()
    assert torch.equal(got, dense)


def oracle_bsr_heads(q, k, v, dense3, scale):
    """Per-head masks through the one-mask oracle, one query head at a time:
    head h takes mask h // (Hq / M) and KV head h // (Hq / Hkv)."""
    B, L, Hq, _ = q.shape
    M, g = dense3.shape[0], Hq // k.shape[2]
    o = torch.zeros(q.shape, dtype=torch.float64)
    lse = torch.zeros((B, L, Hq), dtype=torch.float64)
    for h in range(Hq):
        kh = h // g
        oh, lh = oracle_bsr(q[:, :, h:h + 1], k[:, :, kh:kh + 1], v[:, :, kh:kh + 1],
                            dense3[h // (Hq // M)], scale)
        o[:, :, h:h + 1] = oh
        lse[:, :, h:h + 1] = lh
    return o, lse


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("num_masks", [2, 4])
def test_per_head_masks(dtype, D, num_masks):
    """Stacked masks: each head (group) sees only its own mask."""
    L, B, Hq, Hkv = 320, 2, 4, 2
    kinds = [synth.window_mask(L, 90),
             synth.sparse_mask(L, synth.gen(61), window=64, block=64, globals_per_block=2,
                               random_blocks=1),
             torch.ones(L, L, dtype=torch.uint8).tril(),
             (torch.rand(L, L, generator=synth.gen(62)) < 0.25).to(torch.uint8)]
    dense3 = torch.stack(kinds[:num_masks])
    q, k, v = qkv(B, L, Hq, Hkv, D, dtype, 63 + D)
    o_ref, lse_ref = oracle_bsr_heads(q, k, v, dense3, 1 / D ** 0.5)
    o, lse, m = bsr(q, k, v, dense3)
    assert m.num_masks == num_masks
    check(f"bsr heads M={num_masks} {dtype} D={D}", o, o_ref, lse, lse_ref, dtype)


def test_per_head_masks_equal_separate_calls():
    """Mask per head in one call == one single-mask call per head, bit for bit."""
    L, Hq, D = 256, 4, 64
    dense3 = torch.stack([synth.window_mask(L, 40 + 30 * h) for h in range(Hq)])
    q, k, v = qkv(1, L, Hq, Hq, D, torch.float16, 64)
    o, lse, _ = bsr(q, k, v, dense3)
    for h in range(Hq):
        oh, lh, _ = bsr(q[:, :, h:h + 1].contiguous(), k[:, :, h:h + 1].contiguous(),
                        v[:, :, h:h + 1].contiguous(), dense3[h])
        assert torch.equal(o[:, :, h:h + 1], oh) and torch.equal(lse[:, :, h:h + 1], lh)


# ---- row-wise kernel -----------------------------------------------------------

def small_mask(kind, L, seed):
    if kind == "sparse":
        return synth.sparse_mask(L, synth.gen(seed), window=96, block=64, globals_per_block=2,
                                 random_blocks=1)
    if kind == "window":
        return synth.window_mask(L, 100)
    if kind == "cols":  # columns-only globals plus a narrow window: sparse part tiles
        d = synth.window_mask(L, 8)
        d[:, ::64] = 1
        d[:, 1::64] = 1
        return d
    if kind == "random":
        d = (torch.rand(L, L, generator=synth.gen(seed)) < 0.05).to(torch.uint8)
        d[70] = 0  # a query row with no valid key
        d[:, 128:192] = 0
        return d
    return torch.ones(L, L, dtype=torch.uint8).tril()


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["sparse", "window", "cols", "random", "causal"])
def test_rows_small_masks(dtype, D, kind):
    L, B, Hq, Hkv = 320, 2, 4, 2
    dense = small_mask(kind, L, 81)
    q, k, v = qkv(B, L, Hq, Hkv, D, dtype, 83 + D)
    o_ref, lse_ref = oracle_bsr(q, k, v, dense, 1 / D ** 0.5)
    o, lse, _ = bsr(q, k, v, dense, kernel="row")
    check(f"bsr rows {dtype} D={D} {kind}", o, o_ref, lse, lse_ref, dtype)


@pytest.mark.parametrize("D", [64, 128])
def test_rows_per_head_masks(D):
    L, B, Hq, Hkv = 256, 1, 4, 4
    dense3 = torch.stack([small_mask(kd, L, 90 + n)
                          for n, kd in enumerate(["cols", "random", "window", "sparse"])])
    q, k, v = qkv(B, L, Hq, Hkv, D, torch.bfloat16, 95)
    o_ref, lse_ref = oracle_bsr_heads(q, k, v, dense3, 1 / D ** 0.5)
    o, lse, m = bsr(q, k, v, dense3, kernel="row")
    check(f"bsr rows heads D={D}", o, o_ref, lse, lse_ref, torch.bfloat16)


def test_rows_unread_blocks_never_read():
    """NaN in K/V of a 16-key block in which no query row holds a valid
    element (keys 48..63, inside stored outer tiles) leaves the row-wise
    output bit-identical: the kernel never loads such a block."""
    L, D = 256, 64
    dense = small_mask("cols", L, 0)
    dense[:, 48:64] = 0
    q, k, v = qkv(1, L, 2, 2, D, torch.float16, 96)
    o1, l1, m = bsr(q, k, v, dense, kernel="row")
    assert m.nnz_full + m.nnz_part == 16  # every outer tile stays stored
    k2, v2 = k.clone(), v.clone()
    k2[:, 48:64] = float("nan")
    v2[:, 48:64] = float("nan")
    o2, l2, _ = bsr(q, k2, v2, dense, kernel="row")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_auto_kernel_matches_choice():
    """kernel="auto" runs the selector's choice: bit-identical to that kernel."""
    L, D = 512, 64
    dense = small_mask("cols", L, 0)
    q, k, v = qkv(1, L, 2, 2, D, torch.float16, 97)
    m = ra().attn_bsr_encode_host(dense)
    choice = m.plan(D, 2, 1)["kernel"]
    md = m.to(DEV)
    assert md.plan(D, 2, 1)["kernel"] == choice
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    oa, la = ra().attn_prefill_bsr(qd, kd, vd, md, kernel="auto")
    oc, lc = ra().attn_prefill_bsr(qd, kd, vd, md, kernel=choice)
    torch.cuda.synchronize()
    assert torch.equal(oa, oc) and torch.equal(la, lc)
