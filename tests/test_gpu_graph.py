"""Entry points captured in HIP graphs (torch.cuda.CUDAGraph on ROCm).

No entry point allocates, fills memory or synchronises, so a serving loop
can capture them.  Each graph is replayed several times, with eager work of
the program and synchronisations between the replays, and every replay must
equal the eager result bit for bit.
"""
import pytest
import torch

import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def ra():
    import reduction_attention_amd
    return reduction_attention_amd


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def check_replays(g, outs, eager, noise):
    """Replay g three times; before each, scribble over the outputs with
    eager work and synchronise; after each, compare with the eager result."""
    for rep in range(3):
        noise()
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, want in zip(outs, eager):
            assert torch.equal(t, want), f"replay {rep} differs from the eager result"


def test_decode_chunk_and_flat_in_graphs():
    lengths = [700, 1, 64, 0, 513, 2048]
    q, k, v, kv = synth.decode_inputs(len(lengths), 8, 2, 128, lengths, torch.bfloat16, seed=3)
    q, k, v, kv = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    B, Hq, D = q.shape
    for plan in ("chunk", "flat"):
        o = torch.empty_like(q)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
        if plan == "chunk":
            s = 5
            ws = torch.empty(ra().attn_decode_workspace_bytes(B, Hq, D, s), dtype=torch.uint8,
                             device=DEV)
            call = lambda st: ra().attn_decode_splitkv(q, k, v, kv, max(lengths), num_splits=s, o=o,
                                                       lse=lse, workspace=ws, stream=st)
        else:
            P = 7
            ws = torch.empty(ra().attn_decode_flat_workspace_bytes(B, Hq, D, max(lengths),
                                                                   k.shape[0], P),
                             dtype=torch.uint8, device=DEV)
            call = lambda st: ra().attn_decode_splitkv_flat(q, k, v, kv, max(lengths), num_pieces=P,
                                                            o=o, lse=lse, workspace=ws, stream=st)
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        eager = (o.clone(), lse.clone())
        g = capture(call)
        scratch = torch.randn(1 << 20, device=DEV)
        check_replays(g, (o, lse), eager, lambda: scratch.mul_(1.0001))


def test_decode_noalloc_in_graph():
    """The entry point that allocates nothing, for callers under graph
    capture: its split partials live in the library's own device array, so
    the graph holds no workspace.  (The first call, made eagerly here as a
    serving loop would before capturing, looks the array's address up.)"""
    lengths = [700, 1, 64, 0, 513, 2048]
    q, k, v, kv = synth.decode_inputs(len(lengths), 8, 2, 128, lengths, torch.bfloat16, seed=5)
    q, k, v, kv = q.to(DEV), k.to(DEV), v.to(DEV), kv.to(DEV)
    B, Hq, D = q.shape
    s = 5
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
    call = lambda st: ra().attn_decode_splitkv_noalloc(q, k, v, kv, max(lengths), o, lse=lse,
                                                        num_splits=s, stream=st)
    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    ws = torch.empty(ra().attn_decode_workspace_bytes(B, Hq, D, s), dtype=torch.uint8, device=DEV)
    o2, l2 = ra().attn_decode_splitkv(q, k, v, kv, max(lengths), num_splits=s, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, eager[0]) and torch.equal(l2, eager[1])
    g = capture(call)
    scratch = torch.randn(1 << 20, device=DEV)
    check_replays(g, (o, lse), eager, lambda: scratch.mul_(1.0001))


def test_mla_and_prefill_in_one_graph():
    g0 = synth.gen(4)
    qm = synth.randn((3, 16, 576), torch.bfloat16, g0).to(DEV)
    cm = synth.randn((900, 576), torch.bfloat16, g0).to(DEV)
    kvm = synth.indptr([400, 200, 300]).to(DEV)
    om = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=DEV)
    lm = torch.empty((3, 16), dtype=torch.float32, device=DEV)
    wsm = torch.empty(ra().attn_mla_decode_workspace_bytes(3, 16, 4), dtype=torch.uint8, device=DEV)
    qo, kvp = synth.indptr([300, 64]), synth.indptr([300, 130])
    q = synth.randn((364, 8, 128), torch.bfloat16, g0).to(DEV)
    k = synth.randn((430, 2, 128), torch.bfloat16, g0).to(DEV)
    v = synth.randn((430, 2, 128), torch.bfloat16, g0).to(DEV)
    qo, kvp = qo.to(DEV), kvp.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty((364, 8), dtype=torch.float32, device=DEV)

    def call(st):
        ra().attn_mla_decode(qm, cm, kvm, 400, 192 ** -0.5, num_splits=4, o=om, lse=lm,
                             workspace=wsm, stream=st)
        ra().attn_prefill(q, k, v, qo, kvp, 300, 300, causal=True, o=o, lse=lse, stream=st)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = (om.clone(), lm.clone(), o.clone(), lse.clone())
    g = capture(call)
    scratch = torch.randn(1 << 20, device=DEV)
    check_replays(g, (om, lm, o, lse), eager, lambda: scratch.add_(1.0))
