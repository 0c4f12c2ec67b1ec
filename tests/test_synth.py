"""The seeded input generators: determinism and the stated mask recipe."""
import torch

import synth


def test_same_seed_same_inputs():
    a = synth.workload("tiny_decode_fp32").make()
    b = synth.workload("tiny_decode_fp32").make()
    for key in ("q", "k", "v", "kv_indptr"):
        assert torch.equal(a[key], b[key])


def test_loguniform_lengths_range_and_determinism():
    n1 = synth.loguniform_lengths(64, 128, 32768, synth.gen(3))
    n2 = synth.loguniform_lengths(64, 128, 32768, synth.gen(3))
    assert n1 == n2 and all(128 <= n <= 32768 for n in n1)
    assert max(n1) > 8 * min(n1)  # spread over orders of magnitude


def test_sparse_mask_recipe():
    L, blk = 512, 64
    m = synth.sparse_mask(L, synth.gen(5), window=256, block=blk, globals_per_block=2,
                          random_blocks=2).bool()
    w = synth.window_mask(L, 256).bool()
    assert bool((m | ~w).all())                      # window included
    glob = torch.zeros(L, dtype=torch.bool)
    for b in range(L // blk):
        glob[b * blk:b * blk + 2] = True
    assert bool(m[:, glob].all()) and bool(m[glob, :].all())  # symmetric globals
    # every query block row has at least `random_blocks` fully valid key blocks
    nb = L // blk
    full = m.view(nb, blk, nb, blk).all(3).all(1)
    assert bool((full.sum(1) >= 2).all())


def test_window_mask_definition():
    m = synth.window_mask(6, 2)
    expect = torch.tensor([[1, 0, 0, 0, 0, 0], [1, 1, 0, 0, 0, 0], [0, 1, 1, 0, 0, 0],
                           [0, 0, 1, 1, 0, 0], [0, 0, 0, 1, 1, 0], [0, 0, 0, 0, 1, 1]],
                          dtype=torch.uint8)
    assert torch.equal(m, expect)


def test_stacked_workload_masks_differ():
    w = synth.workload("bsr_heads_prefill_fp16")
    m = w.mask()
    assert m.shape == (w.num_masks, w.L, w.L) and w.Hq % w.num_masks == 0
    assert not torch.equal(m[0], m[1])  # random blocks drawn per mask
    assert torch.equal(m, w.mask())     # deterministic
