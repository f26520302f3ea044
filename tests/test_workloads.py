"""Host checks of the seeded synthetic input generators (CPU only)."""

import torch

from workloads import synth


def test_weights_are_seeded_and_shaped():
    a = synth.weight_bf16(256, 384, seed=3, outlier_frac=0.001)
    b = synth.weight_bf16(256, 384, seed=3, outlier_frac=0.001)
    c = synth.weight_bf16(256, 384, seed=4, outlier_frac=0.001)
    assert a.dtype == torch.bfloat16 and a.shape == (256, 384)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    base = synth.weight_bf16(256, 384, seed=3)
    changed = (a.view(torch.int16) != base.view(torch.int16)).sum().item()
    assert changed <= round(0.001 * 256 * 384)
    assert 0.015 < a.float().std().item() < 0.03


def test_activation_outlier_channels():
    x = synth.act_bf16(64, 4096, seed=5).float()
    col_rms = x.pow(2).mean(0).sqrt()
    big = (col_rms > 8).sum().item()
    assert big == round(0.01 * 4096)


def test_moe_counts_sum_and_skew():
    counts = synth.moe_routing_counts(4096, 128, 8, seed=11)
    assert counts.sum().item() == 4096 * 8
    assert counts.max().item() > 4 * counts.float().median().item()
    off = synth.offsets_from_counts(counts)
    assert off[0].item() == 0 and off[-1].item() == 4096 * 8
    assert torch.all(off[1:] >= off[:-1])


def test_moe_routing_token_indices():
    """The router's token indices in expert order: the same picks as the counts, each expert's
    segment lists the distinct tokens that chose it in increasing order, and every token appears
    once per pick (top_k times)."""
    import torch

    T, E, k = 512, 16, 4
    counts, ids = synth.moe_routing(T, E, k, seed=12)
    assert torch.equal(counts, synth.moe_routing_counts(T, E, k, seed=12))
    assert ids.dtype == torch.int32 and ids.numel() == T * k
    off = synth.offsets_from_counts(counts)
    for e in range(E):
        seg = ids[int(off[e]):int(off[e + 1])]
        assert bool((seg[1:] > seg[:-1]).all())
    assert torch.equal(torch.bincount(ids.long(), minlength=T), torch.full((T,), k))
