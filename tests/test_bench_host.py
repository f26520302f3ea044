"""Host-side logic of the benchmark (no GPU): the serving layout and the CPU oracle's partition."""

import bench
from workloads import synth


def test_serving_layout_concatenates_shared_inputs():
    groups = bench.serving_layout(synth.DENSE_LINEARS_QWEN3_8B)
    assert [g[0] for g in groups] == ["qkv_proj", "o_proj", "gate_up_proj", "down_proj"]
    assert dict((g[0], g[1:]) for g in groups) == {
        "qkv_proj": (6144, 4096), "o_proj": (4096, 4096), "gate_up_proj": (24576, 4096),
        "down_proj": (4096, 12288)}
    # same weight bytes as the separate linears
    assert sum(n * k for _, n, k in groups) == sum(n * k for _, n, k in synth.DENSE_LINEARS_QWEN3_8B)


def test_partition_by_bytes_assigns_each_tensor_once_and_balances():
    tensors = [("w", f"t{i}", 0, 0, 0, b) for i, b in enumerate([150, 150, 50, 50, 12, 12, 1, 1, 1])]
    for procs in (1, 2, 3, 4, 9):
        shares, load = bench.partition_by_bytes(tensors, procs)
        assert len(shares) == procs
        flat = sorted(t[1] for s in shares for t in s)
        assert flat == sorted(t[1] for t in tensors)
        assert load == [sum(t[-1] for t in s) for s in shares]
        # greedy largest-first: no share exceeds the lightest one by more than the largest item
        assert max(load) - min(load) <= max(t[-1] for t in tensors)
