"""Host logic of the synthetic workloads: the parameter counts the configs
state, and one data-parallel rank's share of a list."""
import workloads as W


def test_parameter_counts():
    assert W.llama2_100m().total_params == 109_529_856
    assert W.llama2_7b().total_params == 6_738_415_616
    assert len(W.llama2_7b().shapes) == 291
    assert W.llama2_13b_bf16().total_params == 13_015_864_320
    assert len(W.llama2_13b_bf16().shapes) == 363


def test_rank_shares_partition_the_list():
    """Eight ranks' shares cover the flattened list exactly once, in order, cut
    at multiples of 128 elements; whole tensors keep their shapes, cut ones
    become named 1-D pieces."""
    full = W.llama2_7b().shapes
    total = sum(W.numel(s) for _, s in full)
    flat = []  # (tensor name, start, end) in the order the ranks hold them
    for r in range(8):
        share = W.shard_shapes(full, r, 8)
        assert sum(W.numel(s) for _, s in share) == total // 8  # 7B divides evenly into 128-aligned eighths
        for name, s in share:
            if "[" in name:
                base, rng = name[:-1].split("[")
                a, b = (int(x) for x in rng.split(":"))
                assert len(s) == 1 and s[0] == b - a
            else:
                base, a, b = name, 0, W.numel(s)
            flat.append((base, a, b))
    # walking the pieces rebuilds every tensor from 0 to its size, in list order
    pos = {}
    order = []
    for base, a, b in flat:
        assert pos.get(base, 0) == a
        pos[base] = b
        if not order or order[-1] != base:
            order.append(base)
    assert order == [n for n, _ in full]
    assert all(pos[n] == W.numel(s) for n, s in full)
    # the cut points are 128-aligned in the flattened list
    off, cuts = 0, set()
    for r in range(8):
        cuts.add(off)
        off += sum(W.numel(s) for _, s in W.shard_shapes(full, r, 8))
    assert all(c % 128 == 0 for c in cuts)


def test_rank0_of_8_workload():
    w = W.llama2_7b_rank0_of_8()
    assert w.total_params == 842_301_952
    assert w.shapes[0][0] == "tok_embeddings" and w.shapes[-1][0] == "layers.3.w_gate[0:36971008]"
    assert W.shard_shapes([("x", (1000,))], 1, 3) == [("x[256:640]", (384,))]
