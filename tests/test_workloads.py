"""The seeded generators: determinism, bf16 rounding, and the layout recipes."""
import numpy as np
import pytest

import workloads


def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # exact ties round to even
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(workloads.bf16_round(x), ref)
    bits = workloads.bf16_bits(x)
    assert np.array_equal(bits, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_tensors_deterministic_and_ordered():
    a = workloads.make_tensors(1, 2, 16, 8, "bf16", 7)
    b = workloads.make_tensors(1, 2, 16, 8, "bf16", 7)
    for n in a:
        assert np.array_equal(a[n], b[n])
    sub = workloads.make_tensors(1, 2, 16, 8, "bf16", 7, names=("v",))
    assert np.array_equal(sub["v"], a["v"])
    c = workloads.make_tensors(1, 2, 16, 8, "bf16", 8)
    assert not np.array_equal(a["q"], c["q"])
    f = workloads.make_tensors(1, 2, 16, 8, "fp32", 7)
    assert np.array_equal(workloads.bf16_round(f["q"]), a["q"])


def test_short_example_layout():
    w = workloads.get("packed_short_4k")
    seg = w.seg()
    assert seg.shape == (4, 4096) and seg.dtype == np.int32
    assert np.array_equal(seg, w.seg())
    for b in range(4):
        assert np.all(np.diff(seg[b]) >= 0) and seg[b, 0] == 0
        lens = workloads.segment_lengths(seg[b])
        assert sum(lens) == 4096
        assert all(8 <= L <= 1024 for L in lens[:-1])
        assert 20 <= len(lens) <= 80
    med = np.median(np.concatenate([workloads.segment_lengths(seg[b])[:-1] for b in range(4)]))
    assert 50 <= med <= 130


def test_long_document_layout():
    seg = workloads.get("packed_long_64k").seg()
    assert seg.shape == (1, 65536)
    lens = workloads.segment_lengths(seg[0])
    assert sum(lens) == 65536
    assert all(1024 <= L <= 16384 for L in lens[:-1]) and 1 <= lens[-1] <= 16384


def test_single_and_none_layouts():
    assert workloads.get("causal_16k").seg() is None
    s = workloads.get("tiny_causal_fp32").seg()
    assert s.shape == (1, 256) and not s.any()


def test_seg_from_lengths_rejects_bad_rows():
    with pytest.raises(ValueError):
        workloads.seg_from_lengths([[3, 4]], 8)
