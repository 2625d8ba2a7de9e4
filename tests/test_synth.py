"""The seeded input generator: definition, statistics, bf16 rounding."""
import numpy as np
import torch

import synth

M64 = (1 << 64) - 1


def _mix(x):
    # SplitMix64 output function (Vigna), written from its published definition
    z = (x + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_splitmix_reference_values():
    # First outputs of SplitMix64 seeded with 0 (state advances by the golden
    # gamma before each output): published test vector of the generator.
    assert _mix(0) == 0xE220A8397B1DCDAF
    assert _mix(0x9E3779B97F4A7C15) == 0x6E789E6AA1B965F4
    assert synth.mix(0) == 0xE220A8397B1DCDAF


def test_elements_match_definition():
    seed, sid = 3, 1017
    key = _mix(seed ^ ((sid * 0x9E3779B97F4A7C15) & M64))
    got = synth.normal_f32(seed, sid, 40, offset=1000)
    for j in range(40):
        i = 1000 + j
        s = 0
        for h in (_mix((key + 2 * i) & M64), _mix((key + 2 * i + 1) & M64)):
            s += sum((h >> (16 * q)) & 0xFFFF for q in range(4))
        want = np.float32((s - 262140) * (0.02 * np.sqrt(1.5) / 65536))
        assert got[j] == want


def test_statistics():
    x = synth.normal_f32(0, 5, 2_000_000).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 1e-4
    assert np.abs(x).max() <= 0.02 * 4 * np.sqrt(1.5) + 1e-9
    # excess kurtosis of an Irwin-Hall(8) sum is -1.2/8
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3
    assert abs(k + 0.15) < 0.02


def test_bf16_is_round_to_nearest_even():
    f = synth.normal_f32(0, 9, 100_000)
    b = synth.bf16_bits_to_f32(synth.normal_bf16_bits(0, 9, 100_000))
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(b, ref)
    # the one-pass fp32 form holds the same bf16 values, also at an offset
    assert np.array_equal(synth.normal_bf16_f32(0, 9, 100_000), ref)
    assert np.array_equal(synth.normal_bf16_f32(0, 9, 1000, offset=777), ref[777:1777])


def test_prompt_ids():
    p = synth.prompt(1, 5000, 1024)
    assert p.min() >= 0 and p.max() < 1024
    assert len(np.unique(p)) > 900
    assert np.array_equal(p, synth.prompt(1, 5000, 1024))
    assert not np.array_equal(p, synth.prompt(2, 5000, 1024))


def test_streams_differ():
    a = synth.normal_f32(0, synth.stream_id(synth.WQ, synth.TARGET, 0), 64)
    b = synth.normal_f32(0, synth.stream_id(synth.WQ, synth.TARGET, 1), 64)
    c = synth.normal_f32(0, synth.stream_id(synth.WQ, synth.DRAFT), 64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_static_tree_c2_follows_prior():
    """The c2 static tree is the 26 best rank paths (depth <= 5) under the
    context-free prior (0.6, 0.2, 0.1, 0.05), ties by depth then lexicographic."""
    import itertools
    q = np.log([0.6, 0.2, 0.1, 0.05])
    paths = [p for d in range(1, 6) for p in itertools.product(range(4), repeat=d)]

    def closed(sel):
        return all(p[:-1] in sel for p in sel if len(p) > 1)
    best = sorted(paths, key=lambda p: (-sum(q[list(p)]), len(p), p))[:26]
    assert closed(set(best))
    got = synth.STATIC_TREE_C2
    assert set(got) == set(best)
    assert [len(p) for p in got] == sorted(len(p) for p in got)
    assert [sum(1 for p in got if len(p) == d) for d in range(1, 6)] == [4, 8, 7, 5, 2]
