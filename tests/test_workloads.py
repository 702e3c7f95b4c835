"""The seeded input generators (CPU): the normal generator does not depend on
the thread count, and the counter-based generator's two forms (numpy for any
indices, torch integer ops for whole tensors) agree bit for bit and follow
their definition."""

import numpy as np
import torch

import workloads as wl


def test_normal_tensor_independent_of_workers():
    shp = (1, 2, 3, 5, 2, 128)
    a = wl.normal_tensor(shp, 1234, 1)
    cpu = wl.make_inputs(wl.WORKLOADS["tiny"], workers=1)
    cpu4 = wl.make_inputs(wl.WORKLOADS["tiny"], workers=4)
    assert a.shape == shp and a.dtype == np.float32
    for x, y in zip(cpu, cpu4):
        assert torch.equal(x, y)


def test_hash_generators_agree_and_follow_the_definition():
    t = torch.empty((5, 999), dtype=torch.bfloat16)
    wl.hash_fill_(t, 3, 8.0, chunk=1000)                  # several chunks, a ragged last one
    idx = np.arange(t.numel())
    np.testing.assert_array_equal(t.float().numpy().ravel(), wl.hash_values(3, idx, 8.0))
    # the definition, element by element with Python integers
    for i in (0, 1, 4094, 4994):
        h = (i * 2654435761 + 3 * 40503) % 2 ** 32
        v = np.float32((h >> 8) / 2 ** 24 - 0.5) * np.float32(8.0)
        want = torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16).float().item()
        assert wl.hash_values(3, [i], 8.0)[0] == want
    # other tensors draw other values; the range is [-0.5, 0.5) times the gain
    assert not np.array_equal(wl.hash_values(4, idx[:100]), wl.hash_values(3, idx[:100]))
    v = wl.hash_values(0, np.arange(1 << 16))
    assert v.min() >= -0.5 and v.max() <= 0.5
