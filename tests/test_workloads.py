"""The seeded input generators: reproducible, right shapes, outlier channels."""
import numpy as np
import torch

import workloads as WL


def test_shapes_dtypes_and_reproducibility():
    w = WL.workload(1)
    W1, W2 = WL.weight(w), WL.weight(w)
    assert W1.shape == (512, 512) and W1.dtype == torch.float16
    assert torch.equal(W1, W2)
    X = WL.calibration(w)
    assert X.shape == (64, 512)
    idx, b = WL.channel_boosts(w)
    assert len(idx) == 5 and np.all(b[idx] == 20) and np.sum(b != 1) == 5
    # boosted channels have ~20x the mean |x|
    m = X.float().abs().mean(0).numpy()
    others = np.setdiff1d(np.arange(512), idx)
    assert m[idx].mean() > 10 * m[others].mean()


def test_outlier_counts_per_config():
    assert len(WL.channel_boosts(WL.workload(2))[0]) == 20
    assert len(WL.channel_boosts(WL.workload(3, "q"))[0]) == 41
    assert len(WL.channel_boosts(WL.workload(3, "down"))[0]) == 110
    assert len(WL.channel_boosts(WL.workload(4, "up"))[0]) == 82
    assert len(WL.channel_boosts(WL.workload(4, "down"))[0]) == 287
    _, b = WL.channel_boosts(WL.workload(2))
    boosted = b[b != 1]
    assert 5 < np.median(boosted) < 40


def test_shared_inputs_share_channels():
    # q/k/v read the same input tensor: same outlier channels
    a = WL.channel_boosts(WL.workload(3, "q"))[0]
    b = WL.channel_boosts(WL.workload(3, "v"))[0]
    assert np.array_equal(a, b)
    assert WL.workload(4).dtype == torch.bfloat16


def test_alpha_grid_endpoints():
    a = WL.alpha_grid(20)
    assert a[0] == 0.0 and a[-1] == 1.0 and len(a) == 20
