"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_qk_forward_treats_q_and_k_separately():
    """Layerwise QK-Norm normalises the query and the key rows each with its
    own statistic, width and weights (review: "Layerwise vs. headwise
    QK-Norm"; C4 has 5120-wide query rows and 1024-wide key rows)."""
    import numpy as np
    import oracle
    from attention_qk_norm_amd import workloads
    q = workloads.random_rows(3, 40, "f32", 1).numpy()
    k = workloads.random_rows(3, 8, "f32", 2).numpy() * np.float32(5)
    gq = workloads.random_weights(40, "f32", 3).numpy()
    gk = workloads.random_weights(8, "f32", 4).numpy()
    yq, yk = oracle.qk_forward(q, k, gq, gk, 1e-6)
    np.testing.assert_array_equal(yq, oracle.forward(q, gq, 1e-6)[0])
    np.testing.assert_array_equal(yk, oracle.forward(k, gk, 1e-6)[0])
    # the key rows' own statistic: rescaling k leaves y_q alone
    yq2, _ = oracle.qk_forward(q, k * np.float32(8), gq, gk, 1e-6)
    np.testing.assert_array_equal(yq2, yq)


def test_oracle_threads_do_not_change_results():
    import numpy as np
    import oracle
    from attention_qk_norm_amd import workloads
    x = workloads.random_rows(64, 512, "f32", 5).numpy()
    g = workloads.random_weights(512, "f32", 6).numpy()
    oracle.set_threads(1)
    y1, P1 = oracle.forward(x, g, 1e-6, 4)
    oracle.set_threads(4)
    try:
        y4, P4 = oracle.forward(x, g, 1e-6, 4)
    finally:
        oracle.set_threads(1)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(P1, P4)
