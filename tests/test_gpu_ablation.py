"""GPU keep-fp16 channel ablation against the oracle: the channel lists chosen by activation
and by weight magnitude bit-exact, the four output-MSE losses within 1e-5 relative (the bar
of the search losses)."""
import numpy as np
import pytest

import oracle
import weight_only_quantization_gemm_amd as awq
from gen import activations_fp16, normal_fp16
from test_gpu_parity import dev, host, note

pytestmark = pytest.mark.gpu


def _ablate(W, X, n_keep, seed, bits=4):
    K = W.shape[1]
    rnd = np.random.default_rng(seed).permutation(K)[:n_keep].astype(np.int32)
    r = awq.awq_keep_fp16_ablation(dev(W), dev(X), n_keep, dev(rnd) if n_keep else None, bits=bits)
    ref = oracle.keep_fp16_ablation(W, X, n_keep, rnd, bits=bits)
    assert np.array_equal(host(r["keep_activation"]), ref["keep_activation"])
    assert np.array_equal(host(r["keep_weight"]), ref["keep_weight"])
    L, Lr = host(r["loss"]), ref["losses"]
    nz = Lr > 0
    assert np.all(np.abs(L[nz] - Lr[nz]) <= 1e-5 * Lr[nz]), (L, Lr)
    assert np.all(L[~nz] == 0.0)
    return L


@pytest.mark.parametrize("N,K,M,n_keep,bits,lognormal", [
    (64, 512, 32, 5, 4, False),     # direct form of the loss (M < K)
    (64, 512, 600, 5, 4, True),     # Gram form (M >= K)
    (100, 384, 50, 0, 4, False),    # nothing kept: plain rounding
    (48, 256, 300, 256, 4, False),  # everything kept: zero loss
    (96, 640, 300, 7, 3, True),     # 3-bit codes
    (17, 128, 1, 2, 4, False),      # one calibration row
])
def test_ablation_parity(N, K, M, n_keep, bits, lognormal):
    note(f"ablation N={N} K={K} M={M} keep={n_keep} bits={bits}")
    W = normal_fp16((N, K), 0.02, seed=800 + N + K)
    X = activations_fp16(M, K, seed=801 + M, lognormal=lognormal)
    L = _ablate(W, X, n_keep, seed=802, bits=bits)
    if n_keep == 0:
        assert L[0] == L[1] == L[2] == L[3]
    if n_keep == K:
        assert np.all(L[1:] == 0.0)


def test_ablation_ties_go_to_lower_channels():
    note("ablation ties")
    K = 256
    g = np.random.default_rng(9)
    X = (g.choice([-2.0, 2.0], size=(40, K))).astype(np.float16)   # every channel: mean |x| = 2
    W = (g.choice([-0.5, 0.5], size=(32, K))).astype(np.float16)   # every channel: mean |w| = 0.5
    W[:, 200] = np.float16(0.75)                                     # one channel of larger weights
    r = awq.awq_keep_fp16_ablation(dev(W), dev(X), 4, dev(np.arange(4, dtype=np.int32)))
    assert list(host(r["keep_activation"])) == [0, 1, 2, 3]
    assert list(host(r["keep_weight"])) == [200, 0, 1, 2]


def test_ablation_activation_choice_wins_on_outlier_layer():
    """The pages' observation on a synthetic layer with 1% of input channels carrying x20
    activations: keeping those channels recovers much more than keeping the largest-weight
    or random channels."""
    note("ablation observation N=512 K=4096 M=2048")
    W = normal_fp16((512, 4096), 0.02, seed=810)
    X = activations_fp16(2048, 4096, seed=811, lognormal=True)
    L = _ablate(W, X, 41, seed=812)
    note(f"  L none {L[0]:.4e} act {L[1]:.4e} weight {L[2]:.4e} random {L[3]:.4e}")
    assert L[1] < L[2] and L[1] < L[3] and L[1] < L[0]
