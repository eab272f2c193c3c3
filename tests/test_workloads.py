"""Seeded input generators: determinism, storage formats, shapes."""
import numpy as np

import workloads as W


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 tie -> up to 1+2^-6; above the tie rounds up
    assert W.f32_to_bf16_bits(f).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]


def test_generators_are_deterministic_and_lazy():
    w = W.scaled(W.MID, T=64, E=16, d=64, d_ff=32)
    a = W.expert_weights(w, 5)
    stacked = W.all_expert_weights(w)
    for part, full in zip(a, stacked):
        assert np.array_equal(part, full[5])
    assert np.array_equal(W.router_logits(w), W.router_logits(w))
    assert np.array_equal(W.tokens(w), W.tokens(w))
    assert W.tokens(w).dtype == np.uint16


def test_zipf_bias_skews_router():
    z = W.router_logits(W.scaled(W.MID, T=4096))
    top = np.argmax(z, axis=1)
    counts = np.bincount(top, minlength=128)
    assert counts[0] > 3 * counts[64:].mean()


def test_recv_pools_layout():
    w = W.scaled(W.RECV, n_src=3, pool_rows=10, d=16)
    pools = W.recv_pools(w, 1)
    ids = W.recv_local_ids(w, 1)
    assert pools.shape == (3, 11, 16)
    assert np.array_equal(pools[:, 0, :10], ids)
    assert np.all(pools[:, 0, 10:] == 0xFFFF)
    assert ids.max() < 6
