"""The seeded input generator: rounding, determinism and structure."""

import numpy as np
import torch

from block_sparse_attention_losa_amd import synth


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # include exact ties (low 16 bits = 0x8000) to exercise round-half-even
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = synth.round_bf16(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)


def test_round_bf16_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint between the bf16
    # neighbours 1 and 1 + 2^-7; a detour through float32 (which drops the
    # 2^-30) would land on the tie and round to even (1.0)
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8, -(1 + 3 * 2.0 ** -8)])
    assert synth.round_bf16(x).tolist() == [1 + 2.0 ** -7, 1.0, -(1 + 2 * 2.0 ** -7)]


def test_config_shapes_and_tails():
    want = {1: (1024, 16, 64), 2: (32760, 512, 56), 3: (32760, 512, 56),
            4: (118800, 929, 16), 5: (17776, 278, 48)}
    for cid, (n, nb, tail) in want.items():
        cfg = synth.CONFIGS[cid]
        assert cfg.seq_len == n and cfg.num_blocks == nb
        assert n - (nb - 1) * cfg.block == tail


def test_generator_is_deterministic_and_structured():
    cfg = synth.small_config(n_grid=(3, 4, 5), text=7, heads=2, head_dim=128, alpha=(2.0, 0.0))
    a = synth.make_inputs(cfg)
    b = synth.make_inputs(cfg)
    for x, y in zip(a, b):
        assert x.dtype == np.float32 and x.shape == (1, 2, 67, 128)
        assert np.array_equal(x, y)
    q, k, v = a
    # values are on the bf16 grid
    for x in a:
        assert np.array_equal(synth.round_bf16(x.astype(np.float64)), x.astype(np.float64))
    # Q, K and V of a head are independent draws
    assert not np.array_equal(q[0, 0], k[0, 0])
    # the positional term sits in dims 0..63 of video tokens only: with
    # alpha = 2, Q and K share it, so their video rows correlate there
    corr_pos = np.corrcoef(q[0, 0, 7:, :64].ravel(), k[0, 0, 7:, :64].ravel())[0, 1]
    corr_txt = np.corrcoef(q[0, 0, :7].ravel(), k[0, 0, :7].ravel())[0, 1]
    corr_pad = np.corrcoef(q[0, 0, 7:, 64:].ravel(), k[0, 0, 7:, 64:].ravel())[0, 1]
    assert corr_pos > 0.5 and abs(corr_txt) < 0.2 and abs(corr_pad) < 0.1
    # alpha = 0 head: no shared term
    assert abs(np.corrcoef(q[0, 1].ravel(), k[0, 1].ravel())[0, 1]) < 0.1


def test_alpha_draws():
    assert synth.alphas(synth.CONFIGS[1]).tolist() == [3.0, 0.0]
    a2 = synth.alphas(synth.CONFIGS[2])
    assert a2.shape == (12,) and set(a2.tolist()) <= {0.0, 1.0, 2.0, 3.0, 4.0}
    a4 = synth.alphas(synth.CONFIGS[4])
    assert a4.shape == (24,) and (a4 >= 0).all() and (a4 < 4).all()


def test_positions_flatten_t_major():
    cfg = synth.small_config(n_grid=(2, 3, 4))
    p = synth.positions(cfg)
    assert p.shape == (24, 3)
    # token (t*H + h)*W + w
    assert p[(1 * 3 + 2) * 4 + 3].tolist() == [1.0, 1.0, 1.0]
    assert p[(0 * 3 + 1) * 4 + 2].tolist() == [0.0, 0.5, 2 / 3]
