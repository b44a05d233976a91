"""CPU checks of the per-layer registry of frozen lists: validation, the
kept fraction and a safetensors save / load round trip (no GPU needed; the
construction and sparse steps are covered by the GPU tests)."""

import json

import pytest
import torch

from block_sparse_attention_losa_amd import FrozenLists


def _lists(b, h, nb, seed):
    g = torch.Generator().manual_seed(seed)
    idx = torch.stack([torch.randperm(nb, generator=g) for _ in range(b * h * nb)])
    idx = idx.reshape(b, h, nb, nb).to(torch.int32)
    count = torch.randint(1, nb + 1, (b, h, nb), generator=g, dtype=torch.int32)
    return idx, count


def test_round_trip(tmp_path):
    reg = FrozenLists(block=64, threshold=0.99)
    lists = {"blocks.0.attn": _lists(1, 3, 9, 0), "blocks.1.attn": _lists(2, 2, 5, 1)}
    for name, (idx, count) in lists.items():
        reg.set_lists(name, idx, count, head_dim=128)
    reg.set_lists("blocks.2.attn", *_lists(1, 1, 3, 2), head_dim=64, block=128, threshold=0.95)
    path = tmp_path / "frozen.safetensors"
    reg.save(path)
    back = FrozenLists.load(path, device="cpu")
    assert back.layers() == reg.layers() and len(back) == 3
    for name in reg.layers():
        for a, b in zip(reg.lists(name), back.lists(name)):
            assert torch.equal(a, b)
        assert back.kept_fraction(name) == reg.kept_fraction(name)
    e = back._layers["blocks.2.attn"]
    assert (e["block"], e["head_dim"], e["threshold"]) == (128, 64, 0.95)
    assert back.block == 64 and back.threshold == 0.99


def test_kept_fraction_and_validation():
    reg = FrozenLists()
    idx = torch.zeros((1, 1, 4, 4), dtype=torch.int32)
    count = torch.tensor([[[1, 2, 3, 4]]], dtype=torch.int32)
    reg.set_lists("a", idx, count, head_dim=64)
    assert reg.kept_fraction("a") == 10 / 16
    assert "a" in reg and "b" not in reg
    with pytest.raises(TypeError):
        reg.set_lists("b", idx.long(), count, head_dim=64)
    with pytest.raises(ValueError):
        reg.set_lists("b", idx[..., :3], count, head_dim=64)
    with pytest.raises(ValueError):
        reg.set_lists("b", idx, count[..., :3], head_dim=64)


def test_load_rejects_other_files(tmp_path):
    from safetensors.torch import save_file

    path = tmp_path / "other.safetensors"
    save_file({"x": torch.zeros(2)}, str(path), metadata={"format": "something-else"})
    with pytest.raises(ValueError):
        FrozenLists.load(path, device="cpu")
    assert json.loads(json.dumps({"ok": 1}))["ok"] == 1
