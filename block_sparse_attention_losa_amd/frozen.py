"""Per-layer registry of frozen block lists, for applying the method across
the attention layers of a diffusion transformer.

The construction step measures the block masses of every layer and keeps, per
(batch, head, query block), the smallest key-block set reaching the threshold;
every later denoising step reuses those lists unchanged (mlsanity.com paper
index, "Abstract (arXiv)"; legiblepapers, "Summary & Methodology Analysis":
per layer, head and query block; ubos.tech blog, "How It Works in Practice",
Phase 2: the mask is stored for reuse).  :class:`FrozenLists` holds those
lists on the device, one entry per layer name, runs the construction step and
the later sparse steps through the C-ABI, and saves / loads them with
safetensors so a generation can resume from its frozen state.

Only bookkeeping happens here; every computation is a call into
``liblosa.so``.
"""

import json

import torch

from . import api

_FORMAT = "losa-frozen-lists/1"


class FrozenLists:
    """Frozen lists of several attention layers.

    Each layer entry holds ``idx`` ``[B, H, nb, nb]`` and ``count``
    ``[B, H, nb]`` (int32, device), the block size, head dim and threshold it
    was built with, and a launch plan made on first use.
    """

    def __init__(self, block: int = 64, threshold: float = 0.99, max_workspace_bytes=None):
        self.block = int(block)
        self.threshold = threshold
        # cap on the construction step's workspace (None: the full size, one
        # pass over every head); a smaller one costs more passes, not results
        self.max_workspace_bytes = max_workspace_bytes
        self._layers = {}

    # ------------------------------------------------------------ contents
    def __contains__(self, layer):
        return str(layer) in self._layers

    def __len__(self):
        return len(self._layers)

    def layers(self):
        return list(self._layers)

    def lists(self, layer):
        """``(idx, count)`` of a layer."""
        e = self._layers[str(layer)]
        return e["idx"], e["count"]

    def kept_fraction(self, layer) -> float:
        e = self._layers[str(layer)]
        nb = e["count"].shape[-1]
        return float(e["count"].sum().item()) / (e["count"].numel() * nb)

    def set_lists(self, layer, idx, count, head_dim: int, block: int = None, threshold=None):
        """Register lists made elsewhere (validated for shape and type)."""
        block = self.block if block is None else int(block)
        if idx.dtype != torch.int32 or count.dtype != torch.int32:
            raise TypeError("idx and count must be int32")
        if idx.dim() != 4 or count.dim() != 3 or tuple(idx.shape[:3]) != tuple(count.shape) \
                or idx.shape[2] != idx.shape[3]:
            raise ValueError("idx must be [B, H, nb, nb] and count [B, H, nb]")
        self._layers[str(layer)] = {
            "idx": idx.contiguous(), "count": count.contiguous(), "block": block,
            "head_dim": int(head_dim),
            "threshold": self.threshold if threshold is None else threshold, "plan": None}

    # ------------------------------------------------------------ steps
    def construct(self, layer, q, k, v, threshold=None, rows_per_threshold=None, o=None,
                  workspace=None):
        """Construction step of one layer: dense attention with the block mass
        map in one sweep, threshold selection, lists kept.  ``threshold`` is a
        number, or a float64 device tensor with one value per
        ``rows_per_threshold`` rows of the mass map (e.g. per head:
        ``rows_per_threshold = nb``).  Returns the dense attention output
        ``o`` of this step."""
        tau = self.threshold if threshold is None else threshold
        o, _, mass = api.dense_attn_mass(q, k, v, block=self.block, o=o, want_lse=False,
                                         workspace=workspace,
                                         max_workspace_bytes=self.max_workspace_bytes)
        if torch.is_tensor(tau):
            idx, count = api.select_per_row(mass, tau, rows_per_threshold or 1)
            tau_meta = "per-row"
        else:
            idx, count = api.select(mass, float(tau))
            tau_meta = float(tau)
        del mass
        self.set_lists(layer, idx, count, q.shape[-1], self.block, tau_meta)
        return o

    def _plan(self, e):
        if e["plan"] is None:
            e["plan"] = api.sparse_plan(e["count"], block=e["block"], head_dim=e["head_dim"])
        return e["plan"]

    def attend(self, layer, q, k, v, o=None, want_lse=False):
        """A later step of one layer: block-sparse attention over its frozen
        lists (in the launch plan's order).  Returns ``(o, lse)``."""
        e = self._layers[str(layer)]
        if q.shape[-1] != e["head_dim"] or tuple(q.shape[:2]) != tuple(e["count"].shape[:2]):
            raise ValueError("inputs do not match the layer's frozen lists")
        return api.sparse_attn(q, k, v, e["idx"], e["count"], block=e["block"], o=o,
                               want_lse=want_lse, plan=self._plan(e))

    def retained_mass(self, layer, q, k, v):
        """Drift diagnostic of one layer on a later step's inputs: per query
        block, the share of the dense attention mass its frozen list covers."""
        e = self._layers[str(layer)]
        _, lse_k = api.sparse_attn(q, k, v, e["idx"], e["count"], block=e["block"],
                                   want_lse=True, plan=self._plan(e))
        _, lse_d = api.dense_attn(q, k, v, block=e["block"])
        return api.retained_mass(lse_k, lse_d, block=e["block"], head_dim=e["head_dim"])

    def mask(self, layer):
        """The layer's lists as a uint8 ``[B, H, nb, nb]`` mask."""
        e = self._layers[str(layer)]
        return api.block_mask(e["idx"], e["count"])

    # ------------------------------------------------------------ storage
    def save(self, path):
        """Write every layer's lists to a safetensors file (entries of idx at
        and past count are stored as they are)."""
        from safetensors.torch import save_file

        tensors, meta = {}, {}
        for name, e in self._layers.items():
            tensors[f"{name}/idx"] = e["idx"].detach().cpu().contiguous()
            tensors[f"{name}/count"] = e["count"].detach().cpu().contiguous()
            meta[name] = {"block": e["block"], "head_dim": e["head_dim"],
                          "threshold": e["threshold"]}
        save_file(tensors, str(path), metadata={
            "format": _FORMAT, "block": str(self.block),
            "threshold": json.dumps(self.threshold if not torch.is_tensor(self.threshold)
                                    else "per-row"),
            "layers": json.dumps(meta)})

    @classmethod
    def load(cls, path, device="cuda"):
        """Read lists written by :meth:`save` onto ``device``; launch plans
        are rebuilt on first use."""
        from safetensors import safe_open

        with safe_open(str(path), framework="pt", device="cpu") as fh:
            meta = fh.metadata() or {}
            if meta.get("format") != _FORMAT:
                raise ValueError(f"{path} is not a frozen-lists file")
            layers = json.loads(meta["layers"])
            out = cls(block=int(meta["block"]), threshold=json.loads(meta["threshold"]))
            for name, m in layers.items():
                idx = fh.get_tensor(f"{name}/idx").to(device)
                count = fh.get_tensor(f"{name}/count").to(device)
                out.set_lists(name, idx, count, m["head_dim"], m["block"], m["threshold"])
        return out
