"""V-Smooth across denoising steps: which preparation each step runs.

The pages run V-Smooth inside every attention call of a diffusion model and
treat its cost as a scheduling trade: on the B200 it ran in the first quarter
of the steps only (runtimewire article; the chooseai.io brief counts the
clustering inside the attention call).  Consecutive steps see slowly changing
values, so the clustering can be carried from one step to the next:

* ``"cold"``  - k-means from the caller's initial token indices, cfg.iters
  passes (the first step, and every ``refresh`` steps if set);
* ``"warm"``  - ``warm_iters`` passes from the previous step's final centroids;
* ``"reuse"`` - the previous step's permutation, no clustering and no sort;
* ``"off"``   - V-Smooth off: identity order, zero block means.

Steps at or past ``ceil(vsmooth_frac * n_steps)`` run ``after`` ("off" or
"reuse").  The arithmetic of every mode is in the library
(``vsmooth_prepare_warm`` / ``vsmooth_prepare``); this module only decides
and keeps the carried state (centroids, permutation) on the device.
"""
from __future__ import annotations

import dataclasses
import math

import torch

from . import binding as vb


@dataclasses.dataclass(frozen=True)
class VSmoothSchedule:
    n_steps: int
    vsmooth_frac: float = 0.25
    warm_iters: int = 1
    after: str = "off"          # "off" or "reuse"
    refresh: int = 0            # > 0: a cold start every `refresh` steps inside the V-Smooth window

    def __post_init__(self):
        if self.n_steps < 1:
            raise ValueError("n_steps must be >= 1")
        if not 0.0 <= self.vsmooth_frac <= 1.0:
            raise ValueError("vsmooth_frac must lie in [0, 1]")
        if self.warm_iters < 1:
            raise ValueError("warm_iters must be >= 1")
        if self.after not in ("off", "reuse"):
            raise ValueError("after must be 'off' or 'reuse'")
        if self.refresh < 0:
            raise ValueError("refresh must be >= 0")

    @property
    def window(self) -> int:
        """Steps 0 .. window-1 run V-Smooth with clustering."""
        return math.ceil(self.vsmooth_frac * self.n_steps)

    def action(self, step: int) -> str:
        if not 0 <= step < self.n_steps:
            raise ValueError(f"step {step} outside 0..{self.n_steps - 1}")
        if step >= self.window:
            # "reuse" needs a permutation from a clustered step
            return self.after if self.window > 0 else "off"
        if step == 0 or (self.refresh and step % self.refresh == 0):
            return "cold"
        return "warm"


class VSmoothStepper:
    """Runs the scheduled preparation step by step for one attention layer,
    keeping the centroids and permutation between calls."""

    def __init__(self, cfg: vb.VcConfig, schedule: VSmoothSchedule):
        if not cfg.vsmooth:
            raise ValueError("the stepper needs a config with vsmooth on")
        self.cfg = cfg
        self.schedule = schedule
        self.centroids: torch.Tensor | None = None
        self.perm: torch.Tensor | None = None
        self.last_action: str | None = None

    def _cfg(self, vsmooth: bool, iters: int) -> vb.VcConfig:
        c = vb.VcConfig.from_buffer_copy(self.cfg)
        c.vsmooth = int(vsmooth)
        c.iters = iters
        return c

    def prepare(self, step: int, K: torch.Tensor, V: torch.Tensor, init_idx: torch.Tensor,
                out: vb.Prepared | None = None, ws: torch.Tensor | None = None) -> vb.Prepared:
        act = self.schedule.action(step)
        if act == "reuse" and self.perm is None:
            act = "cold"
        if act == "warm" and self.centroids is None:
            act = "cold"
        cshape = (self.cfg.B, self.cfg.H, self.cfg.n_clusters, self.cfg.d)
        if act == "off":
            prep = vb.vsmooth_prepare(self._cfg(False, self.cfg.iters), K, V, None, out=out, ws=ws)
        elif act == "reuse":
            prep = vb.vsmooth_prepare_warm(self.cfg, K, V, perm_in=self.perm, out=out, ws=ws)
        else:
            nxt = torch.empty(cshape, dtype=torch.float32, device=K.device)
            if act == "cold":
                prep = vb.vsmooth_prepare_warm(self.cfg, K, V, init_idx=init_idx, centroids_out=nxt, out=out, ws=ws)
            else:
                prep = vb.vsmooth_prepare_warm(self._cfg(True, self.schedule.warm_iters), K, V,
                                               init_centroids=self.centroids, centroids_out=nxt, out=out, ws=ws)
            self.centroids = nxt
            self.perm = prep.perm.clone()
        self.last_action = act
        return prep


__all__ = ["VSmoothSchedule", "VSmoothStepper"]
