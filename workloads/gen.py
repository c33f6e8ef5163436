"""Seeded synthetic inputs for the five workloads.

This module draws random numbers and lays them out; it computes nothing of
the method.  The same code runs on the CPU or on a GPU (``device``): torch's
generator for that device, seeded from the workload id and the layer, draws
every value.  CPU and GPU draws differ from each other, but each is
deterministic, and a test always hands the oracle the very bytes it gave
the library.

Recipe for one layer of workload ``cfg`` (all float32 draws, then rounded
round-to-nearest-even to the workload dtype):

* Q ``[B, H, n_q, d]`` ~ N(0, 1);
* prompt keys ``[B, H, N_p, d]`` ~ N(0, 1), or Student-t with 4 degrees of
  freedom, built as z0 / sqrt((z1^2 + z2^2 + z3^2 + z4^2) / 4) from five
  standard normals;
* prompt values, generated keys and generated values ~ N(0, 1);
* per (sequence, head) ``n_spans`` non-overlapping spans at random offsets,
  lengths uniform in ``span_len``; their keys are replaced by
  ``alpha * mean_i(q_i) + noise * N(0, 1)`` (the "needles");
* the generated positions are rows ``[N_p, N_p + N_g)``.

Layout: K and V are ``[B, H, N_p + N_g, d]`` with the prompt first.
"""

from dataclasses import dataclass

import numpy as np
import torch

from .configs import CONFIGS, Config

SEED_BASE = 20261202


def _torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def layer_seed(cid, layer):
    """64-bit seed for (workload, layer), derived with numpy's SeedSequence."""
    ss = np.random.SeedSequence(SEED_BASE, spawn_key=(cid, layer))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def span_layout(cfg, layer, b, h):
    """Planted span (offset, length) pairs for one head, non-overlapping, sorted."""
    rng = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(SEED_BASE, spawn_key=(cfg.cid, layer, b, h, 1))))
    lo, hi = cfg.span_len
    lens = rng.integers(lo, hi + 1, size=cfg.n_spans)
    free = cfg.n_prompt - int(lens.sum())
    if free < 0:
        raise ValueError("spans do not fit the prompt")
    cuts = np.sort(rng.integers(0, free + 1, size=cfg.n_spans))
    order = rng.permutation(cfg.n_spans)
    lens = lens[order]
    offs = cuts + np.concatenate([[0], np.cumsum(lens)[:-1]])
    return [(int(o), int(n)) for o, n in zip(offs, lens)]


@dataclass
class LayerInputs:
    cfg: Config
    layer: int
    q: torch.Tensor        # [B, H, n_q, d]
    k: torch.Tensor        # [B, H, N_tot, d]
    v: torch.Tensor        # [B, H, N_tot, d]
    gen_idx: torch.Tensor  # int32 [N_g]
    spans: dict            # (b, h) -> [(offset, length)]


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_layer(cfg, layer=0, device="cpu", spans=True):
    """Draw one layer of workload ``cfg`` on ``device``."""
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    gen = torch.Generator(device=device)
    gen.manual_seed(layer_seed(cfg.cid, layer))
    B, H, d = cfg.batch, cfg.heads, cfg.head_dim
    n_p, n_g = cfg.n_prompt, cfg.n_gen
    q = _randn((B, H, cfg.n_q, d), gen, device)
    k = torch.empty((B, H, n_p + n_g, d), dtype=torch.float32, device=device)
    if cfg.key_law == "normal":
        k[:, :, :n_p] = _randn((B, H, n_p, d), gen, device)
    elif cfg.key_law == "student_t4":
        # Student-t(4): a standard normal over the root of a chi-square(4)/4,
        # the chi-square being a sum of four squared standard normals.
        # Drawn one head at a time to bound the temporary memory.
        for b in range(B):
            for h in range(H):
                z = _randn((5, n_p, d), gen, device)
                chi = (z[1:] * z[1:]).sum(dim=0) / 4.0
                k[b, h, :n_p] = z[0] / torch.sqrt(chi)
    else:
        raise ValueError(cfg.key_law)
    v = torch.empty_like(k)
    v[:, :, :n_p] = _randn((B, H, n_p, d), gen, device)
    k[:, :, n_p:] = _randn((B, H, n_g, d), gen, device)
    v[:, :, n_p:] = _randn((B, H, n_g, d), gen, device)
    layout = {}
    if spans and cfg.n_spans:
        qbar = q.mean(dim=2)  # [B, H, d]
        for b in range(B):
            for h in range(H):
                lay = span_layout(cfg, layer, b, h)
                layout[(b, h)] = lay
                for off, n in lay:
                    noise = _randn((n, d), gen, device)
                    k[b, h, off:off + n] = cfg.alpha * qbar[b, h] + cfg.noise * noise
    dt = _torch_dtype(cfg.dtype)
    gen_idx = torch.arange(n_p, n_p + n_g, dtype=torch.int32, device=device)
    return LayerInputs(cfg, layer, q.to(dt), k.to(dt), v.to(dt), gen_idx, layout)


def to_f64(t):
    """Exact float64 numpy copy of a (possibly device, possibly bf16) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
