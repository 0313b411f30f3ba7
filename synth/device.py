"""Device-side (PyTorch) generator for the multi-GiB workloads.

Same recipe as ``synth.mixture`` -- per-unit Gaussian-mixture keys with
centres on the radius-8 sphere, sigma = 1 noise, N(0, 1) values, queries near
a random centre -- drawn with a seeded ``torch.Generator`` on the GPU because
tens of GiB of host-side draws would take minutes.  Only random draws and
bf16 storage happen here.
"""

from __future__ import annotations

import torch


def fill_mixture(k_out: torch.Tensor, v_out: torch.Tensor, n_tokens: int, components: int,
                 seed: int, radius: float = 8.0, sigma: float = 1.0, chunk_units: int = 8):
    """Fill rows [0, n_tokens) of k_out/v_out ([U, capacity, d] bf16); return centres [U, C, d] f32."""
    U, _, d = k_out.shape
    g = torch.Generator(device=k_out.device)
    g.manual_seed(seed)
    centres = torch.randn((U, components, d), generator=g, device=k_out.device)
    centres = radius * centres / centres.norm(dim=2, keepdim=True)
    for u0 in range(0, U, chunk_units):
        u1 = min(U, u0 + chunk_units)
        z = torch.randint(0, components, (u1 - u0, n_tokens), generator=g, device=k_out.device)
        mu = torch.gather(centres[u0:u1], 1, z[..., None].expand(-1, -1, d))
        k = mu + sigma * torch.randn(mu.shape, generator=g, device=k_out.device)
        k_out[u0:u1, :n_tokens] = k.to(torch.bfloat16)
        v_out[u0:u1, :n_tokens] = torch.randn(mu.shape, generator=g, device=k_out.device).to(torch.bfloat16)
        del z, mu, k
    return centres


def queries(centres: torch.Tensor, group: int, seed: int) -> torch.Tensor:
    """One query per query head near a uniformly chosen centre: [U, group, d] bf16."""
    U, C, d = centres.shape
    g = torch.Generator(device=centres.device)
    g.manual_seed(seed)
    z = torch.randint(0, C, (U, group), generator=g, device=centres.device)
    mu = torch.gather(centres, 1, z[..., None].expand(-1, -1, d))
    return (mu + torch.randn(mu.shape, generator=g, device=centres.device)).to(torch.bfloat16).contiguous()


def rows(units: int, d: int, seed: int, device) -> torch.Tensor:
    """N(0, 1) rows [units, d] bf16 (new decoded keys / values)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((units, d), generator=g, device=device).to(torch.bfloat16).contiguous()


def init_indices(units: int, m: int, k: int, seed: int, device) -> torch.Tensor:
    """k distinct random indices in [0, m) per unit: [units, k] int32."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    r = torch.rand((units, m), generator=g, device=device)
    return torch.argsort(r, dim=1)[:, :k].to(torch.int32).contiguous()


def new_rows(centres: torch.Tensor, count: int, new_components: int, fraction: float, seed: int,
             radius: float = 8.0, sigma: float = 1.0):
    """Keys and values of `count` decoded tokens per unit: round(count * fraction)
    of them near `new_components` fresh centres, the rest near the unit's own
    centres, positions shuffled.  Returns (k, v), each [U, count, d] bf16."""
    U, C, d = centres.shape
    dev = centres.device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    n_new = int(round(count * fraction))
    z_old = torch.randint(0, C, (U, count - n_new), generator=g, device=dev)
    mu = torch.gather(centres, 1, z_old[..., None].expand(-1, -1, d))
    if n_new > 0 and new_components > 0:
        newc = torch.randn((U, new_components, d), generator=g, device=dev)
        newc = radius * newc / newc.norm(dim=2, keepdim=True)
        z_new = torch.randint(0, new_components, (U, n_new), generator=g, device=dev)
        mu = torch.cat([mu, torch.gather(newc, 1, z_new[..., None].expand(-1, -1, d))], dim=1)
    order = torch.argsort(torch.rand((U, count), generator=g, device=dev), dim=1)
    mu = torch.gather(mu, 1, order[..., None].expand(-1, -1, d))
    k = (mu + sigma * torch.randn(mu.shape, generator=g, device=dev)).to(torch.bfloat16).contiguous()
    v = torch.randn(mu.shape, generator=g, device=dev).to(torch.bfloat16).contiguous()
    return k, v
