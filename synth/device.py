"""Seeded synthetic K/V drawn directly in device memory (for the large
workloads whose inputs do not fit a host round trip).  Same laws as
synth.workloads.KVLaw, drawn with torch's device RNG; sampling only."""
from __future__ import annotations


def sample_kv_device(law, n_tokens: int, gen, device):
    """bfloat16 [n_tokens][H][128] on `device` following `law` (outlier or
    heavy-tailed channels per head)."""
    import torch
    H = law.num_heads
    x = torch.randn((n_tokens, H, 128), generator=gen, device=device, dtype=torch.float32)
    for h in range(H):
        ch = torch.as_tensor(law.channels[h], device=device, dtype=torch.long)
        if law.kind == "outlier":
            x[:, h, ch] *= law.scale
        else:
            # Student-t(nu): N / sqrt(chi2_nu / nu), chi2_nu = sum of nu squared normals
            nu = int(law.nu)
            z = torch.randn((n_tokens, len(ch)), generator=gen, device=device)
            c = torch.randn((n_tokens, len(ch), nu), generator=gen, device=device).square().sum(-1)
            x[:, h, ch] = z / torch.sqrt(c / law.nu) * law.scale
    return x.to(torch.bfloat16)


def sample_queries_device(batch: int, num_q_heads: int, gen, device):
    import torch
    return torch.randn((batch, num_q_heads, 128), generator=gen, device=device).to(torch.bfloat16)
