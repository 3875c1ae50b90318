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
    if law.mix is not None:
        mix = torch.as_tensor(law.mix, device=device, dtype=torch.float32)
        x = torch.einsum("nhc,hcd->nhd", x, mix).contiguous()
    return x.to(torch.bfloat16)


def sample_queries_device(batch: int, num_q_heads: int, gen, device):
    import torch
    return torch.randn((batch, num_q_heads, 128), generator=gen, device=device).to(torch.bfloat16)


def fill_bf16_pages_device(pages, k, v, table_row):
    """Place the tokens of one sequence (bfloat16 [L][H][128] on the device)
    into the all-BF16 paged cache `pages` (bfloat16 [num_pages][H][4096]):
    position p goes to slot p % 16 of page table_row[p // 16], K token-major
    (element 128 slot + c), V channel-major (element 2048 + 16 c + slot).
    Data placement only; slots past L in the last page are left as they were
    (zero-padded here)."""
    import torch
    L, H, D = k.shape
    n = (L + 15) // 16
    pad = n * 16 - L
    if pad:
        k = torch.cat([k, k.new_zeros((pad, H, D))])
        v = torch.cat([v, v.new_zeros((pad, H, D))])
    idx = table_row[:n].long()
    pages[idx, :, :2048] = k.reshape(n, 16, H, D).permute(0, 2, 1, 3).reshape(n, H, 2048)
    pages[idx, :, 2048:] = v.reshape(n, 16, H, D).permute(0, 2, 3, 1).reshape(n, H, 2048)
