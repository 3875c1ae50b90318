"""The benchmark fills its all-BF16 paged cache with synth.device's
placement helper; on CPU tensors it must place every token exactly where the
oracle's writer does (same format, independent code)."""
import numpy as np

import oracle as O
import synth
from synth.device import fill_bf16_pages_device


def test_device_fill_matches_oracle_writer():
    import torch
    rng = np.random.default_rng(21)
    H, L, n_pool = 3, 37, 9
    table = rng.permutation(n_pool).astype(np.int32)[None, :3]
    k = synth.f32_to_bf16_bits(rng.standard_normal((L, H, 128)))
    v = synth.f32_to_bf16_bits(rng.standard_normal((L, H, 128)))
    ref = O.new_bf16_pages(n_pool, H)
    O.bf16_pages_write(ref, k, v, np.zeros(L, int), np.arange(L), table)
    pages = torch.zeros((n_pool, H, O.BF16_BLOCK), dtype=torch.bfloat16)
    as_t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    fill_bf16_pages_device(pages, as_t(k), as_t(v), torch.from_numpy(table[0]))
    assert np.array_equal(pages.view(torch.int16).numpy().view(np.uint16), ref)
