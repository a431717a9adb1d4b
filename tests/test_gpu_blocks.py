"""GPU parity of the block copies of the split caches: rpa_copy_blocks
(device, every layer) and rpa_swap_blocks (device <-> pinned host, device ->
device) through the C ABI against the oracle, bit-exact; blocks not named as
destinations keep their bytes."""
import numpy as np
import pytest
import torch

import ragged_paged_kv_scatter_amd as rpa
from oracle import rpa_oracle as O

pytestmark = pytest.mark.gpu


def _pairs(rng, num_blocks, n):
    perm = rng.permutation(num_blocks)
    return np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int64)   # dsts not sources


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


def test_copy_blocks_every_layer():
    print("\n[case] copy_blocks 3 layers", flush=True)
    rng = np.random.default_rng(11)
    g = torch.Generator().manual_seed(11)
    shape = (64, 16, 8, 128)
    ks = [torch.randn(shape, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    vs = [torch.randn(shape, generator=g).to(torch.bfloat16).cuda() for _ in range(3)]
    pairs = _pairs(rng, shape[0], 20)
    ref_k = O.copy_blocks([_bits(k) for k in ks], pairs)
    ref_v = O.copy_blocks([_bits(v) for v in vs], pairs)
    rpa.rpa_copy_blocks(ks, vs, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    for got, ref in zip(ks + vs, ref_k + ref_v):
        np.testing.assert_array_equal(_bits(got), ref)


@pytest.mark.parametrize("direction", ["d2h", "h2d", "d2d"])
def test_swap_blocks(direction):
    print(f"\n[case] swap_blocks {direction}", flush=True)
    rng = np.random.default_rng(12)
    g = torch.Generator().manual_seed(12)
    src = torch.randn((32, 16, 8, 64), generator=g).to(torch.bfloat16)
    dst = torch.randn((48, 16, 8, 64), generator=g).to(torch.bfloat16)
    src_on = src.cuda() if direction in ("d2h", "d2d") else src.pin_memory()
    dst_on = dst.cuda() if direction in ("h2d", "d2d") else dst.pin_memory()
    perm_s, perm_d = rng.permutation(32), rng.permutation(48)
    pairs = np.stack([perm_s[:12], perm_d[:12]], axis=1).astype(np.int64)
    ref = O.swap_blocks(_bits(src), _bits(dst), pairs)
    rpa.rpa_swap_blocks(src_on, dst_on, torch.from_numpy(pairs))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(dst_on), ref)
