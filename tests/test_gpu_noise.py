"""GPU parity of the coordinated noise initialization (DualParal write-up,
section 三, second improvement) against the plain oracle: the chosen pool
indices must be identical (integer work, bit-exact) and the new chunk's noise
an exact copy of those pool frames."""
import numpy as np
import pytest
import torch

from oracle import noise as noise_sim
from chunked_spatio_temporal_amd import chunkattn as ca

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def keys_for(P, seed):
    k = np.random.default_rng(seed).integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
    return k, torch.from_numpy(k.view(np.int32)).to(DEV)


@pytest.mark.parametrize("P,F,E,frame_shape,dt", [
    (12, 8, 4, (16, 60, 104), torch.float32),    # Wan-class 480p latent frames
    (6, 4, 2, (16, 90, 160), torch.bfloat16),    # 720p latent frames, pool = F + E
    (300, 40, 20, (8, 4), torch.float32),         # many small frames
    (4096, 4000, 96, (4,), torch.float32),        # largest pool
    (5, 5, 0, (16,), torch.bfloat16),             # no exclusion: a shuffle of the pool
])
def test_noise_init_chain_matches_oracle(P, F, E, frame_shape, dt):
    pool = torch.randn((P,) + frame_shape, device=DEV).to(dt)
    prev_np, prev_t = None, None
    for chunk in range(4):
        k_np, k_t = keys_for(P, 1000 * P + chunk)
        out, idx = ca.noise_init(pool, k_t, F, prev_t, E if prev_t is not None else 0)
        torch.cuda.synchronize()
        exp_idx = noise_sim.select(P, k_np, F, prev_np, E if prev_np is not None else 0)
        assert idx.cpu().numpy().tolist() == exp_idx.tolist()
        assert torch.equal(out, pool[torch.from_numpy(exp_idx).to(DEV)])
        prev_np, prev_t = exp_idx, idx


def test_noise_init_ties_fall_back_to_pool_index():
    P, F = 64, 64
    pool = torch.arange(P * 4, dtype=torch.float32, device=DEV).view(P, 4)
    keys = torch.zeros(P, dtype=torch.int32, device=DEV)
    out, idx = ca.noise_init(pool, keys, F)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == list(range(P))
    assert torch.equal(out, pool)


def test_noise_init_keys_compare_unsigned():
    """Keys are 32-bit patterns compared as unsigned: 0x80000000 ranks after 1."""
    pool = torch.arange(3 * 4, dtype=torch.float32, device=DEV).view(3, 4)
    k = np.array([0x80000000, 1, 0xFFFFFFFF], np.uint32)
    keys = torch.from_numpy(k.view(np.int32)).to(DEV)
    _, idx = ca.noise_init(pool, keys, 3)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == noise_sim.select(3, k, 3).tolist() == [1, 0, 2]
