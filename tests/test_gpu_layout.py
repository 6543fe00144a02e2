"""GPU parity of the KV append in global order (velox_kv_append) against the
oracle: the moved rows are byte work and must match exactly (every cache row,
written or not); the refreshed key means match the float64 oracle to 1e-5
relative and the other key means stay untouched."""

import numpy as np
import pytest
import torch

import geometry_routed_block_amd as velox
from oracle import layout
from gpu_common import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(H, T, Hl, Wl, d, dtype, chunk, hist_blocks, seed, with_kbar=True):
    say(f"kv_append H={H} T={T} grid={Hl}x{Wl} d={d} {dtype} chunk={chunk} hist={hist_blocks}")
    g = torch.Generator().manual_seed(seed)
    n = T * Hl * Wl
    nb = n // 128
    cap = (hist_blocks + nb + 1) * 128
    k_new = torch.randn(H, n, d, generator=g).to(dtype)
    v_new = torch.randn(H, n, d, generator=g).to(dtype)
    k_cache = torch.randn(H, cap, d, generator=g).to(dtype)
    v_cache = torch.randn(H, cap, d, generator=g).to(dtype)
    kbar = torch.full((H, cap // 128, d), 5.0)
    off = hist_blocks * 128
    cells = torch.from_numpy(velox.gilbert_curve(Wl, Hl)).to(DEV)
    kc_d, vc_d, kb_d = k_cache.to(DEV), v_cache.to(DEV), kbar.to(DEV)
    velox.kv_append(k_new.to(DEV), v_new.to(DEV), T, Hl, Wl, chunk, cells, kc_d, vc_d, off,
                    kbar=kb_d if with_kbar else None)
    torch.cuda.synchronize()
    # oracle on float32 copies (bf16 widens exactly, so equal values = equal bits
    # for these finite, nonzero draws); key means in float64
    kc_ref, vc_ref = k_cache.float().numpy().copy(), v_cache.float().numpy().copy()
    kb_ref = np.full((H, cap // 128, d), 5.0)
    layout.kv_append(kc_ref, vc_ref, kb_ref, k_new.float().numpy(), v_new.float().numpy(), T, Hl,
                     Wl, chunk, off, hist_blocks)
    assert np.array_equal(kc_d.cpu().float().numpy(), kc_ref)
    assert np.array_equal(vc_d.cpu().float().numpy(), vc_ref)
    got_kb = kb_d.cpu().numpy()
    if with_kbar:
        np.testing.assert_allclose(got_kb, kb_ref, rtol=1e-5, atol=1e-6)
    else:
        assert (got_kb == 5.0).all()


@pytest.mark.parametrize("chunk", [0, 1])
def test_append_chunk48_shape_bf16(chunk):
    # 3 latent frames of 32 x 48 tokens = 36 blocks, after 5 chunks of history
    _case(4, 3, 32, 48, 128, torch.bfloat16, chunk, hist_blocks=5 * 36, seed=chunk)


def test_append_fp32_d64_small_odd_grid():
    _case(2, 2, 8, 24, 64, torch.float32, 7, hist_blocks=3, seed=3)   # 384 tokens = 3 blocks


def test_append_single_frame_without_key_means():
    _case(3, 1, 16, 16, 128, torch.bfloat16, 2, hist_blocks=0, seed=4, with_kbar=False)


def test_append_then_route_scores_uses_fresh_means():
    # the appended chunk's key means equal velox_block_mean over the same rows
    H, T, Hl, Wl, d = 2, 3, 32, 48, 128
    n = T * Hl * Wl
    g = torch.Generator().manual_seed(9)
    k_new = torch.randn(H, n, d, generator=g).to(torch.bfloat16).to(DEV)
    v_new = torch.randn(H, n, d, generator=g).to(torch.bfloat16).to(DEV)
    kc = torch.zeros(H, n + 256, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kb = torch.zeros(H, (n + 256) // 128, d, device=DEV)
    cells = torch.from_numpy(velox.gilbert_curve(Wl, Hl)).to(DEV)
    say("kv_append vs block_mean")
    velox.kv_append(k_new, v_new, T, Hl, Wl, 1, cells, kc, vc, 256, kbar=kb)
    ref = velox.block_mean(kc[:, 256:])
    torch.cuda.synchronize()
    torch.testing.assert_close(kb[:, 2:], ref, rtol=1e-6, atol=1e-6)
