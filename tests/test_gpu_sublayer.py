"""GPU parity of the synthetic-weight attention sub-layer (qkv projection, split, QK-Norm + RoPE + store, paged
attention, output projection) against the float64 oracle composition: a varlen prefill step, then decode steps
over the same caches (one row padded).

Tolerance: the GPU path rounds to bf16 five times on the way (qkv, the normalised and rotated q and k, the
attention output, y), each a relative 2^-9; the scores are dot products of 128 such values and move the
softmax weights by about |s| times their relative error.  With unit-size activations this bounds the output
error near 1e-2 of the output's scale, so the test takes max-abs error <= 1e-2 * max(1, max |y|) -- measured:
1.1e-2 and 1.3e-2 on prefill outputs up to 3.8, 4e-3 to 8e-3 on decode outputs up to 1.9."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import log, nan_cache, to_host
from oracle.sublayer import sublayer_step_ref

pytestmark = pytest.mark.gpu

HIDDEN, HQ, HKV, HD = 1024, 16, 8, 128


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


class _Cache:
    def __init__(self, num_blocks, block_size):
        self.dtype, self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim = \
            "bf16", num_blocks, block_size, HKV, HD


def _f64(t):
    return oracle.as_f64(to_host(t), "bf16")


def _check(name, got, want):
    got = _f64(got)
    err = float(np.max(np.abs(got - want)))
    tol = 1e-2 * max(1.0, float(np.max(np.abs(want))))
    log(f"  {name}: max-abs {err:.3e}, max |y| {float(np.max(np.abs(want))):.2f}, tol {tol:.2e}")
    assert np.all(np.isfinite(got)) and err <= tol


@pytest.mark.parametrize("block_size,lens,seed", [(16, [37, 130, 64], 301), (256, [300, 5, 1000, 64], 302)])
def test_prefill_then_decode(pkv, block_size, lens, seed):
    sub = pkv.AttentionSublayer(hidden_size=HIDDEN, num_q_heads=HQ, num_kv_heads=HKV, head_dim=HD, seed=seed)
    w = (_f64(sub.w_qkv), _f64(sub.q_norm_weight), _f64(sub.k_norm_weight), _f64(sub.w_o))
    rng = np.random.default_rng(seed)
    steps = 2
    batch = len(lens) + 1                    # the last decode row is padding (context 0)
    need = [math.ceil((L + steps) / block_size) for L in lens]
    num_blocks = sum(need) + 2
    max_blocks = max(need)
    perm = rng.permutation(num_blocks)
    bt = np.full((batch, max_blocks), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    kc, vc = nan_cache(_Cache(num_blocks, block_size)), nan_cache(_Cache(num_blocks, block_size))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)

    # Prefill of every real sequence's prompt.
    n = sum(lens)
    x = torch.randn(n, HIDDEN, generator=gen, device="cuda").to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    positions = torch.tensor(np.concatenate([np.arange(L) for L in lens]), dtype=torch.int32, device="cuda")
    bt_real = torch.from_numpy(bt[:len(lens)]).cuda()
    y = sub.prefill(x, positions, cu, cu, max(lens), max(lens), bt_real, kc, vc)
    torch.cuda.synchronize()
    xs = _f64(x)
    hist = []
    want = []
    off = 0
    empty = np.zeros((0, HKV, HD))
    for L in lens:
        y_ref, hk, hv = sublayer_step_ref(xs[off:off + L], np.arange(L), empty, empty, *w, HQ, HKV, HD, sub.eps,
                                          sub.theta, sub.scale)
        want.append(y_ref)
        hist.append((hk, hv))
        off += L
    log(f"sub-layer prefill: lens {lens}, block_size {block_size}")
    _check("prefill", y, np.concatenate(want))

    # Decode steps: one new token per real row, plus a padding row.
    bt_dev = torch.from_numpy(bt).cuda()
    for s in range(steps):
        xd = torch.randn(batch, HIDDEN, generator=gen, device="cuda").to(torch.bfloat16)
        ctx = torch.tensor([L + s + 1 for L in lens] + [0], dtype=torch.int32, device="cuda")
        yd = sub.decode(xd, ctx, bt_dev, kc, vc)
        torch.cuda.synchronize()
        xds = _f64(xd)
        want = []
        for b, L in enumerate(lens):
            y_ref, hk, hv = sublayer_step_ref(xds[b:b + 1], [L + s], hist[b][0], hist[b][1], *w, HQ, HKV, HD, sub.eps,
                                              sub.theta, sub.scale)
            hist[b] = (hk, hv)
            want.append(y_ref)
        _check(f"decode step {s}", yd[:len(lens)], np.concatenate(want))
        assert bool((yd[len(lens)] == 0).all()), "the padding row's output is the projection of zeros"
