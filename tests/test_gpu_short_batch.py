"""Batches of short sequences at d = 128 (no sequence longer than two 128-row
query tiles): the work list deals them pair by pair, a pair's query tiles
adjacent in one queue, instead of level by level.

The outputs are compared with the fp64 CPU oracle over the whole batch, for
the one-kernel (at most 256 sequences) and two-kernel forms, plain and
target-aware.  An item's arithmetic does not depend on the queue order or on
which workgroup runs it, so the same sequences computed in a batch that also
holds one longer sequence (which switches the work list to the level order)
must give the same bits.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_close, device_case, from_torch, log

torch = pytest.importorskip("torch")
hstu = pytest.importorskip("generative_recommendation_attention_amd")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

# Lengths around 32-key tiles and 128-row query tiles, and below three key
# tiles (fewer tiles than the kernel keeps in flight).
EDGE = [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 160, 191, 192, 255, 256, 0]


def short_lengths(count, seed):
    rng = np.random.default_rng(seed)
    lengths = EDGE + [int(x) for x in rng.integers(0, 257, size=max(0, count - len(EDGE)))]
    rng.shuffle(lengths)
    return lengths


def run(case, targets=None):
    q, k, v, off = device_case(case)
    if targets is None:
        res = hstu.hstu_attn_fwd(q, k, v, off, case.alpha, case.n)
    else:
        res = hstu.hstu_attn_fwd_targets(q, k, v, off, torch.from_numpy(targets).cuda(),
                                         case.alpha, case.n)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("count", [200, 700])
def test_short_batch_full_compare(dtype, count):
    lengths = short_lengths(count, seed=40 + count)
    case = workloads.make_case(lengths, 2, 128, dtype, seed=4100 + count,
                               sigma=0.5 if dtype == "fp16" else 1.0, n=256.0)
    log(f"short batch {dtype} {count} sequences T={case.total}")
    got = from_torch(run(case), dtype)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 2, 128, case.alpha, case.n, dtype)
    mr, l2 = assert_close(got, ref, dtype, f"short batch {dtype} {count}")
    log(f"  max|err|/max|ref| = {mr:.2e}, rel L2 = {l2:.2e}")


@pytest.mark.parametrize("count", [200, 700])
def test_short_batch_targets_full_compare(count):
    lengths = short_lengths(count, seed=50 + count)
    rng = np.random.default_rng(51 + count)
    tg = np.array([int(rng.integers(0, s + 2)) for s in lengths], np.int32)
    case = workloads.make_case(lengths, 2, 128, "bf16", seed=4200 + count, n=256.0)
    log(f"short batch targets {count} sequences T={case.total}")
    got = from_torch(run(case, tg), "bf16")
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 2, 128, case.alpha, case.n, "bf16",
                     num_targets=tg)
    assert_close(got, ref, "bf16", f"short batch targets {count}")


@pytest.mark.parametrize("count", [200, 700])
@pytest.mark.parametrize("with_targets", [False, True])
def test_short_batch_bitwise_equals_level_order(count, with_targets):
    """The short sequences alone, and the same sequences followed by one of
    300 tokens (three query tiles: the level order), give the same bits."""
    lengths = short_lengths(count, seed=60 + count)
    case = workloads.make_case(lengths, 3, 128, "bf16", seed=4300 + count, n=300.0)
    longer = workloads.make_case(lengths + [300], 3, 128, "bf16", seed=4300 + count, n=300.0)
    t = case.total
    # same leading rows in both batches
    longer.q[:t], longer.k[:t], longer.v[:t] = case.q, case.k, case.v
    tg = tg_long = None
    if with_targets:
        rng = np.random.default_rng(61 + count)
        tg = np.array([int(rng.integers(0, s + 1)) for s in lengths], np.int32)
        tg_long = np.concatenate([tg, np.array([7], np.int32)])
    a = run(case, tg)
    b = run(longer, tg_long)
    assert torch.equal(a.view(torch.int16), b[:t].view(torch.int16))
