"""GPU parity of kda_short_conv (masked depthwise causal conv with cache) against the oracle."""
import numpy as np
import pytest

from linear_attention_recurrence_kda_amd import datagen as D
from tests.gpu_util import check, device, host, say, to_dev

pytestmark = pytest.mark.gpu


def _mask(kind, B, T, seed):
    rng = np.random.default_rng(seed)
    if kind == "none":
        return None
    if kind == "random":
        return (rng.uniform(size=(B, T)) < 0.7).astype(np.uint8)
    lengths = rng.integers(0, T + 1, B)
    return D.padded_layout(lengths, T, ["left" if b % 2 == 0 else "right" for b in range(B)])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [2, 3, 4])
@pytest.mark.parametrize("T", [1, 5, 32, 33, 77])
@pytest.mark.parametrize("kind", ["none", "pad", "random"])
def test_conv_matches_oracle(oracle, dtype, W, T, kind):
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, Dm = 3, 264
    say(f"[case] conv {dtype} W={W} T={T} mask={kind}")
    x = D.np_raw_x(B, T, Dm, dtype, 1, D.TID_XQ)
    w = D.np_conv_weight(Dm, W, 2)
    bias = np.linspace(-0.3, 0.3, Dm).astype(np.float32) if W == 3 else None
    cache = D.np_conv_cache(B, W, Dm, dtype, 3)
    mask = _mask(kind, B, T, 4)
    silu = (W == 2)
    xd, cd = to_dev(x, dtype, dev), to_dev(cache, dtype, dev)
    y = kda.short_conv(xd, to_dev(w, dev=dev), None if bias is None else to_dev(bias, dev=dev),
                       None if mask is None else to_dev(mask, dev=dev), cd, silu=silu)
    ry, rc = oracle.c_short_conv(x, w, bias, mask, cache, silu)
    check("conv y", host(y), ry, dtype)
    # the cache holds stored inputs: exact copies
    assert np.array_equal(host(cd), rc), "conv cache"


def test_conv_without_cache_and_full_continuation_shape(oracle):
    """The cached-continuation workload's conv: 8 sequences x 512 positions, D = 32*128,
    left/right padding, cache in place."""
    from linear_attention_recurrence_kda_amd import kda
    dev = device()
    B, T, Dm = 8, 512, 4096
    say("[case] conv continuation shape 8x512x4096")
    _, cont, sides = D.continuation_lengths(B)
    mask = D.padded_layout(cont, T, sides)
    x = D.np_raw_x(B, T, Dm, "bf16", 5, D.TID_XK) * mask[:, :, None]
    w = D.np_conv_weight(Dm, 4, 6)
    cache = D.np_conv_cache(B, 4, Dm, "bf16", 7)
    cd = to_dev(cache, "bf16", dev)
    y = kda.short_conv(to_dev(x, "bf16", dev), to_dev(w, dev=dev), None, to_dev(mask, dev=dev), cd)
    ry, rc = oracle.c_short_conv(x, w, None, mask, cache)
    check("conv cont y", host(y), ry, "bf16")
    assert np.array_equal(host(cd), rc)
    y0 = kda.short_conv(to_dev(x, "bf16", dev), to_dev(w, dev=dev), None, to_dev(mask, dev=dev), None)
    ry0, _ = oracle.c_short_conv(x, w, None, mask, None)
    check("conv no-cache y", host(y0), ry0, "bf16")
