"""The QKV projection with its fused epilogue (fp_qkv_project) against the float64 oracle, and
fp_index_pooled (the index stage fed the projection's pooled queries) against the oracle index.

bf16 outputs: the device rounds an fp32 accumulator, the oracle a float64 product, so a value may
differ by one bf16 spacing where the product lies near a rounding boundary (plus 1e-5 for fp32
error on values near zero, where the rotation cancels); at most 1% of values may differ at all.
Block means: within 1e-5 of the float64 mean of the device's own rounded values, and as close to
the oracle's as the block's bf16 differences allow (their mean, plus 1e-5).  int8 codes and scales:
equal to the oracle quantiser applied to the device's own rounded values, and within one code of
the oracle's codes."""
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_flexprefill_amd as fpa
import gen
from oracle import index as oi
from oracle import project as op
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fpa.lib()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16_dev(u16):
    return P.dev_bf16(u16)


def _check_bf16(got: torch.Tensor, want: np.ndarray, name: str):
    """At most one bf16 spacing apart (of the larger of the two values, so a step across a power of
    two counts once), plus 1e-5 for the fp32 accumulation and rotation on values near zero."""
    g = got.float().cpu().numpy().astype(np.float64)
    big = np.maximum(np.maximum(np.abs(want), np.abs(g)), 2.0 ** -126)
    spacing = 2.0 ** (np.floor(np.log2(big)) - 7)
    off = np.abs(g - want)
    assert np.all(off <= spacing + 1e-5), (name, float((off - spacing).max()))
    frac = float(np.mean(off > 0))
    say(f"  {name}: {100 * frac:.3f}% of values one bf16 unit off")
    assert frac <= 0.01, (name, frac)
    return g


CASES = [("small-b128-rope-i8", 1024, 256, 4, 2, 128, True, True),
         ("small-b64-norope", 1024, 256, 4, 2, 64, False, True),
         ("3b-dims-b128", 4096, 3072, 6, 2, 128, True, True),
         # an odd number of 64-wide k-steps, 9 token tiles (not a multiple of 8) and 5 column tiles
         # (a partial band of heads): the other branches of the tile order and of the load pipeline
         ("odd-ksteps-ragged-tiles", 1152, 320, 3, 1, 128, True, True)]


@pytest.mark.parametrize("name,S,D,Hq,Hkv,b,rot,i8", CASES, ids=[c[0] for c in CASES])
def test_qkv_project_matches_oracle(name, S, D, Hq, Hkv, b, rot, i8):
    say(f"qkv_project {name}: S={S} D={D} Hq={Hq} Hkv={Hkv} b={b} rope={rot} int8={i8}")
    inp = gen.projection_inputs(S, D, Hq, Hkv, seed=5)
    X, W = _bf16_dev(inp["x"]), _bf16_dev(inp["w"])
    cos = P.dev(inp["cos"]) if rot else None
    sin = P.dev(inp["sin"]) if rot else None
    out = fpa.qkv_project(X, W, Hq, Hkv, b, rope_cos=cos, rope_sin=sin, int8=i8)
    torch.cuda.synchronize()
    ref = op.project(gen.f32_from_bf16_bits(inp["x"]), gen.f32_from_bf16_bits(inp["w"]), Hq, Hkv, b,
                     cos=inp["cos"] if rot else None, sin=inp["sin"] if rot else None)
    for name_ in ("q", "k", "v"):
        g = _check_bf16(out[name_], ref[name_], name_)
        if name_ in ("q", "k"):
            bar = out[name_ + "bar"].cpu().numpy().astype(np.float64)
            own = g.reshape(g.shape[0], S // b, b, 128).mean(axis=2)
            np.testing.assert_allclose(bar, own, rtol=0, atol=1e-5)
            # against the oracle: the block's own bf16 differences, averaged, bound the mean's
            dev_off = np.abs(g - ref[name_]).reshape(g.shape[0], S // b, b, 128).mean(axis=2)
            assert np.all(np.abs(bar - ref[name_ + "bar"]) <= dev_off + 1e-5)
        if i8:
            c8, s8 = out[name_ + "8"].cpu().numpy(), out["s" + name_].cpu().numpy()
            wc, ws = op.quantize(g.astype(np.float32))
            np.testing.assert_array_equal(c8, wc)
            np.testing.assert_array_equal(s8, ws)
            assert np.abs(c8.astype(np.int32) - ref[name_ + "8"].astype(np.int32)).max() <= 1


def test_index_pooled_from_projection():
    """The index stage fed the projection's pooled queries: same result as fp_index on the projected Q, K
    (up to the selection-boundary rule) and as the oracle on them."""
    S, D, Hq, Hkv, b = 4096, 512, 6, 2, 128
    say(f"index_pooled from the projection: S={S} D={D} Hq={Hq} Hkv={Hkv}")
    inp = gen.projection_inputs(S, D, Hq, Hkv, seed=6)
    out = fpa.qkv_project(_bf16_dev(inp["x"]), _bf16_dev(inp["w"]), Hq, Hkv, b, rope_cos=P.dev(inp["cos"]),
                          rope_sin=P.dev(inp["sin"]))
    for gamma, tau in ((0.9, 0.1), (0.9, 10.0)):      # tau = 10 labels every head query-aware
        idx = fpa.index_pooled(out["q"], out["k"], out["qbar"], b, gamma, tau, stats=True)
        plain = fpa.index(out["q"], out["k"], b, gamma, tau, stats=True)
        torch.cuda.synchronize()
        assert int(idx.status.item()) == 0
        Q = out["q"].float().cpu().numpy()
        K = out["k"].float().cpu().numpy()
        ref = oi.index(Q, K, b, gamma, tau)
        s = P.compare_index(idx, ref, gamma, tau)
        P.check_jobs(idx, Hq // Hkv)
        same = torch.equal(idx.row_ptr, plain.row_ptr) and torch.equal(idx.col_idx[:idx.nnz], plain.col_idx[:plain.nnz])
        say(f"  tau={tau}: {s}; patterns {idx.pattern.cpu().numpy().tolist()}; rows identical to fp_index: {same}")
