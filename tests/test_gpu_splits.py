"""GPU parity of the KV-split attention (a work unit's CSR list cut into
contiguous shares balanced by count, partial results merged through their
LSE) against the fp64 oracle, through the C ABI.

Bar: as the unsplit path (selections bit-exact outside the band, outputs
<= 2e-2 for bf16 / fp8 against the oracle, whose fp8 arithmetic walks the
same splits); a bf16 split result also agrees with the unsplit one to within 2e-2 or one bf16 spacing of the value, whichever is
larger: two float32 results on either side of a rounding midpoint round to
neighbouring bf16 outputs, 2^-5 apart at |O| in [4, 8)."""
import numpy as np
import pytest

from harness import (assert_parity, compare, log, make_inputs, run_gpu, sample_tiles,
                     to_device)
from workloads import SHARD_BF16_16K, Workload

pytestmark = pytest.mark.gpu


def runs_agree(a, b, tol=2e-2):
    """Element-wise |a - b| <= max(tol, bf16 spacing at max(|a|, |b|))."""
    m = np.maximum(np.abs(a), np.abs(b)).astype(np.float32)
    lim = np.maximum(tol, np.spacing(m) * 65536.0)  # float32 spacing x 2^16 = bf16 spacing
    return bool((np.abs(a.astype(np.float64) - b.astype(np.float64)) <= lim).all())


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_pooled_amd as bslp
    bslp.load_library()


# A segment uses one split per 24 steps of work (64-key halves of its selected
# blocks plus its correction chunks), so these shapes select densely enough for
# the heavy tiles to split several ways.
SPLIT_SHAPES = [
    Workload("split-bf16-dense-g4", (6000,), 8, 2, 128, 128, "bf16", alpha=0.0, attractors=4),
    Workload("split-fp8-g8", (4000, 3000), 16, 2, 128, 128, "fp8", alpha=0.0, sigma_c=1.5),
    Workload("split-paged-varlen-bf16", (3000, 5000, 77), 8, 4, 128, 128, "bf16", alpha=0.0,
             page_size=64, attractors=4),
    Workload("split-varlen-b64", (3000, 1500), 8, 2, 128, 64, "bf16", alpha=0.0, attractors=4),
]


@pytest.mark.parametrize("splits", [2, 4, 16])
@pytest.mark.parametrize("w", SPLIT_SHAPES, ids=lambda w: w.name)
def test_forced_splits_match_oracle(w, splits):
    inp = make_inputs(w, 11)
    dev = to_device(inp)
    whole = run_gpu(w, inp, correction=True, dev_tensors=dev, kv_splits=1)
    for corr in (True, False):
        g = run_gpu(w, inp, correction=corr, dev_tensors=dev, kv_splits=splits)
        rep = compare(w, inp, g, correction=corr)
        log(f"[split] {w.name} splits={splits} corr={corr}: {rep}")
        assert_parity(w, rep)
    # the heavy segments did split: their rounding differs from the whole walk
    g = run_gpu(w, inp, correction=True, dev_tensors=dev, kv_splits=splits)
    assert not np.array_equal(g.out, whole.out)
    if w.dtype != "fp8":  # fp8 splits round P~ against their own maxima (oracle above)
        assert runs_agree(g.out, whole.out)


@pytest.mark.parametrize("alpha", [0.05, 0.0])
def test_automatic_split_on_a_head_shard(alpha):
    # few work units: the library allows splits, which the heavy tiles of the
    # alpha = 0 selection use (at 0.05 most segments are light and stay whole)
    w = SHARD_BF16_16K.replace(alpha=alpha)
    inp = make_inputs(w, 0)
    dev = to_device(inp)
    auto = run_gpu(w, inp, dev_tensors=dev)
    off = run_gpu(w, inp, dev_tensors=dev, kv_splits=1)
    rep = compare(w, inp, auto, tiles=sample_tiles(w, per_head=6) if alpha == 0 else None)
    log(f"[split] {w.name} auto: {rep}")
    assert_parity(w, rep)
    diff = float(np.abs(auto.out - off.out).max())
    ldiff = float(np.abs(auto.lse - off.lse).max())
    log(f"[split] {w.name} auto vs none: out {diff:.3e} lse {ldiff:.3e}")
    assert runs_agree(auto.out, off.out) and ldiff <= 1e-4
    assert np.array_equal(auto.idx, off.idx)
