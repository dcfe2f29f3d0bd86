"""GPU tests of the matrix-unit ceiling probe (``pts_mfma_ceiling``): with
fragments of known constant values every accumulator has a closed form, so
the probe is checked to run the MFMAs it claims (32 per wave and step, the
fragment set alternating by step parity, each wave on its own fragments)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LANES, WAVES, FRAGS = 64, 8, 24


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _fragments(value_of_wave_and_set):
    """Fragment f of wave w (8 bf16 per lane): set 0 is f < 12, set 1 the rest."""
    vals = np.zeros((WAVES, FRAGS, LANES, 8), dtype=np.float32)
    for w in range(WAVES):
        for f in range(FRAGS):
            vals[w, f] = value_of_wave_and_set(w, f // 12)
    t = torch.from_numpy(vals.reshape(-1)).to(torch.bfloat16)
    return t.cuda()


def _run(pts, frags, blocks, steps):
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda")
    pts.pts_mfma_ceiling(frags, out, stamps, blocks, steps)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(blocks, WAVES, LANES), stamps.cpu().numpy().reshape(blocks, 2)


def test_fragment_bytes_match_the_layout(pts):
    assert pts.PTS_MFMA_CEILING_FRAG_BYTES == WAVES * FRAGS * LANES * 16


def test_ones_give_the_closed_form(pts):
    # Every MFMA adds 32 (one 32-deep dot product of ones) to each of a lane's
    # 4 accumulators of a block; a lane holds 8 x 4 blocks: 128 x 32 x steps.
    frags = _fragments(lambda w, h: 1.0)
    steps = 6
    out, stamps = _run(pts, frags, 4, steps)
    np.testing.assert_array_equal(out, np.full_like(out, 128 * 32 * steps))
    assert (stamps[:, 0] > 0).all() and (stamps[:, 1] > 0).all()


def test_sets_alternate_and_waves_use_their_own_fragments(pts):
    # Wave w's set 0 holds w + 1 and its set 1 holds 2 (w + 1): a pair of steps
    # adds 32 (w + 1)^2 + 32 * 4 (w + 1)^2 = 160 (w + 1)^2 to each accumulator.
    frags = _fragments(lambda w, h: float((w + 1) * (1 + h)))
    steps = 4
    out, _ = _run(pts, frags, 3, steps)
    want = np.array([128 * 160 * (w + 1) ** 2 * (steps // 2) for w in range(WAVES)], dtype=np.float32)
    np.testing.assert_array_equal(out, np.broadcast_to(want[None, :, None], out.shape))


def test_one_block_per_compute_unit_by_default(pts):
    frags = _fragments(lambda w, h: 1.0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.full((cus * 512,), float("nan"), dtype=torch.float32, device="cuda")
    stamps = torch.zeros(cus * 2, dtype=torch.int64, device="cuda")
    pts.pts_mfma_ceiling(frags, out, stamps, 0, 2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), np.full(cus * 512, 128 * 32 * 2, dtype=np.float32))
