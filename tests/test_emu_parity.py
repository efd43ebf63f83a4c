"""The parity cases of the GPU suite, run on the CPU emulation of the HIP
library (the unchanged kernel and engine sources compiled for the host, see
tests/emu).  This checks the kernels' index arithmetic, tiling, ragged tails,
split-K plans and launch logic against the oracle without a GPU; it does not
replace the GPU runs (hardware timing, memory ordering and the instruction
semantics the emulator assumes are checked only there).

Two emulator settings are exercised on the bf16 path: the buffer range check
with and without the scalar offset, and a reversed fiber schedule; results
must not depend on either."""
import numpy as np
import pytest

from tests import parity_cases as cases
from tests.gpu_helpers import emu_backend, gpu_grads, gpu_params, configs, stream_for
from decoder_only_transformer_02_amd import inputs

EMU = emu_backend()


@pytest.fixture
def emu_mode():
    from tests.emu.binding import emu_lib
    L = emu_lib()
    yield L
    L.emu_set_range_mode(0)
    L.emu_set_reverse_order(0)
    L.emu_set_land_early(0)


def test_emu_tiny_fp32_step():
    cases.tiny_fp32_step(EMU)


def test_emu_fp32_ragged_shapes():
    cases.fp32_ragged_shapes(EMU)


def _bf16_step_outputs():
    lc, oc, p = configs(cases.SMALL_BF16, 3, 100)
    x, y = inputs.batch_from_stream(stream_for(p, 301, 2), 3, 100)
    m = EMU.make(lc, 1)
    loss = m.forward(EMU.dev(x), EMU.dev(y))
    m.backward(1.0)
    norm = m.step(6e-4)
    names = m.param_names()
    out = (loss, norm, gpu_grads(m, names), gpu_params(m, names))
    m.close()
    return out


@pytest.mark.parametrize("range_mode", [0, 1])
def test_emu_bf16_ragged_mfma_paths(emu_mode, range_mode):
    """Parity of the ragged bf16 path whether or not the buffer range check
    covers the scalar offset (mode 1 reads garbage past a buffer's end when
    only the scalar offset puts an access there)."""
    emu_mode.emu_set_range_mode(range_mode)
    cases.bf16_ragged_mfma_paths(EMU)


def test_emu_results_independent_of_range_mode_and_schedule(emu_mode):
    """Bitwise the same step with the range check including the scalar
    offset or not, with the fibers of every block scheduled in reverse
    order, and with buffer-to-LDS writes landing at issue instead of at
    their wait (an LDS race, a missing wait or a ring slot refilled while
    still being read would show as a difference)."""
    base = _bf16_step_outputs()
    emu_mode.emu_set_range_mode(1)
    alt = _bf16_step_outputs()
    emu_mode.emu_set_range_mode(0)
    emu_mode.emu_set_reverse_order(1)
    rev = _bf16_step_outputs()
    emu_mode.emu_set_reverse_order(0)
    emu_mode.emu_set_land_early(1)
    early = _bf16_step_outputs()
    for other in (alt, rev, early):
        assert other[0] == base[0] and other[1] == base[1]
        for n in base[2]:
            assert np.array_equal(other[2][n], base[2][n]), n
            assert np.array_equal(other[3][n], base[3][n]), n


def test_emu_bf16_accumulation_matches_one_big_batch():
    cases.bf16_accumulation_matches_one_big_batch(EMU)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_emu_causality_bitwise(preset):
    cases.causality_bitwise(EMU, preset)


def test_emu_determinism_bitwise():
    cases.determinism_bitwise(EMU)


def test_emu_device_init_equals_host_init():
    cases.device_init_equals_host_init(EMU)


def test_emu_error_paths():
    cases.error_paths(EMU)


def test_emu_overfit_single_batch_tracks_oracle():
    cases.overfit_single_batch_tracks_oracle(EMU, steps=12)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_emu_checkpoint_resume_bitwise(preset):
    cases.checkpoint_resume_bitwise(EMU, preset)


@pytest.mark.parametrize("preset", ["bf16", "fp16"])
def test_emu_weight_copies_follow_weights(preset):
    cases.weight_copies_follow_weights(EMU, preset)


def test_emu_arena_guard_detects_overrun():
    cases.arena_guard_detects_overrun(EMU)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_emu_eval_loss_forward_only(preset):
    cases.eval_loss_forward_only(EMU, preset)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_emu_generate_matches_oracle(preset):
    cases.generate_matches_oracle(EMU, preset)


def test_emu_fp16_ragged_step():
    cases.fp16_ragged_step(EMU)


def test_emu_fp16_loss_scaler():
    cases.fp16_loss_scaler(EMU)
