"""GPU parity of the HIP training step (through the C ABI) against the CPU
oracle on identical seeded inputs, at small configurations that span several
tiles and ragged tails.  The case bodies are in tests/parity_cases.py; the
same cases run on the CPU emulation of the library in tests/test_emu_parity.py.

Tolerances: the fp32 path within 1e-4 relative on the loss (and on every
gradient, relative L2) and 1e-3 max-abs on the post-AdamW parameters; the
bf16 path within 2e-2 relative on the loss, per-tensor gradient cosine
>= 0.999, and the post-AdamW rule of check_post_adamw (1e-3 where the two
gradients agree in sign)."""
import pytest

from tests import parity_cases as cases
from tests.gpu_helpers import GPU

pytestmark = pytest.mark.gpu


def test_tiny_fp32_step():
    cases.tiny_fp32_step(GPU)


def test_fp32_ragged_shapes():
    cases.fp32_ragged_shapes(GPU)


def test_bf16_ragged_mfma_paths():
    cases.bf16_ragged_mfma_paths(GPU)


def test_bf16_accumulation_matches_one_big_batch():
    cases.bf16_accumulation_matches_one_big_batch(GPU)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_causality_bitwise(preset):
    cases.causality_bitwise(GPU, preset)


def test_determinism_bitwise():
    cases.determinism_bitwise(GPU)


def test_device_init_equals_host_init():
    cases.device_init_equals_host_init(GPU)


def test_error_paths():
    cases.error_paths(GPU)


def test_overfit_single_batch_tracks_oracle():
    cases.overfit_single_batch_tracks_oracle(GPU)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_checkpoint_resume_bitwise(preset):
    cases.checkpoint_resume_bitwise(GPU, preset)


@pytest.mark.parametrize("preset", ["bf16", "fp16"])
def test_weight_copies_follow_weights(preset):
    cases.weight_copies_follow_weights(GPU, preset)


def test_arena_guard_detects_overrun():
    cases.arena_guard_detects_overrun(GPU)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_eval_loss_forward_only(preset):
    cases.eval_loss_forward_only(GPU, preset)


@pytest.mark.parametrize("preset", ["fp32", "bf16"])
def test_generate_matches_oracle(preset):
    cases.generate_matches_oracle(GPU, preset)


def test_fp16_ragged_step():
    cases.fp16_ragged_step(GPU)


def test_fp16_loss_scaler():
    cases.fp16_loss_scaler(GPU)
