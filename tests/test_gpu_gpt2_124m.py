"""GPU parity at the GPT-2 124M shapes: one block in isolation at its full
size (B=16, T=1024), the full step on one sequence against the whole oracle
step, the B=16 batch on sampled rows, and the unpadded vocabulary.  The
whole steps at the workloads' real batch shapes are in
test_gpu_workloads_full.py."""
import pytest

from tests import parity_cases as cases
from tests.gpu_helpers import GPU

pytestmark = pytest.mark.gpu


def test_block_124m_full_size():
    cases.block_124m(GPU, 16, 1024)


def test_gpt2_124m_step_one_sequence():
    cases.step_124m_one_sequence(GPU, 1024)


def test_gpt2_124m_full_batch_sampled_rows():
    cases.full_batch_rows_and_determinism(GPU, 16, 1024)


def test_unpadded_vocabulary_and_padding_effect():
    cases.unpadded_vocabulary_and_padding_effect(GPU, 1024)


def test_accumulated_step_two_micro_steps_one_sequence():
    """Gradient accumulation at T=512: two micro-steps of one sequence at
    loss scale 1/2, then clip and AdamW at lr(132) = 6e-4."""
    cases.accumulated_step_vs_oracle(GPU, B=1, T=512, micro=2)
