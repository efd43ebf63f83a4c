"""The GPT-2 124M parity cases on the CPU emulation of the library, at the
model's full width (C=768, 12 heads, vocabulary 50304 or 50257) with fewer
layers and tokens than the GPU tests use, so that the classifier, the
cross-entropy rows of 50304 / 50257 logits and the weight-gradient plans of
the 124M matrices run their own code paths on the CPU.

Two cases run by default; the rest take one to three minutes each and run
when the environment sets EMU_124M=1."""
import os

import pytest

from tests import parity_cases as cases
from tests.gpu_helpers import emu_backend

EMU = emu_backend()
slow = pytest.mark.skipif(os.environ.get("EMU_124M") != "1",
                          reason="long CPU emulation; set EMU_124M=1 to run")


def test_emu_full_step_unpadded_vocab_with_backward():
    cases.full_step_vs_oracle(EMU, cases.G124U, 2, 64, n_layer=2)


def test_emu_block_124m():
    cases.block_124m(EMU, 1, 256)


@slow
def test_emu_full_step_padded_vocab():
    cases.full_step_vs_oracle(EMU, cases.G124, 2, 64, n_layer=2)


@slow
def test_emu_accumulated_step_two_micro_steps():
    cases.accumulated_step_vs_oracle(EMU, B=2, T=32, micro=2, n_layer=2)


@slow
def test_emu_accumulation_equals_sum_of_micro_steps():
    cases.accumulation_equals_sum_of_micro_steps(EMU, B=2, T=32, micro=4, n_layer=2)


@slow
def test_emu_unpadded_vocabulary_and_padding_effect():
    cases.unpadded_vocabulary_and_padding_effect(EMU, 64, n_layer=2)


@slow
def test_emu_full_batch_rows_and_determinism():
    cases.full_batch_rows_and_determinism(EMU, 2, 64, n_layer=2)


@slow
def test_emu_step_124m_one_sequence_all_layers():
    cases.step_124m_one_sequence(EMU, 64)


@slow
def test_emu_generate_124m_width():
    cases.generate_matches_oracle(EMU, "124m", B=2, T0=8, T=14, n_layer=2)


@slow
def test_emu_full_step_fp32_124m_width():
    cases.full_step_fp32_vs_oracle(EMU, 2, 64, n_layer=2)


@slow
def test_emu_full_step_fp16_124m_width():
    cases.full_step_vs_oracle(EMU, cases.G124, 2, 64, n_layer=2, compute="fp16")
