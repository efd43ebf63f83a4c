"""GPU parity of whole optimizer steps at the workloads' real batch shapes
(GPT-2 124M, bf16):
  * B=16, T=1024, vocabulary padded to 50304 (the benchmark workload);
  * the unpadded vocabulary 50257 (ragged classifier tiles) with backward,
    B=4, T=1024;
  * the accumulated step's micro-batch shape B=32, T=512 with two real
    micro-steps at lr(132), and the full 32-micro-step accumulation against
    the sum of the micro-steps' gradients;
  * sampling with the key/value cache at the 124M shape (4 sequences, a
    64-token prefix, 64 new tokens);
  * the whole step in fp32 throughout (fp32 matrix-core GEMMs), B=4, T=1024;
  * the whole step with fp16 operands and dynamic loss scaling, B=4, T=1024.
The oracle takes each batch as one-sequence micro-batches (exactly the same
step by linearity of accumulation, pinned on the CPU), so it never holds a
whole batch's logits.  Each test stays well under pytest's 900 s limit on the
GPU host; they are collected after the small-configuration tests."""
import pytest

from tests import parity_cases as cases
from tests.gpu_helpers import GPU

pytestmark = pytest.mark.gpu


def test_full_step_B16_T1024_padded_vocab():
    cases.full_step_vs_oracle(GPU, cases.G124, 16, 1024)


def test_full_step_unpadded_vocab_with_backward():
    cases.full_step_vs_oracle(GPU, cases.G124U, 4, 1024)


def test_accumulated_step_B32_T512_two_micro_steps():
    cases.accumulated_step_vs_oracle(GPU, B=32, T=512, micro=2)


def test_accumulation_of_32_micro_steps_equals_their_sum():
    cases.accumulation_equals_sum_of_micro_steps(GPU, B=32, T=512, micro=32)


def test_generate_124m_with_kv_cache():
    cases.generate_matches_oracle(GPU, "124m", B=4, T0=64, T=128)


def test_full_step_fp32_124m():
    cases.full_step_fp32_vs_oracle(GPU, 4, 1024)


def test_full_step_fp16_124m():
    cases.full_step_vs_oracle(GPU, cases.G124, 4, 1024, compute="fp16")
