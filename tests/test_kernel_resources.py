"""The compiler's per-kernel resource report of the gfx950 build
(_build/kernel_resources.json, written by build()): no hot-path kernel
spills to scratch, no kernel exceeds the 160 KB of LDS per CU, and the
kernels whose speed depends on waves in flight keep their occupancy.  The
CPU emulation cannot see any of this; one rewrite of the cross-entropy had
gone from three waves per SIMD to one without any test noticing."""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT = os.path.join(ROOT, "_build", "kernel_resources.json")
CSRC = os.path.join(ROOT, "decoder_only_transformer_02_amd", "csrc")

# kernels on the training, evaluation and sampling paths (mangled-name parts)
HOT = ["k_gemm_nt", "k_gemm_tn", "k_gemm_f32m", "k_splitk_reduce", "k_attn_fwd64", "k_attn_dq64",
       "k_attn_dkv64", "k_xent", "k_loss_reduce", "k_ln_fwd", "k_ln_bwd", "k_ln_param_reduce", "k_colsum",
       "k_embed_fwd", "k_sort_runs", "k_merge_runs", "k_emb_seg", "k_dwpe", "k_sumsq", "k_norm_finalize",
       "k_adamw", "k_to_bf16", "k_to_f16", "k_kv_store", "k_attn_decode", "k_sample"]

# minimum waves per SIMD: (name part, floor, why)
FLOORS = [
    ("k_xentIDF16bLi25E", 3, "one row per block held in registers: needs rows in flight"),
    ("k_attn_fwd64", 3, "the softmax of one wave overlaps the MFMA of another"),
    ("k_attn_dq64", 3, "with its MFMA results in VGPRs (attention.hip's build option)"),
    ("k_attn_dkv64", 2, ""),
    ("k_ln_fwdIDF16bLi4E", 4, "its grid puts four waves on every SIMD"),
    ("k_ln_bwdIDF16bLi4E", 2, "its grid puts two waves on every SIMD"),
    ("k_ln_fwdIDF16bLi3ELb1E", 4, "the 768-wide variant of the 124M model"),
    ("k_ln_bwdIDF16bLi3ELb1E", 4, "the 768-wide variant: no column tests, unconditional prefetch, 128 registers"),
    ("k_gemm_ntIDF16bLi256ELi256E", 2, "two waves per SIMD at the 256x256 tile"),
    ("k_gemm_tnIDF16bLi256ELi256E", 2, ""),
    ("k_gemm_ntIDF16bLi256ELi192E", 1, ""),
    ("k_adamw", 8, ""),
    ("k_sumsq", 8, ""),
]


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(REPORT):
        pytest.skip("no build: run __graft_entry__.build() first")
    newest = max(os.path.getmtime(os.path.join(CSRC, f)) for f in os.listdir(CSRC))
    if os.path.getmtime(REPORT) < newest:
        pytest.skip("the build is older than the sources: run __graft_entry__.build() again")
    with open(REPORT) as f:
        return json.load(f)


def _match(report, part):
    return {k: v for k, v in report.items() if part in k}


def test_every_hot_kernel_is_reported(report):
    for part in HOT:
        assert _match(report, part), part


def test_no_hot_kernel_spills(report):
    for part in HOT:
        for k, v in _match(report, part).items():
            assert v.get("scratch", 0) == 0, (k, v)


def test_lds_fits_a_cu(report):
    for k, v in report.items():
        assert v.get("lds", 0) <= 160 * 1024, (k, v)


@pytest.mark.parametrize("part,floor,why", FLOORS)
def test_occupancy_floors(report, part, floor, why):
    ks = _match(report, part)
    assert ks, part
    for k, v in ks.items():
        assert v["occupancy"] >= floor, (k, v, why)


def test_attention_keeps_mfma_results_in_vgprs(report):
    """The attention kernels are built with their MFMA results in VGPRs, so
    no accumulator registers are allocated (the softmax would otherwise
    copy them back and forth every key tile)."""
    for part in ("k_attn_fwd64", "k_attn_dq64", "k_attn_dkv64"):
        for k, v in _match(report, part).items():
            assert v.get("agpr", 0) == 0, (k, v)
