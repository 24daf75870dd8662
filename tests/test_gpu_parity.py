"""GPU vs oracle parity on the five workloads (lock-step, every call checked).

Small cases run every sequence through the oracle; full-size cases run every iteration
on the GPU in the launch configuration the benchmark times, check resampling and the
KV state for every prompt, and check the verify outputs on sampled sequences.
"""
import pytest
import torch

from tests import gpu_harness as H
from workloads import configs as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_c1_tiny_all_iterations():
    H.run(C.C1, C.C1.iters)


def test_c2_single_prompt_all_iterations():
    H.run(C.C2, C.C2.iters)


def test_c3_downsized_all_sequences():
    # B=2 prompts, full vocabulary (8 tiles per row incl. a ragged last tile)
    H.run(C.downsized(C.C3, B=2, iters=12), 12, label="/small")


def test_c3_full_size_all_iterations_sampled():
    H.run(C.C3, C.C3.iters, sample=3, label="/full")


def test_c4_downsized_all_sequences_with_sps():
    cfg = C.C4.scaled(name="c4_small", B=2, N=8, V=20011, iters=10, n_sets=2)
    H.run(cfg, 10, label="/small")


def test_c4_full_size_all_iterations_sampled_with_sps():
    H.run(C.C4, C.C4.iters, sample=2, sps_sample=3, label="/full")


def test_c5_downsized_all_sequences():
    cfg = C.C5.scaled(name="c5_small", B=1, N=128, V=30011, iters=12, n_sets=2)
    H.run(cfg, 12, label="/small")


def test_c5_full_size_all_iterations_sampled():
    H.run(C.C5, C.C5.iters, sample=2, label="/full")
