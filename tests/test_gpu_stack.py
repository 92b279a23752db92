"""Model-level check of the HEAL path on a small random-initialised Llama-style stack (2 layers, d 1024, 8/2
heads, FFN 3584, vocab 4096, 64-token prompt, 8 greedy steps; the full-size stack runs from
``tests/llama_stack.py --full``).  Against the FP64 forward of ``oracle.stack``: the HEAL path must give the
FP64 argmax at every teacher-forced step and decode the same tokens on its own, with a final-hidden normwise
error that the INT16 quantisation of Q/K/V bounds (per (token, head) rounding, about 1e-4 relative per
attention), and far below the plain-bf16 path's."""
import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu


def test_small_stack_agrees_with_fp64(heal):
    import llama_stack

    banner("decoder stack 2 layers, d 1024: HEAL and bf16 against FP64")
    res = llama_stack.run(llama_stack.SMALL, seed=0)
    h, b = res["heal"], res["bf16"]
    print(f"[stack] heal {h}\n[stack] bf16 {b}")
    assert h["teacher_forced_agreement"] == 1.0 and h["free_running_first_divergence"] is None
    assert h["final_hidden_normwise_err_max"] < 2e-4
    assert h["final_hidden_normwise_err_max"] < b["final_hidden_normwise_err_max"] / 20
