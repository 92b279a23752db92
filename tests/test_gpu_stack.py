"""Model-level check of the HEAL path on random-initialised Llama-style stacks, against the FP64 forward of
``oracle.stack``: a small one (2 layers, d 1024, 8/2 heads, FFN 3584, vocab 4096, 64-token prompt, 8 greedy steps)
and the full-size one of the model-level configuration (32 layers, d 4096, 32/8 heads, FFN 14336, vocab 128256,
512-token prompt, 64 greedy steps).  The HEAL path must give the FP64 argmax at every teacher-forced step and
decode the same tokens on its own, with a final-hidden normwise error that the INT16 quantisation of Q/K/V bounds
(per (token, head) rounding, about 1e-4 relative per attention), and far below the plain-bf16 path's."""
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


def test_full_stack_agrees_with_fp64(heal):
    """The full-size stack of the model-level configuration: 32 layers, d 4096, 32/8 heads, FFN 14336, vocabulary
    128256, 512-token prompt, 64 greedy steps (about a minute, and about 70 GB of host memory for the FP64
    model).  The HEAL path must give the FP64 argmax at all 64 teacher-forced steps and never leave the FP64
    tokens when decoding on its own, with a final-hidden error far below plain bf16's."""
    import llama_stack

    banner("decoder stack 32 layers, d 4096, 512 + 64 tokens: HEAL and bf16 against FP64")
    res = llama_stack.run(llama_stack.FULL, seed=0)
    h, b = res["heal"], res["bf16"]
    summary = (f"HEAL: teacher-forced {h['teacher_forced_agreement']:.4f}, first divergence "
               f"{h['free_running_first_divergence']}, final-hidden error max {h['final_hidden_normwise_err_max']:.3e}; "
               f"bf16: teacher-forced {b['teacher_forced_agreement']:.4f}, first divergence "
               f"{b['free_running_first_divergence']}, final-hidden error max {b['final_hidden_normwise_err_max']:.3e}; "
               f"smallest FP64 top-2 gap {res['fp64_top2_gap_min']:.2e}")
    print(f"[stack] {summary}")
    assert h["teacher_forced_agreement"] == 1.0, summary
    assert h["free_running_first_divergence"] is None, summary
    assert h["final_hidden_normwise_err_max"] < 2e-3, summary
    assert h["final_hidden_normwise_err_max"] < b["final_hidden_normwise_err_max"] / 20, summary
    assert h["teacher_forced_agreement"] >= b["teacher_forced_agreement"], summary
    # time per output token, one graph-replayed decode step each: the global FP32 pipeline streams twice the
    # weight bytes of the native bf16 one
    t = res["tpot"]
    print(f"[stack] tpot {t}")
    assert 0 < t["bf16_ms"] < t["fp32_ms"] and t["heal_ms"] > 0, t
