"""Oracle for the attention forward and backward passes: plain, slow, float64 CPU code.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call,
link or execute anything under ``oracle/``; only the test suite, the smoke
check and the bench's CPU-baseline leg do. It shares no code with the HIP
path (no kernels, headers, helpers, tables or constants); the only module
both sides use is ``attn_inputs``, which draws the seeded inputs and holds
none of the attention arithmetic.

Contents
  attention_f64        one-shot safe softmax attention, the plain definition
  attention_rows_f64   the same for a chosen subset of query rows
  attention_bwd_f64    the backward pass: dQ, dK, dV (and D) in closed form
  attention_loss_f64   sum(O * dO), the scalar those are the gradients of
  blockwise_f64        the streaming recurrence with the lagging-max rule
                       (used only to pin the recurrence and its rescale
                       counts; never the parity reference)
  ex2_emu_deg3         float32 CPU model of the degree-3 software exp2
                       (C, built with gcc; see ex2_emu.c)
  ex2_emu              the same with the degree-4 or degree-5 polynomial
  fit_ex2_poly         the fit that produced the degree-4/5 coefficients
  round_to_format      cast to bf16 / OCP E4M3 / OCP E5M2 (nearest-even,
                       saturating)
  lagging_max_p_cast_f64
                       the pages' simulation of P cast to a narrow type
                       (times 2^max_offset) under the lagging max

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force at 50 digits, library routines that differ from the ones used
here, and the numbers the pages print. No function is "parity unpinned".
"""
from .attention import attention_f64, attention_rows_f64, blockwise_f64
from .attention_bwd import attention_bwd_f64, attention_loss_f64
from .ex2_emu import ex2_emu, ex2_emu_deg3, build_ex2_emu
from .fit_ex2_poly import fit_ex2_poly
from .p_cast import lagging_max_p_cast_f64, rel_l2, round_to_format

__all__ = ["attention_f64", "attention_rows_f64", "blockwise_f64", "attention_bwd_f64", "attention_loss_f64",
           "ex2_emu", "ex2_emu_deg3", "build_ex2_emu", "fit_ex2_poly", "lagging_max_p_cast_f64", "rel_l2", "round_to_format"]
