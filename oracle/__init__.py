"""CPU oracle for the fused weight-gradient GEMM + optimizer step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.

What it computes is the plain, unfused definition of the method described on
the page "docs(audit): FORGE assessment + residency-aware epilogue-fusion
track" (Tessera PR 565): the weight gradient dW = X^T dY reduced over all
tokens (section "What's already in tree and easy to miss", the transposed-lhs
matmul), rounded once to float32, then an ordinary float32 AdamW or
SGD-momentum step (section "Claim hygiene on the source": the public release
ships AdamW and SGD only). Fusion changes where the gradient lives, not its
value (section "Math verified, not asserted", P1), so the unfused definition
is the reference for the fused kernels.

fp8 inputs (the paper's fp8 row in P6) are in ``lowp.py``, with the model of
the fp8 matrix instruction's dot product (its C helper is ``fp8_dot.c``). The
precision variants of P6 (a bf16-rounded gradient, bf16 moments) and the
float64 reference they are measured against are in ``ref.py`` too; the P6
study itself in ``precision_study.py``.

Parity pins (tests that check this package against closed forms, exact
rational arithmetic, hand-worked examples and invariants) live in
tests/test_oracle_pins.py, tests/test_precision_oracle.py,
tests/test_dgrad_oracle.py and tests/test_fp8_oracle.py; the fp8 model's two
constants are pinned bit for bit against the instruction by GPU regression
tests on designed inputs (tests/test_gpu_fp8.py).
Parity unpinned: the exact summation order inside the GPU contraction (only
the accumulation floor in ``floor.py`` bounds it), and the magnitudes the page
quotes without their setups (2.24x at 50% routing; ~900x / ~1x, which the
study reproduces under a stated reading of the error measure).
"""
from .ref import (  # noqa: F401
    ClipNotFusable,
    adamw_moments,
    adamw_param,
    adamw_step,
    adamw_step_f64,
    adamw_step_mixed,
    bf16_bits_to_f64,
    bf16_round,
    dgrad,
    dgrad_f64,
    grouped_adamw_step,
    grouped_sgdm_step,
    grouped_wgrad,
    sgdm_step,
    wgrad,
    wgrad_f64,
    wgrad_rows,
)
from .lowp import E4M3, E5M2, acc_floor_fp8, fp8_to_f64, wgrad_fp8, wgrad_fp8_f64  # noqa: F401
from .floor import (StateFloor, acc_floor, acc_floor_rows, dgrad_floor,  # noqa: F401
                    sgdm_arith_floor)
