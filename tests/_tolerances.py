"""Acceptance bars of the GPU parity tests against the fp64 oracle, over real tokens."""

F32_MAX_ABS = 1e-5
# FP32 I/O on exact FP32 arithmetic, by data class (qk_mult -> (max abs, rel L2)): the FP32 bar
# on N(0,1) data; with Q, K scaled by 8 about five times the worst error of a NumPy model of
# exactly the kernel's FP32 arithmetic (tests/test_f32_model.py), since FP32 itself errs by
# ~2e-5 at those logits.
F32_TOL = {1.0: (F32_MAX_ABS, 1e-5), 8.0: (1e-4, 1e-5)}
BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
# FP32 I/O with split-bf16 matrix-core products ("f32_split"): about five times the
# worst error of a NumPy model of exactly that arithmetic (tests/test_split_model.py)
# on N(0,1) data, and on data with Q, K scaled by 8 (logits ~64x larger, errors with them).
SPLIT_TOL = {1.0: (5e-5, 3e-5), 8.0: (4e-3, 3e-4)}  # qk_mult -> (max abs, rel L2)
# Fused AdaLN + residual (FP32 arithmetic): float32 output within ADALN_F32_ABS, about five times
# the worst error of a float32 NumPy model of the same steps (tests/test_adaln_model.py); bf16
# output adds one round-to-nearest-even rounding, at most 2^-9 of the value.
ADALN_F32_ABS = 1e-5
ADALN_BF16_REL = 2.0 ** -8
