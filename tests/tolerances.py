"""Error budgets shared by the CPU pins and the GPU parity tests.

One rounding of normally distributed data to bf16 (8 significant bits,
round to nearest even) leaves a relative L2 error of U_BF16 = 1.66e-3
(measured on 2e6 samples at several scales; pinned in
test_oracle_pins.test_bf16_rounding_error_of_normal_data). Independent
roundings add in quadrature, so a result that passes through k bf16
materialisations on its way from the inputs sits about sqrt(k) * U_BF16 from
the exact fp64 value. The bounds below allow a factor 1.5 on that: the
activations amplify a relative error in their input by up to ~1.3 (GELU near
h = 1: h * gelu'(h) / gelu(h) = 1.28), and small test shapes fluctuate.

This estimate holds for activations whose derivative is continuous. ReLU and
ReGLU are not: rounding h moves values across the kink at 0, which flips
relu'(h) between 0 and 1, and the error then grows like sqrt(P(flip)) rather
than linearly (3e-2 measured at 384 x 272 x 528). Their backward is compared
with the rounded dataflow only.
"""

import math

U_BF16 = 1.66e-3
MARGIN = 1.5


def rounding_bound(k: int) -> float:
    """Relative L2 bound of a result that went through k bf16 roundings."""
    return MARGIN * math.sqrt(k) * U_BF16


# bf16 roundings on the chain of each gradient of the LayerNorm-MLP backward,
# as the oracle's round_intermediates mode takes them: xn and h1 (the
# forward's saved pre-activation; both halves when gated), act, dact, dh1 and
# dxn, each counted once where it feeds the gradient.
#   dkernel2 = act^T grad            : xn, h1, act
#   dbias1   = rows-sum of dh1 (fp32) : xn, h1, dact
#   dkernel1 = xn^T dh1              : xn, h1, dact, dh1
#   dx, dgamma, dbeta (from dxn)     : xn, h1, dact, dh1, dxn
#   dbias2   = rows-sum of grad      : none
_BWD_ROUNDINGS = {"dkernel2": 3, "dbias1": 3, "dkernel1": 4, "dx": 5, "dgamma": 5, "dbeta": 5, "dbias2": 0}
# gradients the library writes in bf16 (one more rounding at the output)
BWD_BF16_OUTPUTS = ("dx", "dkernel1", "dkernel2")


def bwd_roundings(name: str, gated: bool, output_rounded: bool) -> int:
    """Number of bf16 roundings between the inputs and gradient `name`."""
    k = _BWD_ROUNDINGS[name]
    if gated and k > 0:
        k += 1          # h1 holds two independently rounded halves
    if output_rounded and name in BWD_BF16_OUTPUTS:
        k += 1
    return k
