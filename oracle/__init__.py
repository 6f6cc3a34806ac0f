"""CPU oracle for the QJL key-cache sketch: plain, slow, float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package
entry point and the CPU-baseline leg of the benchmark may import it.  The HIP
library never calls it, and it shares no code with the HIP library: it has its
own random streams (rng.py), sketch construction (sketch.py) and quantizer /
estimator (qjl.py).

Parity status of each function:
  rng.*            pinned: SplitMix64 published outputs; Gaussian moments and
                   a Kolmogorov-Smirnov test; permutation validity.
  sketch.sylvester, sketch.fwht
                   pinned: scipy.linalg.hadamard, H H^T = d I.
  sketch.make_fqjl / fqjl_apply / FqjlSketch.explicit
                   pinned: the stepwise chain equals the explicit product for
                   d <= 64; coordinate variance ||k||^2 over G; exact
                   unbiasedness conditional on D and P (Monte Carlo).
  sketch.make_dense
                   pinned: Gaussian moments; the exact S values themselves are
                   "parity unpinned" by the pages (the generator is ours) and
                   are tied to the HIP library only through the sketch export.
  qjl.pack_bits / unpack_bits
                   pinned: hand-computed words for a hand-written sketch.
  qjl.quantize / project / score / estimator_constant
                   pinned: Monte-Carlo unbiasedness over sketch seeds (within
                   3 standard errors), the closed-form variance, error ~ m^-1/2,
                   the dither factor sqrt(1 + rho^2), invariances and special
                   cases.
  rng.dither_magnitudes / dither_signs / dither
                   pinned: sign words written out by hand from the
                   definition; half-normal magnitudes; one key's dither is
                   N(0, 1) over sketch draws (moments, KS, E exp(-t xi^2));
                   fair, per-key signs; the dither-factor Monte Carlo.
  FQJL distortion magnitude: no closed form on the pages -> "parity unpinned";
                   only its decrease with m is tested.
  attention.softmax_rows / decode_attention
                   pinned: scipy.special.softmax; a two-key closed form; zero
                   scores and zero scale give the mean of the values; key
                   permutation invariance; a dominant key returns its value row.
"""
from . import rng, sketch, qjl, attention  # noqa: F401
