"""Seeded synthetic inputs shared by the GPU path's tests/bench and by the oracle's tests.

This module only produces input bytes. It holds none of the matrix-multiply arithmetic: no
products, no accumulation, no output rounding, no tolerance. Both sides read the very same
bf16 bit patterns, generated here on the host.

Generator (counter based, so any element can be produced independently of the others):

* ``splitmix64(seed, c)``: the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014) applied to the state
  ``seed + (c + 1) * 0x9E3779B97F4A7C15 (mod 2**64)``.
* Normal element ``i`` of a stream: ``u1 = ((splitmix64(seed, 2i) >> 11) + 1) * 2**-53`` in
  (0, 1], ``u2 = (splitmix64(seed, 2i + 1) >> 11) * 2**-53`` in [0, 1), and
  ``z = sqrt(-2 ln u1) * cos(2 pi u2)`` (the cosine branch of the Box-Muller transform), in
  float64; then ``z * sigma`` is cast to float32 (round to nearest even) and the float32 value is
  rounded to bfloat16 (round to nearest even).
* Integer element ``i``: ``(splitmix64(seed, i) >> 32) % (2r + 1) - r``, an integer in
  [-r, r], exactly representable in bfloat16 for the small ``r`` used.
* Element ``i`` of an R x C matrix is its row-major logical index ``row * C + col``; the leading
  dimension of the buffer it is written to does not change the values.
"""

from .generate import (  # noqa: F401
    GAMMA,
    splitmix64,
    normal_bf16,
    integer_bf16,
    ones_bf16,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    matrix,
)
from .workloads import WORKLOADS, Workload, workload  # noqa: F401
