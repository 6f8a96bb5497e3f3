"""fp64 CPU oracle for the OrbitQuant quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library (``free_bit_quantization_amd``);
the two sides meet only through seeded inputs and the library's outputs.

Sources (pages on OrbitQuant, cited by title and section):

* "OrbitQuant: data-agnostic quantization for image and video" (rcap.io
  summary of the paper) -- the mechanism paragraphs ("core trick",
  "rotation cancels", "Randomized Permuted Block-Hadamard") and the
  offline / online pseudo-code.  This is the method authority.
* "OrbitQuant quantizes FLUX.1 and Wan 2.1 with no calibration data"
  (aiweekly.co) -- one Lloyd-Max codebook per input dimension.

Modules:

* :mod:`oracle.rpbh`      -- seeded RPBH rotation, dense and fast forms.
* :mod:`oracle.codebook`  -- the marginal f_d and the Lloyd-Max quantizer.
* :mod:`oracle.quant`     -- weight / activation quantization, index
  packing, dequantized product, GELU.
* :mod:`oracle.rtn`       -- INT4 round-to-nearest weights and the W4A16
  linear of the AdaLN modulation projections.

Every function computes in float64 and follows the pages' steps in their
order; a library primitive (matmul, searchsorted, betainc) serves as a
step where named.  Readings of points the pages leave open are listed in
the repository's design notes and restated at each function.
"""

from . import rpbh, codebook, quant  # noqa: F401
