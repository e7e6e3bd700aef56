"""CPU oracle for E2Former-V2's on-the-fly equivariant attention (test infrastructure).

This package is test infrastructure.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP
library and its Python binding) never does, and it imports nothing from the
product path.  The only code it shares with the GPU side is the seeded input
generator package ``gen``, which holds none of the method's arithmetic.

Everything here is plain, slow, float64 numpy that follows the definitions
on the pages:

* ``sh``      real solid harmonics R_l(r), l <= 2 (the geometric encoding
              R^(l_f)(r) of the E2Former-V2 write-up, section 2.3);
* ``cg``      Clebsch-Gordan coefficients from Racah's formula and the
              real-basis coupling tensors (dense SO(3) tensor product);
* ``wigner``  Wigner-D matrices of a rotation, fitted from the harmonics;
* ``tp``      the dense channel-wise tensor product h (x) R(r) summed over
              paths, and a separate reference EAAS used only to check
              Proposition 4.3;
* ``attn``    the three-step attention with every edge materialised.

Pins (tests marked ``not gpu``) tie each function to something other than
itself: sympy's Clebsch-Gordan routine, scipy's spherical harmonics,
textbook coupling identities, group properties of D, Proposition 4.3 (EAAS
equals the dense product), rotation equivariance, and a reduction of the
attention to torch's scaled-dot-product attention.
"""

from . import attn, cg, sh, tp, wigner  # noqa: F401
from .attn import attn_forward  # noqa: F401
from .tp import eaas_reference, paths, tp_dense  # noqa: F401
