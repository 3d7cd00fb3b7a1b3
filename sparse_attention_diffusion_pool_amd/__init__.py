"""libpisa for MI355X (gfx950): PISA piecewise sparse attention forward pass.

The computation lives in libpisa.so (HIP kernels behind the C ABI of include/pisa.h); this
package only builds it (``build``) and binds it (``_lib``).
"""

from ._lib import (DTYPE_BF16, DTYPE_F32, PHASE_EXACT, PHASE_FIRST, PHASE_ZEROTH,  # noqa: F401
                   ROUTING_COV, ROUTING_PLAIN, Plan, PisaError, header_functions, load,
                   pisa_attention)
