"""CPU oracle for the MoE token dispatch / grouped expert FFN / combine path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, the graft entry's ``smoke()`` check
and the bench's ``cpu_baseline`` leg use it. It shares no code with the HIP
library and imports nothing from it.

Everything is plain NumPy in float64, written to be checked by eye against
the layer's definition; see ``oracle.moe`` for the layer's functions,
``oracle.optim`` for the optimizer update, ``oracle.aux`` for the auxiliary
losses and routing metrics, ``oracle.ep`` for the expert-parallel token
exchange, and the passages each one follows.
"""
from .moe import *  # noqa: F401,F403
from .moe import __all__ as _moe_all
from .optim import *  # noqa: F401,F403
from .optim import __all__ as _optim_all
from .aux import *  # noqa: F401,F403
from .aux import __all__ as _aux_all
from .ep import *  # noqa: F401,F403
from .ep import __all__ as _ep_all

__all__ = list(_moe_all) + list(_optim_all) + list(_aux_all) + list(_ep_all)
