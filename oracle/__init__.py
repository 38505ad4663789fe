"""fp64 CPU oracle for the KDA forward. Test infrastructure only: see ``kda_oracle``."""
from .kda_oracle import (DEFAULT_EPS, document_bounds, kda_document, kda_forward,  # noqa: F401
                         kda_tasks, l2_normalise, default_workers)
from .kda_oracle_bwd import kda_backward, kda_document_backward  # noqa: F401,E402
