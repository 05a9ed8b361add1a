"""CPU oracle (test infrastructure only): see ``oracle/dgq_oracle.py``.

Only the test suite, the smoke check and the bench's cpu_baseline leg may import this package.
"""

from .dgq_oracle import *  # noqa: F401,F403
from .dgq_oracle import (  # noqa: F401
    AppendState,
    HeadCompressed,
    SegParams,
    compress_head,
    decode_attention,
    rel_err,
)
