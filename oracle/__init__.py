"""Plain, slow, fp64 CPU oracle for the NSNQuant KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code, table or constant generator with it.

Sources: the English gist.science explainer "NSNQuant: A Double Normalization
Approach for Calibration-Free Low-Bit Vector Quantization of KV Cache"
(gist.science/paper/2505.18231), Technical Summary, sections
"1. Normalize-Shift-Normalize (NSN)", "2. Hadamard Transform",
"3. Vector Quantization and Codebook" and "4. Implementation Details".
Every function names the section it follows; where the page is silent the
function states the reading it takes.
"""

from .nsn import *  # noqa: F401,F403
from .nsn import __all__  # noqa: F401
