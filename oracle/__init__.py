"""Reference oracle for the WaveFilter per-step sparse-attention path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 CPU
implementation of what the path computes, written from the WaveFilter pages
(arXiv 2606.00724: section 2.1 equations 1-4, section 2.2 equation 5,
Figure 2 and section 3.1).  It exists to check the HIP library, and only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it.  It shares no code with the HIP library and imports nothing from
it; the library never calls back into it.

Every function works on one (layer, sequence, head) at a time, on float64
arrays that hold exactly the (already rounded) input values.
"""

from .wavefilter import (  # noqa: F401
    HAAR_G,
    HAAR_H,
    DB2_G,
    DB2_H,
    analysis_step_periodic,
    dwt_pyramid,
    analysis_step,
    synthesis_step,
    haar_pyramid,
    haar_reconstruct,
    level_scores,
    top_k,
    select,
    attend,
    select_attend,
    attend_selected,
    refresh_top,
    SelectResult,
)
