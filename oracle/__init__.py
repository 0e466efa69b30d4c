"""Plain, slow fp64 CPU oracle for the fused chunked KL distillation loss.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The product path (``output_projection_kl_amd``) never imports it and
shares no code with it.
"""

from .fkl_oracle import (  # noqa: F401
    teacher_distribution,
    forward,
    backward,
    forward_rows,
    grad_h_rows,
    grad_W_rows,
    dense_teacher_grid,
    topk_teacher,
    forward_terms,
    backward_terms,
)
