"""CPU oracle for the SSD forward: test infrastructure only.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import this
package.  The product path (the HIP library and its binding) never imports, links or runs
anything here, and nothing here imports the product path.

Contents
  forward(...)          fp64 sequential recurrence (plain C, OpenMP over (batch, head)),
                        see ``ssd_oracle.c``; this is the reference every GPU result is
                        compared with.
  chunked_forward(...)  the chunked two-algorithm form in fp64 numpy, following the
                        aiwiki "State Space Duality" page ("Two algorithms for one operator"
                        and its PyTorch sketch) with the corrections listed in its
                        docstring; it also returns the per-chunk states, for localising
                        kernel bugs.  Pinned against ``forward`` by the CPU tests.
  discretize            the discretisation front-end (llms.blog "The Selection Mechanism"):
                        Delta = softplus(dt + bias), log a = -Delta exp(A_log), B-bar = Delta B;
                        ``discretize.forward_dt`` runs the recurrence in that form.
  backward              the adjoint of the recurrence in fp64 (plain C, ``ssd_oracle_bwd.c``):
                        the gradients of <dy, y> + <dfinal, final> with respect to every input.
  varlen                packed variable-length batches: every sequence of a packed batch
                        through the recurrence by itself (``varlen.forward_varlen``).
"""
from .recurrence import Oracle, build, default_oracle, forward, default_threads
from .chunked import chunked_forward
from . import discretize
from . import backward
from . import varlen

__all__ = ["Oracle", "build", "default_oracle", "forward", "default_threads", "chunked_forward", "discretize", "backward",
           "varlen"]
