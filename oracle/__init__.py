"""fp64 CPU oracle of the target-verify path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this
package.  It shares no code with the HIP library.
"""
from .tv_oracle import (SEQ_OK, SEQ_BAD_PARENT, SEQ_POOL_FULL, widen, build_plan, anc_to_bits,
                        State, from_scratch, from_entries, prefix_rows, verify_attention,
                        Scratch, build_scratch, accept, refresh, StepResult, step)
from .draft_tree import expanded_count, candidate_count, build_draft_tree
