"""fp64 CPU oracle for GQLA decode attention (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP library in decode_attention_02_amd/.
"""
from . import gqla_ref  # noqa: F401
