"""libgdn: the gated delta-rule (Gated DeltaNet) recurrence on AMD Instinct MI355X.

The compute path is the HIP library ``libgdn.so`` behind the C ABI in
``include/gdn.h``; ``gated_delta_rule_serial_amd.gdn`` is its ctypes binding
(argument marshalling only) and ``gated_delta_rule_serial_amd.synth`` draws the
seeded synthetic workloads.  Importing the package does not load the library;
the first call does, and raises if it is not built.
"""
from . import synth  # noqa: F401
from .gdn import (  # noqa: F401
    GdnError,
    decode_step,
    gate_prologue,
    gdn_decode_step,
    gdn_decode_step_slots,
    gdn_gate_prologue,
    gdn_prefill,
    gdn_prefill_slots,
    prefill,
)
