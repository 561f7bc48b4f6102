"""Seeded synthetic inputs for the Adasum combiner.

This package only draws random numbers and lays out segment tables.  It holds
none of the combiner's arithmetic, and it is the one module that both sides of
every parity check use: the HIP path receives the tensors it returns, the
oracle receives the same tensors copied to the host.

The five workloads mirror the shapes and value statistics of the models the
text trains (ResNet-50, BERT-Large, BERT-Base) plus a small case and a stress
case; see ``shapes.py`` for the segment tables and ``generate.py`` for values.
"""

from .shapes import (  # noqa: F401
    CONFIGS,
    bert_lengths,
    config_offsets,
    offsets_from_lengths,
    resnet50_lengths,
)
from .generate import Workload, cancelling_pairs, make_workload, random_case, segment_params  # noqa: F401
