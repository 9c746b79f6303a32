"""Seeded synthetic inputs for fusion groups.

This package holds input generators and the neutral text form of an op DAG.
It does none of the arithmetic a fusion group computes: it draws random
numbers, lays out shapes and parses/prints DAG text.  Both the CPU oracle
(``oracle/``) and the GPU path (``elementwise_reduction_groups_amd``) read
their inputs from here; neither imports the other.
"""
from .dag import Node, parse_dag, format_dag, random_chain_dag, OPS  # noqa: F401
from . import configs  # noqa: F401
