"""SEED decode-time shallow recurrent state engine for AMD Instinct MI355X (gfx950).

Importing the package loads nothing native.  The HIP library and its
Python binding live in ``sink_rank_recurrent_amd.binding``; the seeded
synthetic inputs in ``sink_rank_recurrent_amd.workloads``.
"""
__all__ = ["binding", "workloads"]
