"""Seeded synthetic inputs for block-top-k sparse paged decode.

This package only draws random inputs (paged KV pools, page tables, sequence
lengths, queries) with the shapes and value structure of the workloads the
method is evaluated on.  It holds none of the method's arithmetic: no
centroids, no scores, no selection and no attention.  Both the fp64 oracle
(through the tests) and the GPU library (through the tests and the benchmark)
consume what it produces; neither is imported here.
"""

from .workloads import (  # noqa: F401
    Workload,
    PageLayout,
    WORKLOADS,
    SMALL_WORKLOADS,
    get_workload,
    build_layout,
    make_kv_pool,
    draw_query_group,
    make_queries,
    step_seq_lens,
    completed_pages,
    setup_full_pages,
    rope_tables,
)
