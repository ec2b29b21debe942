"""Page-selected sparse paged decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libpsd.so (HIP kernels behind the C-ABI of include/psd.h);
this package only marshals arguments to it and sizes device buffers.
"""
from .api import (PsdError, PsdShape, decode_step, decode_workspace_bytes, dense_decode,
                  make_shape,
                  page_meta_update, select_merge, select_pages, select_score,
                  select_sparse_decode, select_sparse_decode_workspace_bytes,
                  select_coverage_workspace_bytes, select_pages_coverage,
                  select_workspace_bytes, sparse_decode, status_string, version)
from .runner import DecodeStep

__all__ = ["DecodeStep", "PsdError", "PsdShape", "decode_step", "decode_workspace_bytes",
           "dense_decode",
           "make_shape", "page_meta_update", "select_merge", "select_pages", "select_score",
           "select_sparse_decode", "select_sparse_decode_workspace_bytes", "select_workspace_bytes",
           "select_coverage_workspace_bytes", "select_pages_coverage",
           "sparse_decode", "status_string", "version"]
