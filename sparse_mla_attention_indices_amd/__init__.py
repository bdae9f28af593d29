"""Sparse MLA forward over top-k indices for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libsmla.so`` (hand-written HIP kernels);
``sparse_mla_attention_indices_amd.smla`` is its thin Python binding.
``workloads`` generates seeded synthetic inputs. Nothing is imported eagerly so
that the input generators can be used without the GPU library.
"""

__all__ = ["smla", "workloads"]
