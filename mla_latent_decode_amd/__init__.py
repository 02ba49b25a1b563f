"""QK-Normed MLA latent decode for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libqkmla.so`` (hand-written HIP
kernels); :mod:`mla_latent_decode_amd.ops` binds it for torch tensors.  Loading
the ops raises if the library has not been built: there is no fallback path.
"""
from .inputs import DSV3, TINY, WORKLOADS, Shape, make_inputs, workload_inputs  # noqa: F401
from .layout import cache_bytes_per_token, decode_flops_per_token  # noqa: F401
