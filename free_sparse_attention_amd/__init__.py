"""Combined sparse decode attention for MI355X (gfx950).

The computation lives in ``libfsa.so`` (HIP kernels behind the C ABI of
``include/fsa.h``); this package is its thin ctypes binding plus the build
script.  PyTorch is used only for device memory and streams.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    Dims,
    FsaError,
    LayerCfg,
    append_decode_attn,
    append_kv,
    build_page_meta,
    cfg,
    dense_decode_attn,
    dense_decode_workspace_bytes,
    device_memory,
    describe_step,
    dims,
    import_kv_plain,
    load,
    max_work_items,
    meta_bytes,
    quest_scores,
    read_probe,
    one_launch_stalls,
    set_one_launch,
    build_flags,
    select_pages,
    sparse_decode_attn,
    sparse_decode_attn_noalloc,
    sparse_decode_attn_launches,
    NOALLOC_SCRATCH_BYTES,
    sparse_decode_workspace_bytes,
    validate_inputs,
)
