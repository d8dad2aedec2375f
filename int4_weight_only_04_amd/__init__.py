"""MI355X-native INT4 weight-only decode GEMV (gfx950 HIP kernels behind a C ABI).

    from int4_weight_only_04_amd import w4
    pw, ps = w4.pack(q, s_bits, group)          # host packer (W4T4 layout)
    w4.gemv(pw_dev, ps_dev, x, y, n, k, group)   # y = W x on the GPU
    w4.gemv_gateup_silu(...); w4.Sweep([...], use_graph=True).run()
"""
from . import w4  # noqa: F401

__all__ = ["w4"]
