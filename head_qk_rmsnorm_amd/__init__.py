"""Fused in-place QK RMSNorm + rotary position embedding for AMD MI355X (gfx950).

The compute path is the HIP library ``libqknr.so`` (C ABI declared in
``include/qknr.h``); ``binding`` marshals torch tensors into it and
``torch_ops`` registers the ops as torch custom ops (``torch.ops.qknr.*``).
``workloads`` draws seeded synthetic inputs for tests and the benchmark.
"""
