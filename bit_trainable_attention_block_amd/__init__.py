"""SageBwd INT8 attention for MI355X (gfx950).

The compute path is the C-ABI library ``libsage.so`` built from the HIP
sources in ``csrc/``; ``binding`` marshals PyTorch device tensors and streams
into it.  ``workloads`` holds the seeded synthetic inputs.
"""
