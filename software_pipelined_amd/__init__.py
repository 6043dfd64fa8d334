"""MI355X-native fused attention (forward, split-KV decoding, backward, MLA
decoding) and Mamba2 ChunkScan: gfx950 HIP kernels behind a C ABI.

``software_pipelined_amd.attn`` is the ctypes binding of ``libattn.so``;
``software_pipelined_amd.inputs`` holds the seeded synthetic workloads.
"""
