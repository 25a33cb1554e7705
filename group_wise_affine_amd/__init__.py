"""libqmm: affine group-wise quantized matmul for MI355X (gfx950).

The HIP library and its binding live in ``group_wise_affine_amd.qmm``;
``group_wise_affine_amd.synth`` holds the seeded input generators.
"""
