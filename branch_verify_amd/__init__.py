"""MI355X (gfx950) multi-branch draft-verification step for masked diffusion LMs.

The compute path is the C-ABI library libsfv.so (hand-written HIP kernels);
`branch_verify_amd.sfv` is its thin ctypes binding.  `synth` draws seeded
synthetic inputs.  Nothing here computes on the CPU."""
