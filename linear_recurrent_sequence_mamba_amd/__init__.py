"""libm3ssm: the Mamba-3 SSM core recurrence (prefill scan and decode step)
as hand-written HIP kernels for gfx950 behind a C ABI."""
