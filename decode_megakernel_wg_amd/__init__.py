"""MI355X-native decode megakernel: one persistent HIP kernel per decode step of a
parallel-transformer MoE decoder (gfx950), behind a C ABI (include/mk.h)."""
