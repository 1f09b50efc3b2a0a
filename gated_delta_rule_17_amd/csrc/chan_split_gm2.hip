// Two-pass chunk kernels for a per-key-channel decay, bf16 I/O, gate mode 2
// (per-channel erase gate, beta write gate).
#include "launch.hpp"
#include "chan_split_kernel.hpp"

#define GDR_GM 2
#define GDR_NAME(x) chan_split_gm2_##x
#include "chan_split_instances.inc"
