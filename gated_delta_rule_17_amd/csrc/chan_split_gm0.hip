// Two-pass chunk kernels for a per-key-channel decay, bf16 I/O, gate mode 0
// (beta erase gate, beta write gate).
#include "launch.hpp"
#include "chan_split_kernel.hpp"

#define GDR_GM 0
#define GDR_NAME(x) chan_split_gm0_##x
#include "chan_split_instances.inc"
