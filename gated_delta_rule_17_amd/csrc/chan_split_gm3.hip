// Two-pass chunk kernels for a per-key-channel decay, bf16 I/O, gate mode 3
// (beta erase gate, per-channel write gate).
#include "launch.hpp"
#include "chan_split_kernel.hpp"

#define GDR_GM 3
#define GDR_NAME(x) chan_split_gm3_##x
#include "chan_split_instances.inc"
