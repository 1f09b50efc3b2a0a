// Pipelined chunk kernel for a per-key-channel decay, bf16 I/O, gate mode 3
// (beta erase gate, per-value-channel write gate).
#include "launch.hpp"
#include "chan_kernel.hpp"

#define GDR_GM 3
#define GDR_NAME(x) chan_gm3_##x
#define GDR_CHAN_CASES(X) X(128, 64) X(128, 32) X(128, 16) X(64, 64) X(64, 32) X(64, 16)
#include "chan_instances.inc"
