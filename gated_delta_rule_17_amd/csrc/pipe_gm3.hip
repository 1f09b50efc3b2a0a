// Pipelined chunk kernel, bf16 I/O, beta erase gate, write gate mode 3
// (per value channel).
#include "launch.hpp"
#include "pipe_kernel.hpp"

#define GDR_GM 3
#define GDR_NAME(x) pipe_gm3_##x
#define GDR_PIPE_CASES(X) X(128, 4) X(128, 2) X(128, 1) X(64, 4) X(64, 2) X(64, 1)
#include "pipe_instances.inc"
