// Pipelined chunk kernel, bf16 I/O, beta erase gate, write gate mode 0
// (beta).
#include "launch.hpp"
#include "pipe_split_kernel.hpp"

#define GDR_GM 0
#define GDR_NAME(x) pipe_gm0_##x
#define GDR_PIPE_CASES(X) X(128, 64) X(128, 32) X(128, 16) X(64, 64) X(64, 32) X(64, 16)
#include "pipe_instances.inc"
