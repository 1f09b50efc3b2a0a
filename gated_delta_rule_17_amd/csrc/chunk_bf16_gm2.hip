// bf16 I/O, bf16 MFMA operands, fp32 accumulation and state; gate mode 2.
#include "launch.hpp"

#define GDR_IO bf16
#define GDR_CT bf16
#define GDR_GM 2
#define GDR_NAME(x) chunk_bf16_gm2_##x
// bf16 I/O with a per-channel decay runs the pipelined kernels; this one
// covers no or a scalar decay with the per-channel erase gate.
#define GDR_CASES(X) X(128, 64, false) X(128, 32, false) X(128, 16, false) X(64, 64, false) X(64, 32, false) X(64, 16, false)
#include "chunk_instances.inc"
