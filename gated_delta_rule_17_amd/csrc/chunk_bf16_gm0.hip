// bf16 I/O, bf16 MFMA operands, fp32 accumulation and state; gate mode 0.
#include "launch.hpp"

#define GDR_IO bf16
#define GDR_CT bf16
#define GDR_GM 0
#define GDR_NAME(x) chunk_bf16_gm0_##x
// no and scalar decay go to the pipelined kernel
#define GDR_CASES(X) X(128, 64, true) X(128, 32, true) X(128, 16, true) X(64, 64, true) X(64, 32, true) X(64, 16, true)
#include "chunk_instances.inc"
