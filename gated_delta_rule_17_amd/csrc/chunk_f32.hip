// fp32 I/O with fp32 MFMA (v_mfma_f32_16x16x4_f32) throughout, for the
// tighter fp32 tolerance.  dk = 64 only: at dk = 128 the fp32 operand tiles
// do not fit the 160 KB of LDS.  All four gate modes.
#include "launch.hpp"

#define GDR_IO float
#define GDR_CT float
#define GDR_CASES(X) X(64, 32, false) X(64, 16, false) X(64, 32, true) X(64, 16, true)

#define GDR_GM 0
#define GDR_NAME(x) chunk_f32_gm0_##x
#include "chunk_instances.inc"
#undef GDR_GM
#undef GDR_NAME
#define GDR_GM 1
#define GDR_NAME(x) chunk_f32_gm1_##x
#include "chunk_instances.inc"
#undef GDR_GM
#undef GDR_NAME
#define GDR_GM 2
#define GDR_NAME(x) chunk_f32_gm2_##x
#include "chunk_instances.inc"
#undef GDR_GM
#undef GDR_NAME
#define GDR_GM 3
#define GDR_NAME(x) chunk_f32_gm3_##x
#include "chunk_instances.inc"
