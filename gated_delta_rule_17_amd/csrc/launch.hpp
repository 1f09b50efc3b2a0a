// Internal launcher interface between the C-ABI host code and the kernel
// translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_kernel.hpp"
#include "step_kernel.hpp"

namespace gdr {

// Chunk kernel instances, one pair of functions per (precision, gate mode):
// *_lds returns the LDS bytes of an instance or -1 if there is none; *_launch
// launches it (hipErrorInvalidValue if there is none).
#define GDR_DECLARE(name)                                                                      \
  int name##_lds(int dk, int dvs, bool chan);                                                  \
  hipError_t name##_launch(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s);
GDR_DECLARE(chunk_bf16_gm0)
GDR_DECLARE(chunk_bf16_gm1)
GDR_DECLARE(chunk_bf16_gm2)
GDR_DECLARE(chunk_bf16_gm3)
GDR_DECLARE(chunk_f32_gm0)
GDR_DECLARE(chunk_f32_gm1)
GDR_DECLARE(chunk_f32_gm2)
GDR_DECLARE(chunk_f32_gm3)
#undef GDR_DECLARE

// Pipelined kernel (bf16 I/O, no or scalar decay, beta erase gate), one pair
// per write-gate mode (0 = beta, 3 = per value channel).
#define GDR_DECLARE(name)                  \
  int name##_lds(int dk, int dvs);        \
  hipError_t name##_launch(const ChunkParams& p, int dk, int dvs, int grid, hipStream_t s);
GDR_DECLARE(pipe_gm0)
GDR_DECLARE(pipe_gm3)
#undef GDR_DECLARE

// true when the pipelined kernel covers (io, decay kind, erase kind)
inline bool pipe_covers(bool bf16io, int decay, int erase) { return bf16io && decay != 2 && erase == 0; }

inline int pipe_lds(int gm, int dk, int dvs) { return gm == 0 ? pipe_gm0_lds(dk, dvs) : pipe_gm3_lds(dk, dvs); }

inline hipError_t launch_pipe(int gm, const ChunkParams& p, int dk, int dvs, int grid, hipStream_t s) {
  return gm == 0 ? pipe_gm0_launch(p, dk, dvs, grid, s) : pipe_gm3_launch(p, dk, dvs, grid, s);
}

// gate mode of (erase, write): 0 = (BETA, BETA), 1 = (CHANNEL, CHANNEL),
// 2 = (CHANNEL, BETA), 3 = (BETA, CHANNEL)
inline int gate_mode(int erase, int write) {
  return erase == 0 ? (write == 0 ? 0 : 3) : (write == 0 ? 2 : 1);
}

inline int chunk_lds(bool bf16io, int gm, int dk, int dvs, bool chan) {
  switch ((bf16io ? 4 : 0) + gm) {
    case 0: return chunk_f32_gm0_lds(dk, dvs, chan);
    case 1: return chunk_f32_gm1_lds(dk, dvs, chan);
    case 2: return chunk_f32_gm2_lds(dk, dvs, chan);
    case 3: return chunk_f32_gm3_lds(dk, dvs, chan);
    case 4: return chunk_bf16_gm0_lds(dk, dvs, chan);
    case 5: return chunk_bf16_gm1_lds(dk, dvs, chan);
    case 6: return chunk_bf16_gm2_lds(dk, dvs, chan);
    default: return chunk_bf16_gm3_lds(dk, dvs, chan);
  }
}

inline hipError_t launch_chunk(bool bf16io, int gm, const ChunkParams& p, int dk, int dvs, bool chan, int grid,
                               hipStream_t s) {
  switch ((bf16io ? 4 : 0) + gm) {
    case 0: return chunk_f32_gm0_launch(p, dk, dvs, chan, grid, s);
    case 1: return chunk_f32_gm1_launch(p, dk, dvs, chan, grid, s);
    case 2: return chunk_f32_gm2_launch(p, dk, dvs, chan, grid, s);
    case 3: return chunk_f32_gm3_launch(p, dk, dvs, chan, grid, s);
    case 4: return chunk_bf16_gm0_launch(p, dk, dvs, chan, grid, s);
    case 5: return chunk_bf16_gm1_launch(p, dk, dvs, chan, grid, s);
    case 6: return chunk_bf16_gm2_launch(p, dk, dvs, chan, grid, s);
    default: return chunk_bf16_gm3_launch(p, dk, dvs, chan, grid, s);
  }
}

// returns hipErrorInvalidValue when (io, dk, dv) has no instance
hipError_t launch_step(const StepParams& p, int io_bf16, int dk, int dv, int grid, hipStream_t s);
bool step_supported(int dk, int dv);

}  // namespace gdr
