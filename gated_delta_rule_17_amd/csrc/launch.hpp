// Internal launcher interface between the C-ABI host code and the kernel
// translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_kernel.hpp"
#include "step_kernel.hpp"

namespace gdr {

// LDS bytes of a chunk kernel instance, or -1 if this build has no such instance.
int chunk_lds_bf16(int dk, int dvs, bool chan);
int chunk_lds_f32(int dk, int dvs, bool chan);

hipError_t launch_chunk_bf16(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s);
hipError_t launch_chunk_f32(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s);
// returns hipErrorInvalidValue when (io, dk, dv) has no instance
hipError_t launch_step(const StepParams& p, int io_bf16, int dk, int dv, int grid, hipStream_t s);
bool step_supported(int dk, int dv);

}  // namespace gdr
