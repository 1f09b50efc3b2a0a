// Internal launcher interface between the C-ABI host code and the kernel
// translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_kernel.hpp"
#include "recur_kernel.hpp"
#include "step_kernel.hpp"

namespace gdr {

// One-pass chunk kernel instances, one pair of functions per (precision, gate
// mode): *_lds returns the LDS bytes of an instance or -1 if there is none;
// *_launch launches it (hipErrorInvalidValue if there is none).  With bf16
// I/O only the per-channel erase gate under no or a scalar decay runs here.
#define GDR_DECLARE(name)                                                                      \
  int name##_lds(int dk, int dvs, bool chan);                                                  \
  hipError_t name##_launch(const ChunkParams& p, int dk, int dvs, bool chan, int grid, hipStream_t s);
GDR_DECLARE(chunk_bf16_gm1)
GDR_DECLARE(chunk_bf16_gm2)
GDR_DECLARE(chunk_f32_gm0)
GDR_DECLARE(chunk_f32_gm1)
GDR_DECLARE(chunk_f32_gm2)
GDR_DECLARE(chunk_f32_gm3)
#undef GDR_DECLARE

// Pipelined kernel (bf16 I/O, no or scalar decay, beta erase gate), one pair
// per write-gate mode (0 = beta, 3 = per value channel).
// *_split_launch enqueues the two-pass form (dk 128, slices of 16 or 32):
// prep_grid chunk workgroups writing records to p.ws, then the pipelined
// kernel reading them.
#define GDR_DECLARE(name)                  \
  int name##_lds(int dk, int dvs);        \
  hipError_t name##_launch(const ChunkParams& p, int dk, int dvs, int grid, hipStream_t s); \
  hipError_t name##_split_launch(const ChunkParams& p, int dk, int dvs, int grid, int prep_grid, hipStream_t s); \
  int name##_split_lds(int dk, int dvs);
GDR_DECLARE(pipe_gm0)
GDR_DECLARE(pipe_gm3)
#undef GDR_DECLARE

// bytes of one chunk's record in the scalar-decay two-pass form: the ten
// non-zero 16 x 16 blocks of A and of A_qk, 336 chunk scalars, rounded up to
// 256 (matches PipeRec in pipe_kernel.hpp)
constexpr int64_t kPipeRecBytes = 11776;

// LDS bytes of the second pass of the scalar-decay two-pass form (-1: none)
inline int pipe_split_lds(int gm, int dk, int dvs) {
  return gm == 0 ? pipe_gm0_split_lds(dk, dvs) : pipe_gm3_split_lds(dk, dvs);
}

inline hipError_t launch_pipe_split(int gm, const ChunkParams& p, int dk, int dvs, int grid, int prep_grid,
                                    hipStream_t s) {
  return gm == 0 ? pipe_gm0_split_launch(p, dk, dvs, grid, prep_grid, s)
                 : pipe_gm3_split_launch(p, dk, dvs, grid, prep_grid, s);
}

// Pipelined kernel for a per-key-channel decay (bf16 I/O), one pair per gate
// mode.
#define GDR_DECLARE(name)                  \
  int name##_lds(int dk, int dvs);        \
  hipError_t name##_launch(const ChunkParams& p, int dk, int dvs, int grid, hipStream_t s);
GDR_DECLARE(chan_gm0)
GDR_DECLARE(chan_gm1)
GDR_DECLARE(chan_gm2)
GDR_DECLARE(chan_gm3)
#undef GDR_DECLARE

// Two-pass kernels for a per-key-channel decay (bf16 I/O, dk 128, value
// slices of 16 or 32), one pair per gate mode: *_lds gives the second pass's
// LDS bytes (-1: no instance); *_launch enqueues both passes (prep_grid
// chunk workgroups, then grid slice workgroups) with workspace ws.
#define GDR_DECLARE(name)                 \
  int name##_lds(int dk, int dvs);       \
  hipError_t name##_launch(const ChunkParams& p, void* ws, int dk, int dvs, int grid, int prep_grid, hipStream_t s);
GDR_DECLARE(chan_split_gm0)
GDR_DECLARE(chan_split_gm1)
GDR_DECLARE(chan_split_gm2)
GDR_DECLARE(chan_split_gm3)
#undef GDR_DECLARE

inline int chan_split_lds(int gm, int dk, int dvs) {
  switch (gm) {
    case 0: return chan_split_gm0_lds(dk, dvs);
    case 1: return chan_split_gm1_lds(dk, dvs);
    case 2: return chan_split_gm2_lds(dk, dvs);
    default: return chan_split_gm3_lds(dk, dvs);
  }
}

inline hipError_t launch_chan_split(int gm, const ChunkParams& p, void* ws, int dk, int dvs, int grid,
                                    int prep_grid, hipStream_t s) {
  switch (gm) {
    case 0: return chan_split_gm0_launch(p, ws, dk, dvs, grid, prep_grid, s);
    case 1: return chan_split_gm1_launch(p, ws, dk, dvs, grid, prep_grid, s);
    case 2: return chan_split_gm2_launch(p, ws, dk, dvs, grid, prep_grid, s);
    default: return chan_split_gm3_launch(p, ws, dk, dvs, grid, prep_grid, s);
  }
}

// bytes of one chunk's workspace record (dk 128): E_bar, Q_gamma, K_tail
// rows, the ten non-zero 16 x 16 blocks of A and of A_qk, gamma_C (matches
// SplitRec in chan_split_kernel.hpp)
constexpr int64_t kSplitRecBytes = 3 * 64 * 128 * 2 + 2 * 10 * 16 * 16 * 2 + 128 * 4;

// Plain fp32 chunk kernel (plain_kernel.hpp): io fp32 or bf16, dk 64 or 128,
// value slices of 16 columns.  plain_lds gives the LDS bytes (-1: no instance).
int plain_lds(int dk);
hipError_t launch_plain(const ChunkParams& p, bool bf16io, int dk, int grid, hipStream_t s);
// Its two-pass form (plain_split_kernel.hpp): prep_grid chunk workgroups
// write the records to the arrays of ws (plain_split_layout in
// bwd_params.hpp), then grid slice workgroups run the recurrence.
// Its recurrence runs on the matrix cores with slices of 64 columns, or on
// the vector ALUs with slices of 16 (the per-value-channel beta, erase kind
// 2, whose substitution differs per column; or a caller's 16-column split).
struct BwdWs;
inline int plain_split_slice(int erase, int dv, int dv_split) {
  return (erase == 2 || dv % 64 != 0 || dv_split == 16) ? 16 : 64;
}
int plain_split_lds(int dk, int dvs);
hipError_t launch_plain_split(const ChunkParams& p, const BwdWs& ws, bool bf16io, int dk, int dvs, int grid,
                              int prep_grid, hipStream_t s);

// Chunk kernel chosen for (io, dk, decay kind, erase kind, qmix): the plain
// fp32 kernel takes the per-value-channel beta (erase 2), a time-varying
// lambda (qmix 2) and fp32 I/O at dk 128; otherwise the pipelined kernels take
// bf16 I/O, the scalar-decay one the beta erase gate only; the rest go to the
// one-pass kernel.
enum ChunkKernel { kOnePass = 0, kPipe = 1, kChan = 2, kPlain = 3 };
inline ChunkKernel chunk_kernel_for(bool bf16io, int dk, int decay, int erase, int qmix) {
  if (erase == 2 || qmix == 2 || (!bf16io && dk == 128)) return kPlain;
  if (!bf16io) return kOnePass;
  if (decay == 2) return kChan;
  return erase == 0 ? kPipe : kOnePass;
}

inline int chan_lds(int gm, int dk, int dvs) {
  switch (gm) {
    case 0: return chan_gm0_lds(dk, dvs);
    case 1: return chan_gm1_lds(dk, dvs);
    case 2: return chan_gm2_lds(dk, dvs);
    default: return chan_gm3_lds(dk, dvs);
  }
}

inline hipError_t launch_chan(int gm, const ChunkParams& p, int dk, int dvs, int grid, hipStream_t s) {
  switch (gm) {
    case 0: return chan_gm0_launch(p, dk, dvs, grid, s);
    case 1: return chan_gm1_launch(p, dk, dvs, grid, s);
    case 2: return chan_gm2_launch(p, dk, dvs, grid, s);
    default: return chan_gm3_launch(p, dk, dvs, grid, s);
  }
}

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
    case 5: return chunk_bf16_gm1_lds(dk, dvs, chan);
    case 6: return chunk_bf16_gm2_lds(dk, dvs, chan);
    default: return -1;
  }
}

inline hipError_t launch_chunk(bool bf16io, int gm, const ChunkParams& p, int dk, int dvs, bool chan, int grid,
                               hipStream_t s) {
  switch ((bf16io ? 4 : 0) + gm) {
    case 0: return chunk_f32_gm0_launch(p, dk, dvs, chan, grid, s);
    case 1: return chunk_f32_gm1_launch(p, dk, dvs, chan, grid, s);
    case 2: return chunk_f32_gm2_launch(p, dk, dvs, chan, grid, s);
    case 3: return chunk_f32_gm3_launch(p, dk, dvs, chan, grid, s);
    case 5: return chunk_bf16_gm1_launch(p, dk, dvs, chan, grid, s);
    case 6: return chunk_bf16_gm2_launch(p, dk, dvs, chan, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// returns hipErrorInvalidValue when (io, dk, dv) has no instance
hipError_t launch_step(const StepParams& p, int io_bf16, int dk, int dv, int grid, hipStream_t s);
bool step_supported(int dk, int dv);

// multi-token recurrent kernel (recur_kernel.hpp): one workgroup of dv
// threads per (batch, head)
bool recur_supported(int dk, int dv);
hipError_t launch_recur(const RecurParams& p, bool bf16io, int dk, int dv, int grid, hipStream_t s);

// backward (bwd_kernel.hpp): record pass, reverse state pass, product and
// key passes, and the per-head lambda reduction, on one stream
struct BwdParams;
bool bwd_supported(int dk, int dv);
hipError_t launch_bwd(const BwdParams& p, bool bf16io, int dk, int dv, int BH, hipStream_t s);

// standalone output epilogue over rows of dv values; y may equal o
bool norm_gate_supported(int dv);
hipError_t launch_norm_gate(const void* o, const void* gate, const float* nw, void* y, int64_t rows, int dv,
                            bool bf16io, float eps, hipStream_t s);

}  // namespace gdr
