// libgdr host side: argument validation, launch planning and dispatch for
// the C ABI declared in include/gdr.h.  Validation is pure host code and runs
// before any HIP call, so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/gdr.h"
#include "bwd_params.hpp"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

gdr_status fail(gdr_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

constexpr int kOpChunk = 0, kOpStep = 1, kOpRecur = 2;

// bytes of beta: [B,T,H], or [B,T,H,dv] under the per-value-channel beta
int64_t beta_bytes(const gdr_args* a) {
  const int64_t tokens = int64_t(a->B) * a->H * a->T;
  return tokens * 4 * (a->erase == GDR_GATE_VALUE ? a->dv : 1);
}
// bytes of lambda: [H], or [B,T,H] for a time-varying lambda
int64_t lambda_bytes(const gdr_args* a) {
  return 4 * (a->qmix == 2 ? int64_t(a->B) * a->H * a->T : int64_t(a->H));
}

// a struct of ABI version 1 ends before the workspace fields, one of
// version 2 before the epilogue fields
constexpr size_t kArgsV1Size = offsetof(gdr_args, workspace);
constexpr size_t kArgsV2Size = offsetof(gdr_args, out_gate);

struct Workspace {
  void* ptr;
  uint64_t bytes;
};
Workspace workspace_of(const gdr_args* a) {
  if (a->struct_size < kArgsV2Size) return Workspace{nullptr, 0};
  return Workspace{a->workspace, a->workspace ? a->workspace_bytes : 0};
}

// the output epilogue of a call (gate == nullptr: none)
struct Epilogue {
  const void* gate;
  const float* weight;
  float eps;
};
constexpr float kDefaultEps = 1e-6f;
Epilogue epilogue_of(const gdr_args* a) {
  if (a->struct_size < sizeof(gdr_args) || !a->out_gate) return Epilogue{nullptr, nullptr, 0.f};
  return Epilogue{a->out_gate, a->norm_weight, a->norm_eps > 0.f ? a->norm_eps : kDefaultEps};
}

// Workspace bytes of the two-pass form for slice width dvs, or 0 when that
// form does not apply: it serves the two pipelined kernels (bf16 I/O) at dk
// 128 with slices of 16 or 32 columns (few heads), where a single pass would
// repeat every chunk's state-independent work in many slices, and the plain
// fp32 kernel (16-column slices) at every shape.
int64_t split_bytes(const gdr_args* a, int dvs) {
  const gdr::ChunkKernel kern = gdr::chunk_kernel_for(a->io == GDR_BF16, a->dk, a->decay, a->erase, a->qmix);
  if (kern == gdr::kPlain) {
    // the plain kernel's two-pass form: one record per chunk for every shape
    if (a->T < 1) return 0;
    const int64_t nrec = int64_t(a->B) * a->H * ((a->T + GDR_CHUNK - 1) / GDR_CHUNK);
    return gdr::plain_split_layout(nrec, a->dk, nullptr, nullptr);
  }
  if ((kern != gdr::kChan && kern != gdr::kPipe) || a->dk != 128 || (dvs != 16 && dvs != 32) || a->T < 1)
    return 0;
  const int64_t nchunks = (a->T + GDR_CHUNK - 1) / GDR_CHUNK;
  return int64_t(a->B) * a->H * nchunks * (kern == gdr::kChan ? gdr::kSplitRecBytes : gdr::kPipeRecBytes);
}

gdr::ChunkKernel kernel_for(const gdr_args* a) {
  return gdr::chunk_kernel_for(a->io == GDR_BF16, a->dk, a->decay, a->erase, a->qmix);
}

int dvs_candidates(const gdr_args* a, int* out) {
  if (kernel_for(a) == gdr::kPlain) {
    out[0] = 16;
    return 1;
  }
  if (a->io == GDR_BF16) {
    out[0] = 64; out[1] = 32; out[2] = 16;
    return 3;
  }
  out[0] = 32; out[1] = 16;
  return 2;
}

int chunk_lds(const gdr_args* a, int dvs) {
  const int gm = gdr::gate_mode(a->erase, a->write);
  switch (kernel_for(a)) {
    case gdr::kPipe: return gdr::pipe_lds(gm, a->dk, dvs);
    case gdr::kChan: return gdr::chan_lds(gm, a->dk, dvs);
    case gdr::kPlain: return dvs == 16 ? gdr::plain_lds(a->dk) : -1;
    default: return gdr::chunk_lds(a->io == GDR_BF16, gm, a->dk, dvs, a->decay == GDR_DECAY_CHANNEL);
  }
}

// pipelined kernels: two consumer waves (one for a 16-column slice) plus four
// producer waves (scalar decay) or four elementwise and two Gram waves
// (per-channel decay); one-pass and plain kernels: four waves
int chunk_block(const gdr_args* a, int dvs) {
  const int ncw = dvs >= 32 ? 2 : 1;
  switch (kernel_for(a)) {
    case gdr::kPipe: return 64 * (ncw + 4);
    case gdr::kChan: return 64 * (ncw + 6);
    default: return 256;
  }
}

gdr_status validate_impl(const gdr_args* a, int op, bool check_ptrs = true) {
  if (!a) return fail(GDR_E_NULL, "gdr_args pointer is NULL");
  if (a->struct_size < kArgsV1Size)
    return fail(GDR_E_ARGS, "struct_size %u is smaller than the version-1 gdr_args (%zu bytes)", a->struct_size,
                kArgsV1Size);
  if (op != kOpChunk && op != kOpStep && op != kOpRecur) return fail(GDR_E_ARGS, "unknown op %d", op);
  if (a->B < 1 || a->H < 1 || a->T < 0)
    return fail(GDR_E_SHAPE, "need B >= 1, H >= 1, T >= 0 (got B=%d H=%d T=%d)", a->B, a->H, a->T);
  if (op == kOpStep && a->T != 1) return fail(GDR_E_SHAPE, "the recurrent step needs T == 1 (got %d)", a->T);
  const int chunk = a->chunk ? a->chunk : GDR_CHUNK;
  if (chunk != GDR_CHUNK) return fail(GDR_E_SHAPE, "chunk must be 64 (got %d)", a->chunk);
  if (a->dk < 1 || a->dv < 1) return fail(GDR_E_SHAPE, "need dk, dv >= 1 (got %d, %d)", a->dk, a->dv);
  if (a->io != GDR_F32 && a->io != GDR_BF16) return fail(GDR_E_DTYPE, "unknown io dtype %d", a->io);
  if (a->decay < GDR_DECAY_NONE || a->decay > GDR_DECAY_CHANNEL)
    return fail(GDR_E_ARGS, "unknown decay kind %d", a->decay);
  if (a->erase < GDR_GATE_BETA || a->erase > GDR_GATE_VALUE)
    return fail(GDR_E_ARGS, "unknown erase kind %d", a->erase);
  if (a->write < GDR_GATE_BETA || a->write > GDR_GATE_VALUE)
    return fail(GDR_E_ARGS, "unknown write kind %d", a->write);
  if ((a->erase == GDR_GATE_VALUE) != (a->write == GDR_GATE_VALUE))
    return fail(GDR_E_ARGS, "the per-value-channel beta gates erase and write together: both kinds must be VALUE");
  if (a->qmix < 0 || a->qmix > 2) return fail(GDR_E_ARGS, "qmix must be 0, 1 or 2 (got %d)", a->qmix);
  if (a->qmix && a->erase != GDR_GATE_BETA)
    return fail(GDR_E_ARGS, "qmix mixes the query into the beta-gated erase direction; erase must be BETA");
  const int64_t BH = int64_t(a->B) * a->H;
  const int64_t tokens = BH * a->T;
  const int64_t dmax = a->dk > a->dv ? a->dk : a->dv;
  // Kernels address a sequence with 32-bit element offsets (T * H * d) and a
  // chunk's rows with 32-bit byte offsets (up to 64 rows of H * d fp32).
  if (BH > (int64_t(1) << 30) || tokens * dmax > (int64_t(1) << 46) ||
      int64_t(a->T) * a->H * dmax >= (int64_t(1) << 31) || int64_t(a->H) * dmax * 4 * 64 >= (int64_t(1) << 32))
    return fail(GDR_E_SHAPE, "problem too large (need T * H * max(dk, dv) < 2^31 and H * max(dk, dv) < 2^24)");

  const bool has_tok = a->T > 0;
  const bool need_beta = a->erase != GDR_GATE_CHANNEL || a->write != GDR_GATE_CHANNEL;
  if (check_ptrs && has_tok) {
    if (!a->q || !a->k || !a->v || !a->o) return fail(GDR_E_NULL, "q, k, v and o are required when T > 0");
    if (a->decay != GDR_DECAY_NONE && !a->g) return fail(GDR_E_NULL, "g is required for decay kind %d", a->decay);
    if (need_beta && !a->beta) return fail(GDR_E_NULL, "beta is required by a BETA gate");
    if (a->erase == GDR_GATE_CHANNEL && !a->b) return fail(GDR_E_NULL, "b is required by erase CHANNEL");
    if (a->write == GDR_GATE_CHANNEL && !a->w) return fail(GDR_E_NULL, "w is required by write CHANNEL");
    if (a->qmix && !a->lambda) return fail(GDR_E_NULL, "lambda is required by qmix");
  }
  if (a->decay == GDR_DECAY_NONE && a->g) return fail(GDR_E_ARGS, "g given with decay NONE");
  const Epilogue epi = epilogue_of(a);
  if (check_ptrs && epi.gate && !epi.weight) return fail(GDR_E_NULL, "norm_weight is required with out_gate");

  if (check_ptrs) {
    // alignment
    const void* al16[] = {a->q, a->k, a->v, a->o, a->state_in, a->state_out, a->b, a->w,
                          a->decay == GDR_DECAY_CHANNEL ? a->g : nullptr};
    for (const void* p : al16)
      if (p && !aligned(p, 16)) return fail(GDR_E_ALIGN, "a tensor pointer is not 16-byte aligned");
    if (epi.gate && !aligned(epi.gate, 16)) return fail(GDR_E_ALIGN, "out_gate is not 16-byte aligned");
    const void* al4[] = {a->beta, a->lambda, a->g, epi.weight};
    for (const void* p : al4)
      if (p && !aligned(p, 4)) return fail(GDR_E_ALIGN, "a gate pointer is not 4-byte aligned");

    // aliasing
    const int64_t ioe = a->io == GDR_BF16 ? 2 : 4;
    const int64_t gsz = a->decay == GDR_DECAY_CHANNEL ? tokens * a->dk * 4 : tokens * 4;
    const Range ins[] = {rng("q", a->q, tokens * a->dk * ioe),     rng("k", a->k, tokens * a->dk * ioe),
                         rng("v", a->v, tokens * a->dv * ioe),     rng("g", a->g, gsz),
                         rng("beta", a->beta, beta_bytes(a)),      rng("b", a->b, tokens * a->dk * 4),
                         rng("w", a->w, tokens * a->dv * 4),       rng("lambda", a->lambda, lambda_bytes(a)),
                         rng("state_in", a->state_in, BH * a->dk * a->dv * 4),
                         rng("out_gate", epi.gate, tokens * a->dv * ioe),
                         rng("norm_weight", epi.weight, int64_t(a->dv) * 4)};
    const Range ro = rng("o", a->o, tokens * a->dv * ioe);
    const Range rs = rng("state_out", a->state_out, BH * a->dk * a->dv * 4);
    for (const Range& r : ins) {
      if (overlap(ro, r)) return fail(GDR_E_ARGS, "o overlaps input %s", r.name);
      const bool same_state = (r.name[0] == 's') && r.lo == rs.lo;
      if (!same_state && overlap(rs, r)) return fail(GDR_E_ARGS, "state_out overlaps input %s", r.name);
    }
    if (overlap(ro, rs)) return fail(GDR_E_ARGS, "o overlaps state_out");
  }

  // what the library implements
  if (op == kOpChunk) {
    if (a->io == GDR_BF16 && a->dk != 64 && a->dk != 128)
      return fail(GDR_E_UNSUPPORTED, "bf16 chunk path supports dk in {64, 128} (got %d)", a->dk);
    if (a->io == GDR_F32 && a->dk != 64 && a->dk != 128)
      return fail(GDR_E_UNSUPPORTED, "fp32 chunk path supports dk in {64, 128} (got %d)", a->dk);
    if (a->dv % 16 != 0 || a->dv > 256)
      return fail(GDR_E_UNSUPPORTED, "dv must be a multiple of 16 up to 256 (got %d)", a->dv);
    int cand[3];
    const int nc = dvs_candidates(a, cand);
    if (a->dv_split) {
      bool ok = false;
      for (int i = 0; i < nc; ++i) ok |= cand[i] == a->dv_split;
      if (!ok || a->dv % a->dv_split != 0)
        return fail(GDR_E_UNSUPPORTED, "dv_split %d is not an available slice width dividing dv=%d",
                    a->dv_split, a->dv);
    } else {
      bool ok = false;
      for (int i = 0; i < nc; ++i) ok |= (a->dv % cand[i] == 0);
      if (!ok) return fail(GDR_E_UNSUPPORTED, "no slice width divides dv=%d", a->dv);
    }
    if (epi.gate && !gdr::norm_gate_supported(a->dv))
      return fail(GDR_E_UNSUPPORTED, "the chunk path's output epilogue needs dv in {64, 128, 256} (got %d)", a->dv);
  } else if (op == kOpStep) {
    if (!gdr::step_supported(a->dk, a->dv))
      return fail(GDR_E_UNSUPPORTED, "recurrent step supports dk, dv in {64, 128} (got %d, %d)", a->dk, a->dv);
  } else {
    if (!gdr::recur_supported(a->dk, a->dv))
      return fail(GDR_E_UNSUPPORTED, "the recurrent form supports dk, dv in {64, 128} (got %d, %d)", a->dk, a->dv);
  }
  return GDR_OK;
}

gdr_status plan_impl(const gdr_args* a, int op, gdr_plan_info* out, Workspace ws) {
  const int64_t BH = int64_t(a->B) * a->H;
  gdr_plan_info pi{};
  pi.block = 256;
  pi.passes = 1;
  if (op == kOpStep) {
    pi.grid = static_cast<int32_t>(BH);
    pi.dv_slice = a->dv;
    pi.lds_bytes = 0;
    pi.n_chunks = 1;
  } else if (op == kOpRecur) {
    // one workgroup of dv threads per (batch, head); 8 tokens staged in LDS
    pi.grid = static_cast<int32_t>(BH);
    pi.block = a->dv;
    pi.dv_slice = a->dv;
    pi.lds_bytes = 4 * 8 * a->dk * 4 + 8 * (a->dv / 64) * 4 + 3 * 8 * a->dv * 4;
    pi.n_chunks = 0;
  } else {
    int cand[3];
    const int nc = dvs_candidates(a, cand);
    int dvs = a->dv_split;
    if (!dvs) {
      for (int i = 0; i < nc && !dvs; ++i)
        if (a->dv % cand[i] == 0 && BH * (a->dv / cand[i]) >= 256) dvs = cand[i];
      for (int i = nc - 1; i >= 0 && !dvs; --i)
        if (a->dv % cand[i] == 0) dvs = cand[i];
    }
    pi.dv_slice = dvs;
    pi.grid = static_cast<int32_t>(BH * (a->dv / dvs));
    pi.n_chunks = (a->T + GDR_CHUNK - 1) / GDR_CHUNK;
    const int64_t need = split_bytes(a, dvs);
    if (need > 0 && ws.ptr && ws.bytes >= static_cast<uint64_t>(need)) {
      pi.passes = 2;
      const gdr::ChunkKernel kern = kernel_for(a);
      const int gm = gdr::gate_mode(a->erase, a->write);
      if (kern == gdr::kPlain) {
        // the two-pass plain form picks its own slice width
        pi.dv_slice = gdr::plain_split_slice(a->erase, a->dv, a->dv_split);
        pi.grid = static_cast<int32_t>(BH * (a->dv / pi.dv_slice));
        pi.lds_bytes = gdr::plain_split_lds(a->dk, pi.dv_slice);
        pi.block = 256;
      } else {
        pi.lds_bytes = kern == gdr::kChan ? gdr::chan_split_lds(gm, a->dk, dvs) : gdr::pipe_split_lds(gm, a->dk, dvs);
        pi.block = 64 * ((dvs >= 32 ? 2 : 1) + 4);
      }
    } else {
      pi.passes = 1;
      pi.lds_bytes = chunk_lds(a, dvs);
      pi.block = chunk_block(a, dvs);
    }
    if (pi.lds_bytes < 0)
      return fail(GDR_E_UNSUPPORTED, "no kernel instance for io=%d dk=%d slice=%d", a->io, a->dk, dvs);
  }
  if (out) *out = pi;
  return GDR_OK;
}

gdr_status plan_impl(const gdr_args* a, int op, gdr_plan_info* out) {
  return plan_impl(a, op, out, workspace_of(a));
}

// The body of the chunk entry points: validation, plan and launch, with the
// workspace given explicitly (the caller's, or the library's static scratch).
gdr_status chunk_fwd_impl(const gdr_args* a, void* stream, Workspace ws, bool check_ws);

// the output epilogue of a chunk call: a second kernel over o, in place
gdr_status chunk_epilogue(const gdr_args* a, hipStream_t st) {
  const Epilogue epi = epilogue_of(a);
  if (!epi.gate || a->T == 0) return GDR_OK;
  const hipError_t e = gdr::launch_norm_gate(a->o, epi.gate, epi.weight, a->o, int64_t(a->B) * a->T * a->H, a->dv,
                                             a->io == GDR_BF16, epi.eps, st);
  if (e != hipSuccess) return fail(GDR_E_HIP, "output epilogue launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

// ---- scratch of the no-allocation entry point ------------------------------
// Device memory of the two-pass records for callers that cannot allocate.
// Every device the library runs on holds its own copy of this array until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address on the current device comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch.
constexpr uint64_t kScratchBytes = GDR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

gdr_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDR_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_E_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GDR_E_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_validate(const gdr_args* a, int op) { return validate_impl(a, op); }

gdr_status gdr_plan(const gdr_args* a, int op, gdr_plan_info* out) {
  gdr_status s = validate_impl(a, op, /*check_ptrs=*/false);
  if (s != GDR_OK) return s;
  return plan_impl(a, op, out);
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_args* a, void* stream) {
  gdr_status s = validate_impl(a, kOpChunk);
  if (s != GDR_OK) return s;
  // the plan as it would be with a workspace of unlimited size
  gdr_plan_info pi;
  s = plan_impl(a, kOpChunk, &pi);
  if (s != GDR_OK) return s;
  int64_t need = split_bytes(a, pi.dv_slice);
  // the plain kernel has a single-pass form that needs no records
  if (need > static_cast<int64_t>(kScratchBytes) && kernel_for(a) == gdr::kPlain) need = 0;
  if (need > static_cast<int64_t>(kScratchBytes))
    return fail(GDR_E_SHAPE,
                "the two-pass records of this call need %lld bytes; the no-allocation entry point's scratch "
                "holds %llu (use gdr_chunk_fwd with a caller workspace)",
                static_cast<long long>(need), static_cast<unsigned long long>(kScratchBytes));
  if (need == 0) return chunk_fwd_impl(a, stream, Workspace{nullptr, 0}, false);
  void* ptr = nullptr;
  s = scratch_ptr(&ptr);
  if (s != GDR_OK) return s;
  return chunk_fwd_impl(a, stream, Workspace{ptr, kScratchBytes}, false);
}

gdr_status gdr_workspace_size(const gdr_args* a, uint64_t* bytes) {
  if (!bytes) return fail(GDR_E_NULL, "bytes pointer is NULL");
  *bytes = 0;
  gdr_status s = validate_impl(a, kOpChunk, /*check_ptrs=*/false);
  if (s != GDR_OK) return s;
  gdr_plan_info pi;
  s = plan_impl(a, kOpChunk, &pi);
  if (s != GDR_OK) return s;
  *bytes = static_cast<uint64_t>(split_bytes(a, pi.dv_slice));
  return GDR_OK;
}

gdr_status gdr_chunk_fwd(const gdr_args* a, void* stream) {
  gdr_status s = validate_impl(a, kOpChunk);
  if (s != GDR_OK) return s;
  return chunk_fwd_impl(a, stream, workspace_of(a), true);
}

}  // extern "C"

namespace {

gdr_status chunk_fwd_impl(const gdr_args* a, void* stream, Workspace ws, bool check_ws) {
  gdr_plan_info pi;
  gdr_status s = plan_impl(a, kOpChunk, &pi, ws);
  if (s != GDR_OK) return s;
  if (a->T == 0 && !a->state_out) return GDR_OK;
  if (pi.passes == 2 && check_ws) {
    // the workspace of the two-pass form: aligned, and apart from every
    // other buffer of the call
    if (!aligned(ws.ptr, 256)) return fail(GDR_E_ALIGN, "workspace is not 256-byte aligned");
    const int64_t tokens = int64_t(a->B) * a->H * a->T;
    const int64_t BH = int64_t(a->B) * a->H;
    const int64_t ioe = a->io == GDR_BF16 ? 2 : 4;
    const Range rw = rng("workspace", ws.ptr, static_cast<int64_t>(ws.bytes));
    const Range others[] = {rng("q", a->q, tokens * a->dk * ioe),    rng("k", a->k, tokens * a->dk * ioe),
                            rng("v", a->v, tokens * a->dv * ioe),    rng("o", a->o, tokens * a->dv * ioe),
                            rng("g", a->g, a->decay == GDR_DECAY_CHANNEL ? tokens * a->dk * 4 : tokens * 4),
                            rng("beta", a->beta, beta_bytes(a)),
                            rng("b", a->b, tokens * a->dk * 4),      rng("w", a->w, tokens * a->dv * 4),
                            rng("lambda", a->lambda, lambda_bytes(a)),
                            rng("state_in", a->state_in, BH * a->dk * a->dv * 4),
                            rng("state_out", a->state_out, BH * a->dk * a->dv * 4)};
    for (const Range& r : others)
      if (overlap(rw, r)) return fail(GDR_E_ARGS, "workspace overlaps %s", r.name);
  }
  gdr::ChunkParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.g = a->g; p.beta = a->beta; p.b = a->b; p.w = a->w; p.lam = a->lambda;
  p.state_in = a->state_in; p.state_out = a->state_out; p.o = a->o;
  p.B = a->B; p.T = a->T; p.H = a->H; p.DV = a->dv;
  p.decay = a->decay; p.erase = a->erase; p.write = a->write; p.qmix = a->qmix;
  p.nslices = a->dv / pi.dv_slice;
  const bool chan = a->decay == GDR_DECAY_CHANNEL;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int gm = gdr::gate_mode(a->erase, a->write);
  hipError_t e;
  if (pi.passes == 2) {
    const int prep_grid = static_cast<int>(int64_t(a->B) * a->H * pi.n_chunks);
    p.ws = ws.ptr;
    const gdr::ChunkKernel kern = kernel_for(a);
    if (kern == gdr::kPlain) {
      gdr::BwdWs rec;
      gdr::plain_split_layout(prep_grid, a->dk, static_cast<char*>(ws.ptr), &rec);
      e = gdr::launch_plain_split(p, rec, a->io == GDR_BF16, a->dk, pi.dv_slice, pi.grid, prep_grid, st);
    } else if (kern == gdr::kChan) {
      e = gdr::launch_chan_split(gm, p, ws.ptr, a->dk, pi.dv_slice, pi.grid, prep_grid, st);
    } else {
      e = gdr::launch_pipe_split(gm, p, a->dk, pi.dv_slice, pi.grid, prep_grid, st);
    }
    if (e != hipSuccess) return fail(GDR_E_HIP, "two-pass chunk kernels failed to launch: %s", hipGetErrorString(e));
    return chunk_epilogue(a, st);
  }
  switch (kernel_for(a)) {
    case gdr::kPipe: e = gdr::launch_pipe(gm, p, a->dk, pi.dv_slice, pi.grid, st); break;
    case gdr::kChan: e = gdr::launch_chan(gm, p, a->dk, pi.dv_slice, pi.grid, st); break;
    case gdr::kPlain: e = gdr::launch_plain(p, a->io == GDR_BF16, a->dk, pi.grid, st); break;
    default: e = gdr::launch_chunk(a->io == GDR_BF16, gm, p, a->dk, pi.dv_slice, chan, pi.grid, st); break;
  }
  if (e != hipSuccess) return fail(GDR_E_HIP, "chunk kernel launch failed: %s", hipGetErrorString(e));
  return chunk_epilogue(a, st);
}

}  // namespace

extern "C" {

gdr_status gdr_recurrent_step(const gdr_args* a, void* stream) {
  gdr_status s = validate_impl(a, kOpStep);
  if (s != GDR_OK) return s;
  gdr::StepParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.g = a->g; p.beta = a->beta; p.b = a->b; p.w = a->w; p.lam = a->lambda;
  p.state_in = a->state_in; p.state_out = a->state_out; p.o = a->o;
  const Epilogue epi = epilogue_of(a);
  p.gate = epi.gate; p.nw = epi.weight; p.eps = epi.eps;
  p.B = a->B; p.H = a->H;
  p.decay = a->decay; p.erase = a->erase; p.write = a->write; p.qmix = a->qmix;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdr::launch_step(p, a->io == GDR_BF16, a->dk, a->dv, a->B * a->H, st);
  if (e != hipSuccess) return fail(GDR_E_HIP, "step kernel launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

gdr_status gdr_recurrent_fwd(const gdr_args* a, void* stream) {
  gdr_status s = validate_impl(a, kOpRecur);
  if (s != GDR_OK) return s;
  if (a->T == 0 && !a->state_out) return GDR_OK;
  gdr::RecurParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v;
  p.g = a->g; p.beta = a->beta; p.b = a->b; p.w = a->w; p.lam = a->lambda;
  p.state_in = a->state_in; p.state_out = a->state_out; p.o = a->o;
  const Epilogue epi = epilogue_of(a);
  p.gate = epi.gate; p.nw = epi.weight; p.eps = epi.eps;
  p.B = a->B; p.T = a->T; p.H = a->H;
  p.decay = a->decay; p.erase = a->erase; p.write = a->write; p.qmix = a->qmix;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdr::launch_recur(p, a->io == GDR_BF16, a->dk, a->dv, a->B * a->H, st);
  if (e != hipSuccess) return fail(GDR_E_HIP, "recurrent kernel launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

}  // extern "C"

namespace {

// the backward's workspace: fp32 arrays at 256-byte aligned offsets
struct BwdLayout {
  int64_t S, W, dR, dS, T, A, Eb, Qg, Kt, gC, dlam, total;
};
BwdLayout bwd_layout(const gdr_args* f) {
  const int64_t BH = int64_t(f->B) * f->H, N = (f->T + GDR_CHUNK - 1) / GDR_CHUNK, NC = BH * N;
  const int64_t dk = f->dk, dv = f->dv, C = GDR_CHUNK;
  BwdLayout l{};
  int64_t off = 0;
  auto take = [&](int64_t floats) {
    const int64_t o = off;
    off += (floats * 4 + 255) / 256 * 256;
    return o;
  };
  l.S = take(NC * dk * dv);
  l.W = take(NC * C * dv);
  l.dR = take(NC * C * dv);
  l.dS = take(NC * dk * dv);
  l.T = take(NC * C * C);
  l.A = take(NC * C * C);
  l.Eb = take(NC * C * dk);
  l.Qg = take(NC * C * dk);
  l.Kt = take(NC * C * dk);
  l.gC = take(NC * dk);
  l.dlam = take(f->qmix == 1 ? BH * f->T : 0);
  l.total = off;
  return l;
}

gdr_status bwd_validate(const gdr_bwd_args* a, bool check_ptrs, gdr_args* fcopy) {
  if (!a) return fail(GDR_E_NULL, "gdr_bwd_args pointer is NULL");
  if (a->struct_size < sizeof(gdr_bwd_args))
    return fail(GDR_E_ARGS, "struct_size %u is smaller than gdr_bwd_args (%zu bytes)", a->struct_size,
                sizeof(gdr_bwd_args));
  if (!a->fwd) return fail(GDR_E_NULL, "fwd (the forward's arguments) is NULL");
  if (a->fwd->struct_size < kArgsV1Size) return fail(GDR_E_ARGS, "fwd: struct_size too small");
  // the forward's checks, with d_o in the place of o; no state_out, workspace or epilogue
  gdr_args f{};
  std::memcpy(&f, a->fwd, a->fwd->struct_size < sizeof(gdr_args) ? a->fwd->struct_size : sizeof(gdr_args));
  f.struct_size = sizeof(gdr_args);
  f.o = const_cast<void*>(a->d_o);
  f.state_out = nullptr;
  f.workspace = nullptr;
  f.workspace_bytes = 0;
  f.out_gate = nullptr;
  f.norm_weight = nullptr;
  f.dv_split = 0;
  gdr_status s = validate_impl(&f, kOpChunk, check_ptrs);
  if (s != GDR_OK) return s;
  if (!gdr::bwd_supported(f.dk, f.dv))
    return fail(GDR_E_UNSUPPORTED, "the backward supports dk, dv in {64, 128} (got %d, %d)", f.dk, f.dv);
  if (f.erase == GDR_GATE_VALUE)
    return fail(GDR_E_UNSUPPORTED, "the backward does not implement the per-value-channel beta");
  *fcopy = f;
  if (!check_ptrs) return GDR_OK;
  const int64_t tokens = int64_t(f.B) * f.H * f.T, BH = int64_t(f.B) * f.H;
  const bool has_tok = f.T > 0;
  const bool need_beta = f.erase == GDR_GATE_BETA || f.write == GDR_GATE_BETA;
  if (has_tok) {
    if (!a->dq || !a->dk || !a->dv) return fail(GDR_E_NULL, "dq, dk and dv are required when T > 0");
    if (f.decay != GDR_DECAY_NONE && !a->dg) return fail(GDR_E_NULL, "dg is required with a decay");
    if (need_beta && !a->dbeta) return fail(GDR_E_NULL, "dbeta is required by a BETA gate");
    if (f.erase == GDR_GATE_CHANNEL && !a->db) return fail(GDR_E_NULL, "db is required by erase CHANNEL");
    if (f.write == GDR_GATE_CHANNEL && !a->dw) return fail(GDR_E_NULL, "dw is required by write CHANNEL");
  }
  if (f.qmix && !a->dlam) return fail(GDR_E_NULL, "dlam is required by qmix");
  const void* al4[] = {a->dq, a->dk, a->dv, a->dg, a->dbeta, a->db, a->dw, a->dlam, a->dstate, a->d_state};
  for (const void* p : al4)
    if (p && !aligned(p, 4)) return fail(GDR_E_ALIGN, "a gradient pointer is not 4-byte aligned");
  if (a->d_state && !aligned(a->d_state, 16)) return fail(GDR_E_ALIGN, "d_state is not 16-byte aligned");
  const BwdLayout l = bwd_layout(&f);
  if (has_tok) {
    if (!a->workspace || a->workspace_bytes < static_cast<uint64_t>(l.total))
      return fail(GDR_E_ARGS, "the backward needs a workspace of %lld bytes", static_cast<long long>(l.total));
    if (!aligned(a->workspace, 256)) return fail(GDR_E_ALIGN, "workspace is not 256-byte aligned");
  }
  const int64_t ioe = f.io == GDR_BF16 ? 2 : 4;
  const int64_t gsz = f.decay == GDR_DECAY_CHANNEL ? tokens * f.dk * 4 : tokens * 4;
  const Range ins[] = {rng("q", f.q, tokens * f.dk * ioe),      rng("k", f.k, tokens * f.dk * ioe),
                       rng("v", f.v, tokens * f.dv * ioe),      rng("g", f.g, gsz),
                       rng("beta", f.beta, beta_bytes(&f)),     rng("b", f.b, tokens * f.dk * 4),
                       rng("w", f.w, tokens * f.dv * 4),        rng("lambda", f.lambda, lambda_bytes(&f)),
                       rng("state_in", f.state_in, BH * f.dk * f.dv * 4),
                       rng("d_o", a->d_o, tokens * f.dv * ioe), rng("d_state", a->d_state, BH * f.dk * f.dv * 4)};
  const Range outs[] = {rng("dq", a->dq, tokens * f.dk * 4),    rng("dk", a->dk, tokens * f.dk * 4),
                        rng("dv", a->dv, tokens * f.dv * 4),    rng("dg", a->dg, gsz),
                        rng("dbeta", a->dbeta, tokens * 4),     rng("db", a->db, tokens * f.dk * 4),
                        rng("dw", a->dw, tokens * f.dv * 4),    rng("dlam", a->dlam, lambda_bytes(&f)),
                        rng("dstate", a->dstate, BH * f.dk * f.dv * 4),
                        rng("workspace", a->workspace, has_tok ? l.total : 0)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(GDR_E_ARGS, "%s overlaps input %s", outs[i].name, r.name);
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return fail(GDR_E_ARGS, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_bwd_workspace_size(const gdr_bwd_args* a, uint64_t* bytes) {
  if (!bytes) return fail(GDR_E_NULL, "bytes pointer is NULL");
  *bytes = 0;
  gdr_args f;
  gdr_status s = bwd_validate(a, false, &f);
  if (s != GDR_OK) return s;
  *bytes = f.T > 0 ? static_cast<uint64_t>(bwd_layout(&f).total) : 0;
  return GDR_OK;
}

gdr_status gdr_chunk_bwd(const gdr_bwd_args* a, void* stream) {
  gdr_args f;
  gdr_status s = bwd_validate(a, true, &f);
  if (s != GDR_OK) return s;
  gdr::BwdParams p{};
  p.f.q = f.q; p.f.k = f.k; p.f.v = f.v;
  p.f.g = f.g; p.f.beta = f.beta; p.f.b = f.b; p.f.w = f.w; p.f.lam = f.lambda;
  p.f.state_in = f.state_in; p.f.state_out = nullptr; p.f.o = nullptr;
  p.f.B = f.B; p.f.T = f.T; p.f.H = f.H; p.f.DV = f.dv;
  p.f.decay = f.decay; p.f.erase = f.erase; p.f.write = f.write; p.f.qmix = f.qmix;
  p.f.nslices = f.dv / 16;
  p.d_o = a->d_o;
  p.d_st = a->d_state;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv; p.dg = a->dg; p.dbeta = a->dbeta; p.db = a->db; p.dw = a->dw;
  p.dlam = a->dlam; p.dstate = a->dstate;
  p.nchunks = (f.T + GDR_CHUNK - 1) / GDR_CHUNK;
  if (f.T > 0) {
    const BwdLayout l = bwd_layout(&f);
    char* base = static_cast<char*>(a->workspace);
    auto at = [&](int64_t off) { return reinterpret_cast<float*>(base + off); };
    p.ws = gdr::BwdWs{at(l.S), at(l.W), at(l.dR), at(l.dS), at(l.T), at(l.A), at(l.Eb), at(l.Qg), at(l.Kt),
                      at(l.gC), at(l.dlam)};
  }
  if (!a->dstate && p.nchunks == 0 && f.qmix != 1) return GDR_OK;
  const hipError_t e = gdr::launch_bwd(p, f.io == GDR_BF16, f.dk, f.dv, f.B * f.H,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_E_HIP, "backward kernels failed to launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

gdr_status gdr_output_norm_gate(const gdr_norm_args* a, void* stream) {
  if (!a) return fail(GDR_E_NULL, "gdr_norm_args pointer is NULL");
  if (a->struct_size < sizeof(gdr_norm_args))
    return fail(GDR_E_ARGS, "struct_size %u is smaller than gdr_norm_args (%zu bytes)", a->struct_size,
                sizeof(gdr_norm_args));
  if (a->io != GDR_F32 && a->io != GDR_BF16) return fail(GDR_E_DTYPE, "unknown io dtype %d", a->io);
  if (a->rows < 0 || a->rows > (int64_t(1) << 40)) return fail(GDR_E_SHAPE, "rows out of range (%lld)",
                                                                static_cast<long long>(a->rows));
  if (!gdr::norm_gate_supported(a->dv)) return fail(GDR_E_UNSUPPORTED, "dv must be 64, 128 or 256 (got %d)", a->dv);
  if (a->rows == 0) return GDR_OK;
  if (!a->o || !a->gate || !a->weight || !a->y) return fail(GDR_E_NULL, "o, gate, weight and y are required");
  if (!aligned(a->o, 16) || !aligned(a->gate, 16) || !aligned(a->y, 16) || !aligned(a->weight, 4))
    return fail(GDR_E_ALIGN, "o, gate and y must be 16-byte aligned, weight 4-byte aligned");
  const int64_t bytes = a->rows * a->dv * (a->io == GDR_BF16 ? 2 : 4);
  const Range ry = rng("y", a->y, bytes);
  const Range ro = rng("o", a->o, bytes), rg = rng("gate", a->gate, bytes), rw = rng("weight", a->weight, a->dv * 4);
  if ((overlap(ry, ro) && ry.lo != ro.lo) || overlap(ry, rg) || overlap(ry, rw))
    return fail(GDR_E_ARGS, "y overlaps an input (only y == o exactly is allowed)");
  const float eps = a->eps > 0.f ? a->eps : kDefaultEps;
  const hipError_t e = gdr::launch_norm_gate(a->o, a->gate, a->weight, a->y, a->rows, a->dv, a->io == GDR_BF16, eps,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_E_HIP, "output epilogue launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

const char* gdr_status_str(gdr_status s) {
  // any int may arrive through the C ABI: read it as an int, not as the enum
  // (a value outside the enumerators is not a valid gdr_status in C++)
  int v;
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case GDR_OK: return "GDR_OK";
    case GDR_E_NULL: return "GDR_E_NULL";
    case GDR_E_SHAPE: return "GDR_E_SHAPE";
    case GDR_E_DTYPE: return "GDR_E_DTYPE";
    case GDR_E_ALIGN: return "GDR_E_ALIGN";
    case GDR_E_UNSUPPORTED: return "GDR_E_UNSUPPORTED";
    case GDR_E_HIP: return "GDR_E_HIP";
    case GDR_E_ARGS: return "GDR_E_ARGS";
  }
  return "GDR_E_UNKNOWN";
}

const char* gdr_last_error(void) { return g_err.c_str(); }

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

}  // extern "C"
