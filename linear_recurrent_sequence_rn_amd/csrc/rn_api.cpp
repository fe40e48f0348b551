// C ABI of the retention library: host-side validation and kernel dispatch.
// Every argument is checked before the first HIP call, so an invalid call launches
// nothing; failures return a status and leave a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "rn_kernels.h"
#include "rn_retention.h"

namespace {

thread_local char g_err[512] = "";

rn_status fail(rn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

rn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return RN_OK;
  return fail(RN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

enum class Form { kParallel, kChunkwise, kStep };

constexpr uint32_t kKnownFlags = RN_NORM_D_ROW | RN_NORM_R_ROW | RN_EPI_GN | RN_EPI_GATE |
                                 RN_FORCE_GENERIC | RN_CHUNK_PARALLEL | RN_CHUNK_SEGMENTED |
                                 RN_TEST_FORCE_TIMEOUT;

bool dtype_ok(rn_dtype d) { return d == RN_F32 || d == RN_BF16; }

// Validates a descriptor for one form; fills the kernel argument block.
rn_status check_desc(const rn_desc* d, Form form, rn::CallArgs* a) {
  if (!d) return fail(RN_ERR_INVALID_ARG, "desc is NULL");
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->d_k < 1 || d->d_v < 1)
    return fail(RN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d N=%d d_k=%d d_v=%d)", d->B,
                d->H, d->N, d->d_k, d->d_v);
  if (d->d_k % 2) return fail(RN_ERR_INVALID_ARG, "d_k=%d must be even (coordinate pairs)", d->d_k);
  if (d->d_k > rn::kMaxDk) return fail(RN_ERR_UNSUPPORTED, "d_k=%d > %d", d->d_k, rn::kMaxDk);
  if (d->d_v > rn::kMaxDv) return fail(RN_ERR_UNSUPPORTED, "d_v=%d > %d", d->d_v, rn::kMaxDv);
  if (d->H > rn::kMaxHeads) return fail(RN_ERR_UNSUPPORTED, "H=%d > %d", d->H, rn::kMaxHeads);
  if (d->B > 65535) return fail(RN_ERR_UNSUPPORTED, "B=%d > 65535", d->B);
  if (d->N > (1 << 30)) return fail(RN_ERR_UNSUPPORTED, "N=%d > 2^30", d->N);
  if (form == Form::kStep && d->N != 1)
    return fail(RN_ERR_INVALID_ARG, "recurrent step needs N == 1 (got %d)", d->N);
  if (!dtype_ok(d->in_dtype) || !dtype_ok(d->out_dtype))
    return fail(RN_ERR_INVALID_ARG, "unknown dtype (in=%d out=%d)", d->in_dtype, d->out_dtype);
  if (d->flags & ~kKnownFlags) return fail(RN_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  if ((d->flags & RN_CHUNK_PARALLEL) && (d->flags & RN_CHUNK_SEGMENTED))
    return fail(RN_ERR_INVALID_ARG, "RN_CHUNK_PARALLEL and RN_CHUNK_SEGMENTED are exclusive");
  if ((d->flags & RN_EPI_GATE) && !(d->flags & RN_EPI_GN))
    return fail(RN_ERR_INVALID_ARG, "RN_EPI_GATE requires RN_EPI_GN");
  if (form != Form::kParallel && (d->flags & (RN_NORM_D_ROW | RN_NORM_R_ROW)))
    return fail(RN_ERR_INVALID_ARG, "row rescalings apply to the parallel form only");
  if (d->pos0 < 0 || d->pos0 > (int64_t(1) << 40))
    return fail(RN_ERR_INVALID_ARG, "pos0=%lld outside [0, 2^40]", (long long)d->pos0);
  if (!std::isfinite(d->qk_scale)) return fail(RN_ERR_INVALID_ARG, "qk_scale is not finite");
  if ((d->flags & RN_EPI_GN) && !(d->gn_eps >= 0.f && std::isfinite(d->gn_eps)))
    return fail(RN_ERR_INVALID_ARG, "gn_eps must be finite and >= 0");
  if (!d->theta) return fail(RN_ERR_INVALID_ARG, "theta is NULL");
  std::memset(a, 0, sizeof(*a));
  if (d->gamma_pair) {
    // one decay per (head, pair), read by the kernels from device memory
    if (reinterpret_cast<uintptr_t>(d->gamma_pair) % alignof(float))
      return fail(RN_ERR_INVALID_ARG, "gamma_pair must be 4-byte aligned");
    if (d->flags & RN_NORM_D_ROW)
      return fail(RN_ERR_INVALID_ARG, "RN_NORM_D_ROW is defined by a scalar decay; not with gamma_pair");
    a->gpair = d->gamma_pair;
  } else {
    if (!d->gamma) return fail(RN_ERR_INVALID_ARG, "gamma is NULL");
    for (int h = 0; h < d->H; ++h) {
      const float g = d->gamma[h];
      if (!(g > 0.f && g <= 1.f)) return fail(RN_ERR_INVALID_ARG, "gamma[%d]=%g not in (0, 1]", h, g);
      a->hp.gamma[h] = g;
      a->hp.log2g[h] = static_cast<float>(std::log2(static_cast<double>(g)));
    }
  }
  for (int j = 0; j < d->d_k / 2; ++j) {
    if (!std::isfinite(d->theta[j])) return fail(RN_ERR_INVALID_ARG, "theta[%d] is not finite", j);
    a->ap.theta[j] = d->theta[j];
  }
  a->B = d->B; a->H = d->H; a->N = d->N; a->dk = d->d_k; a->dv = d->d_v;
  a->pos0 = d->pos0;
  a->alpha = d->qk_scale;
  a->eps = d->gn_eps;
  a->flags = d->flags;
  a->gn_w = d->gn_weight;
  a->gn_b = d->gn_bias;
  return RN_OK;
}

rn_status check_ptrs(const rn_desc* d, const void* q, const void* k, const void* v,
                     const void* gate, const void* out) {
  if (!q || !k || !v || !out) return fail(RN_ERR_INVALID_ARG, "q/k/v/out pointer is NULL");
  if ((d->flags & RN_EPI_GATE) && !gate) return fail(RN_ERR_INVALID_ARG, "RN_EPI_GATE needs a gate");
  return RN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Device arrays of the serving entry points: only their alignment can be checked on
// the host; their values are read by the kernels.
rn_status check_seq_arrays(const int64_t* pos, const int32_t* lengths, rn::CallArgs* a) {
  if (reinterpret_cast<uintptr_t>(pos) % alignof(int64_t))
    return fail(RN_ERR_INVALID_ARG, "pos must be 8-byte aligned");
  if (reinterpret_cast<uintptr_t>(lengths) % alignof(int32_t))
    return fail(RN_ERR_INVALID_ARG, "lengths must be 4-byte aligned");
  a->pos = pos;
  a->lens = lengths;
  return RN_OK;
}

size_t generic_ws_bytes(const rn_desc* d) {
  return align256(size_t(d->B) * d->H * d->d_k * d->d_v * sizeof(float));
}

}  // namespace

extern "C" {

const char* rn_version(void) { return "0.1.0"; }

const char* rn_last_error(void) { return g_err; }

const char* rn_status_str(rn_status s) {
  switch (s) {
    case RN_OK: return "RN_OK";
    case RN_ERR_INVALID_ARG: return "RN_ERR_INVALID_ARG";
    case RN_ERR_UNSUPPORTED: return "RN_ERR_UNSUPPORTED";
    case RN_ERR_HIP: return "RN_ERR_HIP";
    case RN_ERR_WORKSPACE: return "RN_ERR_WORKSPACE";
    case RN_ERR_EXCHANGE: return "RN_ERR_EXCHANGE";
    case RN_ERR_NONFINITE: return "RN_ERR_NONFINITE";
    default: return "RN_ERR_UNKNOWN";
  }
}

static bool use_mfma_parallel(const rn_desc* d, const rn::CallArgs& a) {
  return !(d->flags & RN_FORCE_GENERIC) && !a.gpair && rn::parallel_mfma_supported(a, d->in_dtype);
}

size_t rn_parallel_workspace_bytes(const rn_desc* desc) {
  rn::CallArgs a;
  if (check_desc(desc, Form::kParallel, &a) != RN_OK) return 0;
  return use_mfma_parallel(desc, a) ? align256(rn::parallel_mfma_ws_bytes(a)) : 0;
}

rn_status rn_retention_parallel(const rn_desc* desc, const void* q, const void* k, const void* v,
                                const void* gate, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kParallel, &a);
  if (s != RN_OK) return s;
  if ((s = check_ptrs(desc, q, k, v, gate, out)) != RN_OK) return s;
  const bool mfma = use_mfma_parallel(desc, a);
  if (mfma) {
    const size_t need = align256(rn::parallel_mfma_ws_bytes(a));
    if (!workspace || workspace_bytes < need)
      return fail(RN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(RN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  g_err[0] = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mfma)
    return hip_status(rn::launch_parallel_mfma(a, desc->out_dtype, q, k, v, gate, out, workspace, st),
                      "parallel (MFMA) launch");
  return hip_status(rn::launch_generic_parallel(a, desc->in_dtype, desc->out_dtype, q, k, v,
                                                gate, out, st),
                    "parallel launch");
}

// Chunkwise schedules: the sequential fused kernel (default where it applies), the
// segmented schedule (on request, and where the sequential kernel's decay range does not
// hold), the chunk-parallel pair (on request, and for one decay per coordinate pair), the
// generic float32 kernel (everything else).
enum class ChunkPath { kSegmented, kParallelPair, kSequential, kGeneric };

static ChunkPath chunk_path(const rn_desc* d, const rn::CallArgs& a) {
  if (d->flags & RN_FORCE_GENERIC) return ChunkPath::kGeneric;
  const bool pair = rn::chunkwise_cp_supported(a, d->in_dtype);
  const bool seg = rn::chunkwise_seg_supported(a, d->in_dtype);
  if (a.gpair) return pair ? ChunkPath::kParallelPair : ChunkPath::kGeneric;
  if ((d->flags & RN_CHUNK_PARALLEL) && pair) return ChunkPath::kParallelPair;
  if ((d->flags & RN_CHUNK_SEGMENTED) && seg) return ChunkPath::kSegmented;
  if (rn::chunkwise_mfma_supported(a, d->in_dtype)) return ChunkPath::kSequential;
  if (seg) return ChunkPath::kSegmented;
  if (pair) return ChunkPath::kParallelPair;
  return ChunkPath::kGeneric;
}

size_t rn_chunkwise_workspace_bytes(const rn_desc* desc, int32_t chunk) {
  rn::CallArgs a;
  if (chunk < 1 || check_desc(desc, Form::kChunkwise, &a) != RN_OK) return 0;
  switch (chunk_path(desc, a)) {
    case ChunkPath::kSegmented: return align256(rn::chunkwise_seg_ws_bytes(a));
    case ChunkPath::kParallelPair: return align256(rn::chunkwise_cp_ws_bytes(a));
    case ChunkPath::kSequential: return align256(rn::chunkwise_mfma_ws_bytes(a));
    default: return generic_ws_bytes(desc);
  }
}

static rn_status chunkwise_call(const rn_desc* desc, int32_t chunk, const int64_t* pos,
                                const int32_t* lengths, const void* q, const void* k,
                                const void* v, const void* gate, const float* state_in,
                                float* state_out, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kChunkwise, &a);
  if (s != RN_OK) return s;
  if ((s = check_seq_arrays(pos, lengths, &a)) != RN_OK) return s;
  if (chunk < 1) return fail(RN_ERR_INVALID_ARG, "chunk=%d must be >= 1", chunk);
  if ((s = check_ptrs(desc, q, k, v, gate, out)) != RN_OK) return s;
  const size_t need = rn_chunkwise_workspace_bytes(desc, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(RN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(RN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  a.chunk = chunk;
  g_err[0] = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const ChunkPath path = chunk_path(desc, a);
  if (path == ChunkPath::kSegmented)
    return hip_status(rn::launch_chunkwise_seg(a, desc->out_dtype, q, k, v, gate, state_in,
                                               state_out, out, workspace, workspace_bytes, st),
                      "chunkwise (segmented) launch");
  if (path == ChunkPath::kParallelPair)
    return hip_status(rn::launch_chunkwise_cp(a, desc->out_dtype, q, k, v, gate, state_in,
                                              state_out, out, workspace, workspace_bytes, st),
                      "chunkwise (chunk-parallel) launch");
  if (path == ChunkPath::kSequential)
    return hip_status(rn::launch_chunkwise_mfma(a, desc->out_dtype, q, k, v, gate, state_in,
                                                state_out, out, workspace, workspace_bytes, st),
                      "chunkwise (sequential MFMA) launch");
  return hip_status(rn::launch_generic_chunkwise(a, desc->in_dtype, desc->out_dtype, q, k, v,
                                                 gate, state_in, state_out, out,
                                                 static_cast<float*>(workspace), st),
                    "chunkwise launch");
}

rn_status rn_retention_chunkwise(const rn_desc* desc, int32_t chunk, const void* q, const void* k,
                                 const void* v, const void* gate, const float* state_in,
                                 float* state_out, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return chunkwise_call(desc, chunk, nullptr, nullptr, q, k, v, gate, state_in, state_out, out,
                        workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- chunkwise form without allocation --------------------------------------------------
// A workspace the library holds in device memory, for callers that cannot allocate. Each
// GPU the library runs on holds its own copy of the array until the process ends; host
// code reaches it only through the address hipGetSymbolAddress returns for the current
// device (the array's name on the host is not a device address).
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up once per device.
rn_status scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(RN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RN_OK;
}
}  // namespace

extern "C" {

rn_status rn_retention_chunkwise_noalloc(const rn_desc* desc, int32_t chunk, const void* q,
                                         const void* k, const void* v, const void* gate,
                                         const float* state_in, float* state_out, void* out,
                                         void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kChunkwise, &a);
  if (s != RN_OK) return s;
  if (chunk < 1) return fail(RN_ERR_INVALID_ARG, "chunk=%d must be >= 1", chunk);
  const size_t need = rn_chunkwise_workspace_bytes(desc, chunk);
  if (need > kScratchBytes)
    return fail(RN_ERR_UNSUPPORTED, "this call needs %zu bytes of workspace; the library's "
                "buffer for calls without allocation holds %zu", need, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != RN_OK) return s;
  return chunkwise_call(desc, chunk, nullptr, nullptr, q, k, v, gate, state_in, state_out,
                        out, ws, kScratchBytes, stream);
}

rn_status rn_chunkwise_check(const rn_desc* desc, int32_t chunk, const void* workspace,
                             size_t workspace_bytes, void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kChunkwise, &a);
  if (s != RN_OK) return s;
  if (chunk < 1) return fail(RN_ERR_INVALID_ARG, "chunk=%d must be >= 1", chunk);
  const ChunkPath path = chunk_path(desc, a);
  if (path == ChunkPath::kGeneric) return RN_OK;   // the float32 kernels record nothing
  if (!workspace) return fail(RN_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < sizeof(uint32_t))
    return fail(RN_ERR_WORKSPACE, "workspace %zu bytes holds no status word", workspace_bytes);
  // The status word is the first word of the MFMA schedules' workspaces. A device
  // pointer is read after the call's stream has finished; anything else (a host copy of
  // the workspace) is read directly.
  uint32_t word = 0;
  hipPointerAttribute_t attr;
  const bool on_device = hipPointerGetAttributes(&attr, workspace) == hipSuccess &&
                         attr.type == hipMemoryTypeDevice;
  (void)hipGetLastError();   // a host pointer leaves an error behind on some runtimes
  if (on_device) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e, "reading the chunkwise status word");
  } else {
    std::memcpy(&word, workspace, sizeof(word));
  }
  g_err[0] = 0;
  if (word & rn::kChunkwiseStatusTimeout)
    return fail(RN_ERR_EXCHANGE, "a cross-workgroup wait of the sequential chunkwise kernel "
                                 "hit its time limit; its outputs are NaN");
  if (word & rn::kChunkwiseStatusNonFinite)
    return fail(RN_ERR_NONFINITE, "the %s chunkwise schedule produced non-finite values",
                path == ChunkPath::kSequential ? "sequential"
                : path == ChunkPath::kSegmented ? "segmented" : "chunk-parallel");
  return RN_OK;
}

rn_status rn_retention_chunkwise_varlen(const rn_desc* desc, int32_t chunk, const int64_t* pos,
                                        const int32_t* lengths, const void* q, const void* k,
                                        const void* v, const void* gate, const float* state_in,
                                        float* state_out, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return chunkwise_call(desc, chunk, pos, lengths, q, k, v, gate, state_in, state_out, out,
                        workspace, workspace_bytes, stream);
}

static rn_status step_call(const rn_desc* desc, const int64_t* pos, const void* q, const void* k,
                           const void* v, const void* gate, float* state, void* out,
                           void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kStep, &a);
  if (s != RN_OK) return s;
  if ((s = check_seq_arrays(pos, nullptr, &a)) != RN_OK) return s;
  if ((s = check_ptrs(desc, q, k, v, gate, out)) != RN_OK) return s;
  if (!state) return fail(RN_ERR_INVALID_ARG, "state pointer is NULL");
  if (reinterpret_cast<uintptr_t>(state) % 16)
    return fail(RN_ERR_INVALID_ARG, "state must be 16-byte aligned");
  g_err[0] = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(rn::launch_decode_step(a, desc->in_dtype, desc->out_dtype, q, k, v, gate,
                                           state, out, st),
                    "recurrent step launch");
}

rn_status rn_retention_recurrent_step(const rn_desc* desc, const void* q, const void* k,
                                      const void* v, const void* gate, float* state, void* out,
                                      void* stream) {
  return step_call(desc, nullptr, q, k, v, gate, state, out, stream);
}

rn_status rn_retention_recurrent_step_at(const rn_desc* desc, const int64_t* pos, const void* q,
                                         const void* k, const void* v, const void* gate,
                                         float* state, void* out, void* stream) {
  if (!pos) return fail(RN_ERR_INVALID_ARG, "pos is NULL");
  return step_call(desc, pos, q, k, v, gate, state, out, stream);
}

// Workspace of the gradients: the matrix-core path's where it may run (it is chosen per
// call, by the pointers' alignment), never less than the float32 path's.
static size_t backward_need(const rn_desc* desc, const rn::CallArgs& a) {
  size_t n = rn::backward_ws_bytes(a);
  if (!(desc->flags & RN_FORCE_GENERIC) && rn::backward_mfma_supported(a, desc->in_dtype))
    n = std::max(n, rn::backward_mfma_ws_bytes(a));
  return align256(n);
}

size_t rn_chunkwise_backward_workspace_bytes(const rn_desc* desc, int32_t chunk) {
  rn::CallArgs a;
  if (chunk < 1 || check_desc(desc, Form::kChunkwise, &a) != RN_OK || a.gpair) return 0;
  return backward_need(desc, a);
}

rn_status rn_retention_chunkwise_backward(const rn_desc* desc, int32_t chunk, const void* q,
                                          const void* k, const void* v, const void* gate,
                                          const float* state_in, const void* dout,
                                          const float* dstate_out, void* dq, void* dk, void* dv,
                                          void* dgate, float* dstate_in, float* dgn_weight,
                                          float* dgn_bias, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  rn::CallArgs a;
  rn_status s = check_desc(desc, Form::kChunkwise, &a);
  if (s != RN_OK) return s;
  if (chunk < 1) return fail(RN_ERR_INVALID_ARG, "chunk=%d must be >= 1", chunk);
  if (desc->gamma_pair)
    return fail(RN_ERR_UNSUPPORTED, "the backward takes one decay per head (gamma_pair is set)");
  if (int64_t(desc->B) * desc->H > 65535)
    return fail(RN_ERR_UNSUPPORTED, "B*H=%lld > 65535 (one grid row per head)",
                (long long)desc->B * desc->H);
  if (!q || !k || !v || !dout || !dq || !dk || !dv)
    return fail(RN_ERR_INVALID_ARG, "q/k/v/dout/dq/dk/dv pointer is NULL");
  if ((desc->flags & RN_EPI_GATE) && (!gate || !dgate))
    return fail(RN_ERR_INVALID_ARG, "RN_EPI_GATE needs gate and dgate");
  const size_t need = backward_need(desc, a);
  if (!workspace || workspace_bytes < need)
    return fail(RN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(RN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  a.chunk = chunk;
  rn::BwArgs x{q, k, v, (desc->flags & RN_EPI_GATE) ? gate : nullptr, dout, state_in, dstate_out,
               dq, dk, dv, (desc->flags & RN_EPI_GATE) ? dgate : nullptr, dstate_in,
               (desc->flags & RN_EPI_GN) ? dgn_weight : nullptr,
               (desc->flags & RN_EPI_GN) ? dgn_bias : nullptr};
  g_err[0] = 0;
  auto a16 = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  const bool mfma = !(desc->flags & RN_FORCE_GENERIC) && rn::backward_mfma_supported(a, desc->in_dtype) &&
                    a16(v) && a16(dv) && a16(dout) &&
                    a16(x.gate) && a16(x.dgate) && reinterpret_cast<uintptr_t>(q) % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(k) % 4 == 0;
  if (mfma)
    return hip_status(rn::launch_backward_mfma(a, desc->out_dtype, x, workspace,
                                               static_cast<hipStream_t>(stream)),
                      "chunkwise backward (matrix cores) launch");
  return hip_status(rn::launch_backward(a, desc->in_dtype, desc->out_dtype, x, workspace,
                                        static_cast<hipStream_t>(stream)),
                    "chunkwise backward launch");
}

// ---- gated multi-scale retention layer ---------------------------------------------------

namespace {

struct LayerPlan {
  rn::LayerArgs L;
  bool gate;
  size_t off_q, off_k, off_v, off_g, off_o, off_ret, ret_bytes, total;
  rn_desc ret_desc;   // the retention call: bf16 head outputs
};

rn_status plan_layer(const rn_desc* d, int32_t d_model, int32_t chunk, LayerPlan* p) {
  rn::CallArgs a;
  rn_status s = check_desc(d, Form::kChunkwise, &a);
  if (s != RN_OK) return s;
  if (chunk < 1) return fail(RN_ERR_INVALID_ARG, "chunk=%d must be >= 1", chunk);
  if (d_model < 1) return fail(RN_ERR_INVALID_ARG, "d_model=%d must be >= 1", d_model);
  if (d->in_dtype != RN_BF16)
    return fail(RN_ERR_UNSUPPORTED, "the layer takes bf16 input and weights (in_dtype)");
  if (d->d_v % 8) return fail(RN_ERR_UNSUPPORTED, "the layer needs d_v %% 8 == 0 (got %d)", d->d_v);
  const int64_t cols = int64_t(d->H) * std::max(d->d_k, d->d_v);
  if (cols > (int64_t(1) << 30) || int64_t(d->B) * d->N > (int64_t(1) << 30) ||
      d_model > (1 << 30))
    return fail(RN_ERR_UNSUPPORTED, "layer dimensions beyond 32-bit GEMM sizes");
  p->L = rn::LayerArgs{d->B, d->H, d->N, d_model, d->d_k, d->d_v};
  p->gate = (d->flags & RN_EPI_GATE) != 0;
  p->ret_desc = *d;
  p->ret_desc.out_dtype = RN_BF16;
  const size_t tok = size_t(d->B) * d->H * d->N;
  const size_t bq = align256(tok * d->d_k * 2), bv = align256(tok * d->d_v * 2);
  p->off_q = 0;
  p->off_k = bq;
  p->off_v = 2 * bq;
  p->off_g = 2 * bq + bv;
  p->off_o = p->off_g + (p->gate ? bv : 0);
  p->off_ret = p->off_o + bv;
  p->ret_bytes = rn_chunkwise_workspace_bytes(&p->ret_desc, chunk);
  p->total = p->off_ret + align256(p->ret_bytes);
  return RN_OK;
}

rn_status blas_status(int st, const char* what) {
  if (st == 0) return RN_OK;
  return fail(RN_ERR_HIP, "%s: %s", what, rn::blas_status_string(st));
}

}  // namespace

size_t rn_msr_layer_workspace_bytes(const rn_desc* desc, int32_t d_model, int32_t chunk) {
  LayerPlan p;
  if (plan_layer(desc, d_model, chunk, &p) != RN_OK) return 0;
  return p.total;
}

rn_status rn_msr_layer_forward(const rn_desc* desc, int32_t d_model, int32_t chunk, const void* x,
                               const void* w_q, const void* w_k, const void* w_v, const void* w_g,
                               const void* w_o, const float* state_in, float* state_out,
                               void* out, void* workspace, size_t workspace_bytes, void* stream) {
  LayerPlan p;
  rn_status s = plan_layer(desc, d_model, chunk, &p);
  if (s != RN_OK) return s;
  if (!x || !w_q || !w_k || !w_v || !w_o || !out)
    return fail(RN_ERR_INVALID_ARG, "x/w_q/w_k/w_v/w_o/out pointer is NULL");
  if (p.gate && !w_g) return fail(RN_ERR_INVALID_ARG, "RN_EPI_GATE needs w_g");
  if (!workspace || workspace_bytes < p.total)
    return fail(RN_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, p.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(RN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  g_err[0] = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void *q = ws + p.off_q, *k = ws + p.off_k, *v = ws + p.off_v, *o = ws + p.off_o;
  void* g = p.gate ? ws + p.off_g : nullptr;
  if ((s = blas_status(rn::layer_project(p.L, x, w_q, desc->d_k, q, st), "projection X W_Q")) ||
      (s = blas_status(rn::layer_project(p.L, x, w_k, desc->d_k, k, st), "projection X W_K")) ||
      (s = blas_status(rn::layer_project(p.L, x, w_v, desc->d_v, v, st), "projection X W_V")))
    return s;
  if (p.gate && (s = blas_status(rn::layer_project(p.L, x, w_g, desc->d_v, g, st), "projection X W_G")))
    return s;
  if ((s = chunkwise_call(&p.ret_desc, chunk, nullptr, nullptr, q, k, v, g, state_in, state_out, o,
                          ws + p.off_ret, p.ret_bytes, stream)) != RN_OK)
    return s;
  // the regrouped heads go to v's region (v is no longer needed; same size)
  return blas_status(rn::layer_output(p.L, o, v, w_o, out, desc->out_dtype, st), "output projection");
}

rn_status rn_groupnorm_gate(int32_t B, int32_t H, int32_t N, int32_t d_v, rn_dtype in_dtype,
                            rn_dtype out_dtype, const void* x, const void* gate, const float* w,
                            const float* b, float eps, void* out, void* stream) {
  if (B < 1 || H < 1 || N < 1 || d_v < 1)
    return fail(RN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d N=%d d_v=%d)", B, H, N, d_v);
  if (d_v > rn::kMaxDv) return fail(RN_ERR_UNSUPPORTED, "d_v=%d > %d", d_v, rn::kMaxDv);
  if (int64_t(B) * H * N > (int64_t(1) << 33))
    return fail(RN_ERR_UNSUPPORTED, "B*H*N too large");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(RN_ERR_INVALID_ARG, "unknown dtype (in=%d out=%d)", in_dtype, out_dtype);
  if (!x || !out) return fail(RN_ERR_INVALID_ARG, "x/out pointer is NULL");
  if (!(eps >= 0.f && std::isfinite(eps))) return fail(RN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (out == x && in_dtype != out_dtype)
    return fail(RN_ERR_INVALID_ARG, "in-place GroupNorm needs in_dtype == out_dtype");
  g_err[0] = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(rn::launch_groupnorm_gate(B, H, N, d_v, in_dtype, out_dtype, x, gate, w, b,
                                              eps, out, st),
                    "groupnorm launch");
}

}  // extern "C"
