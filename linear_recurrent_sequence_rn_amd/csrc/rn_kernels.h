// Host-side launchers of the retention kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>

#include "rn_device.h"

namespace rn {

hipError_t launch_generic_parallel(const CallArgs& a, int in_dt, int out_dt, const void* q,
                                   const void* k, const void* v, const void* gate, void* out,
                                   hipStream_t st);
hipError_t launch_generic_chunkwise(const CallArgs& a, int in_dt, int out_dt, const void* q,
                                    const void* k, const void* v, const void* gate,
                                    const float* s_in, float* s_out, void* out, float* ws,
                                    hipStream_t st);
hipError_t launch_decode_step(const CallArgs& a, int in_dt, int out_dt, const void* q,
                              const void* k, const void* v, const void* gate, float* state,
                              void* out, hipStream_t st);
hipError_t launch_groupnorm_gate(int B, int H, int N, int dv, int in_dt, int out_dt,
                                 const void* x, const void* gate, const float* w, const float* b,
                                 float eps, void* out, hipStream_t st);

// Fused MFMA chunkwise kernel (bf16 inputs, d_k = 256, d_v in {64,128,256,512}).
// Its workspace starts with the call's status word: these bits.
constexpr uint32_t kChunkwiseStatusTimeout = 1u;     // a cross-workgroup wait timed out
constexpr uint32_t kChunkwiseStatusNonFinite = 2u;   // a non-finite output or final state
bool chunkwise_mfma_supported(const CallArgs& a, int in_dt);
size_t chunkwise_mfma_ws_bytes(const CallArgs& a);
hipError_t launch_chunkwise_mfma(const CallArgs& a, int out_dt, const void* q, const void* k,
                                 const void* v, const void* gate, const float* s_in,
                                 float* s_out, void* out, void* ws, size_t ws_bytes,
                                 hipStream_t st);

// Chunk-parallel chunkwise pair: state snapshots, then outputs (bf16, d_k 256, d_v 512).
bool chunkwise_cp_supported(const CallArgs& a, int in_dt);
size_t chunkwise_cp_ws_bytes(const CallArgs& a);
hipError_t launch_chunkwise_cp(const CallArgs& a, int out_dt, const void* q, const void* k,
                               const void* v, const void* gate, const float* s_in, float* s_out,
                               void* out, void* ws, size_t ws_bytes, hipStream_t st);

// Segmented chunkwise schedule: segment-local states, a scan over segments, then the
// outputs of all chunks (bf16, d_k 256, d_v 512, one decay per head).
bool chunkwise_seg_supported(const CallArgs& a, int in_dt);
size_t chunkwise_seg_ws_bytes(const CallArgs& a);
hipError_t launch_chunkwise_seg(const CallArgs& a, int out_dt, const void* q, const void* k,
                                const void* v, const void* gate, const float* s_in, float* s_out,
                                void* out, void* ws, size_t ws_bytes, hipStream_t st);

// Gradients of the chunkwise form: f16-operand MFMA products with float32 accumulation for
// bf16 inputs whose d_k and d_v are multiples of 8, float32 products otherwise.
struct BwArgs {
  const void* q; const void* k; const void* v; const void* gate;
  const void* dout; const float* state_in; const float* dstate_out;
  void* dq; void* dk; void* dv; void* dgate; float* dstate_in;
  float* dgn_w; float* dgn_b;
};
size_t backward_ws_bytes(const CallArgs& a);
hipError_t launch_backward(const CallArgs& a, int in_dt, int out_dt, const BwArgs& x, void* ws,
                           hipStream_t st);
// Matrix-core path of the gradients (bf16 inputs, d_k and d_v multiples of 8; v, dv, dout,
// gate and dgate 16-byte and q, k 4-byte aligned).
bool backward_mfma_supported(const CallArgs& a, int in_dt);
size_t backward_mfma_ws_bytes(const CallArgs& a);
hipError_t launch_backward_mfma(const CallArgs& a, int out_dt, const BwArgs& x, void* ws,
                                hipStream_t st);

// MFMA parallel form (bf16 inputs, d_k = 256, d_v = 512).
bool parallel_mfma_supported(const CallArgs& a, int in_dt);
size_t parallel_mfma_ws_bytes(const CallArgs& a);
hipError_t launch_parallel_mfma(const CallArgs& a, int out_dt, const void* q, const void* k,
                                const void* v, const void* gate, void* out, void* ws,
                                hipStream_t st);

// Gated multi-scale retention layer: rocBLAS projections and output projection (return
// values are rocblas_status codes; 0 = success).
struct LayerArgs {
  int B, H, N, d_model, dk, dv;
};
int layer_project(const LayerArgs& L, const void* x, const void* w, int d, void* y,
                  hipStream_t stream);
int layer_output(const LayerArgs& L, const void* o, void* ot, const void* w_o, void* out,
                 int out_dtype, hipStream_t stream);
const char* blas_status_string(int status);

}  // namespace rn
