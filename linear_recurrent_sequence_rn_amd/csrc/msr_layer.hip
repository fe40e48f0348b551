// Gated multi-scale retention layer around the retention kernels (m0nads notes and
// hwhale notes, "Gated Multi-Scale Retention"): the projections X W_Q, X W_K, X W_V,
// X W_G and the output projection by W_O are plain dense GEMMs and run in rocBLAS (bf16
// operands, float32 accumulation); the retention with its GroupNorm and gate runs in
// the chunkwise kernels; one kernel here regroups the heads' outputs by token for W_O.
//
// Layouts (row-major): X [B, N, d_model]; W_Q, W_K [d_model, H d_k]; W_V, W_G
// [d_model, H d_v]; W_O [H d_v, d_model]; head h owns columns [h d, (h+1) d). rocBLAS is
// column-major, so a row-major product C = A B is issued as C^T = B^T A^T.
//   projection (per batch row b, batched over the H heads): the head's block of W is a
//     column slice (offset h d, leading dimension H d), X_b is shared (stride 0), and
//     the result lands directly in the retention kernels' head-major layout
//     [B, H, N, d] (stride N d per head);
//   output: the heads' outputs [B, H, N, d_v] are regrouped as [B N, H d_v] (one 16-byte
//     copy per 8 values; every row of d_v values stays contiguous), then one GEMM with
//     K = H d_v gives [B N, d_model].
#include <rocblas/rocblas.h>

#include <unordered_map>

#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// o [B, H, N, dv] -> ot [B, N, H, dv]; dv % 8 == 0. Block (row group, h, b) copies
// kRows consecutive rows of one head, 16 bytes (8 bf16) per thread and step. (Putting
// the heads of a row group in neighbouring blocks instead measured 15 % slower.)
constexpr int kRows = 16;
__global__ void __launch_bounds__(256) heads_to_tokens(const uint16_t* __restrict__ o,
                                                       uint16_t* __restrict__ ot, int H, int N,
                                                       int dv) {
  const int vpr = dv / 8;                              // 16-byte pieces per row
  const int h = blockIdx.y, b = blockIdx.z, t0 = blockIdx.x * kRows;
  const int rows = min(kRows, N - t0);
  const u32x4* src = reinterpret_cast<const u32x4*>(o) + ((int64_t(b) * H + h) * N + t0) * vpr;
  u32x4* dst = reinterpret_cast<u32x4*>(ot) + ((int64_t(b) * N + t0) * H + h) * vpr;
  for (int p = threadIdx.x; p < rows * vpr; p += 256) {
    const int r = p / vpr, c = p - r * vpr;
    const u32x4 x = __builtin_nontemporal_load(src + p);
    __builtin_nontemporal_store(x, dst + int64_t(r) * H * vpr + c);
  }
}

// One rocBLAS handle per host thread and device, created on first use and kept for the
// life of the process (a handle is not safe to share between threads that set
// different streams).
rocblas_handle blas_handle(int device, rocblas_status* st) {
  thread_local std::unordered_map<int, rocblas_handle> handles;
  auto it = handles.find(device);
  if (it != handles.end()) {
    *st = rocblas_status_success;
    return it->second;
  }
  rocblas_handle h = nullptr;
  *st = rocblas_create_handle(&h);
  if (*st != rocblas_status_success) return nullptr;
  handles.emplace(device, h);
  return h;
}

}  // namespace

const char* blas_status_string(int status) {
  return rocblas_status_to_string(static_cast<rocblas_status>(status));
}

// Projections of x to one head-major tensor: y[b, h] = x[b] W[:, h d : (h+1) d].
int layer_project(const LayerArgs& L, const void* x, const void* w, int d, void* y,
                  hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return rocblas_status_internal_error;
  rocblas_status st;
  rocblas_handle h = blas_handle(dev, &st);
  if (!h) return st;
  if ((st = rocblas_set_stream(h, stream)) != rocblas_status_success) return st;
  const float one = 1.f, zero = 0.f;
  for (int b = 0; b < L.B; ++b) {
    const uint16_t* xb = static_cast<const uint16_t*>(x) + size_t(b) * L.N * L.d_model;
    uint16_t* yb = static_cast<uint16_t*>(y) + size_t(b) * L.H * L.N * d;
    st = rocblas_gemm_strided_batched_ex(
        h, rocblas_operation_none, rocblas_operation_none, d, L.N, L.d_model, &one,
        w, rocblas_datatype_bf16_r, L.H * d, d,
        xb, rocblas_datatype_bf16_r, L.d_model, 0, &zero,
        yb, rocblas_datatype_bf16_r, d, rocblas_stride(L.N) * d,
        yb, rocblas_datatype_bf16_r, d, rocblas_stride(L.N) * d,
        L.H, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    if (st != rocblas_status_success) return st;
  }
  return rocblas_status_success;
}

// out [B N, d_model] = regroup(o) [B N, H dv] W_O; `ot` receives the regrouped heads.
int layer_output(const LayerArgs& L, const void* o, void* ot, const void* w_o, void* out,
                 int out_dtype, hipStream_t stream) {
  hipLaunchKernelGGL(heads_to_tokens, dim3((L.N + kRows - 1) / kRows, L.H, L.B), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(o), static_cast<uint16_t*>(ot), L.H, L.N,
                     L.dv);
  if (hipGetLastError() != hipSuccess) return rocblas_status_internal_error;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return rocblas_status_internal_error;
  rocblas_status st;
  rocblas_handle h = blas_handle(dev, &st);
  if (!h) return st;
  if ((st = rocblas_set_stream(h, stream)) != rocblas_status_success) return st;
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype ct = out_dtype == RN_F32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
  return rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, L.d_model, L.B * L.N,
                         L.H * L.dv, &one, w_o, rocblas_datatype_bf16_r, L.d_model, ot,
                         rocblas_datatype_bf16_r, L.H * L.dv, &zero, out, ct, L.d_model, out, ct,
                         L.d_model, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
}

}  // namespace rn
