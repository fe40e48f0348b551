// Standalone per-head GroupNorm + swish gate over rows of d_v channels
// (hwhale notes, multi-head paragraph: one GroupNorm group per head; m0nads notes,
// "Gated Multi-Scale Retention": swish gate).
// One 64-lane wave per (b, h, t) row, the row held in registers (<= 8 values per
// lane); mean first, then the biased variance of the centred values; 4 rows per
// 256-thread block. HBM-bound: reads x (+ gate), writes out once.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

template <int IN, int OUT>
__global__ void __launch_bounds__(256) gn_gate_rows(int64_t rows, int H, int N, int dv,
                                                    const void* x, const void* gate,
                                                    const float* w, const float* b, float eps,
                                                    void* out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int head = static_cast<int>((row / N) % H);
  const int64_t off = row * dv;
  float xv[kMaxDv / 64];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxDv / 64; ++i) {
    const int c = lane + 64 * i;
    xv[i] = c < dv ? Elem<IN>::load(x, off + c) : 0.f;
    s += xv[i];
  }
  const float mean = wave_sum(s) / dv;
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxDv / 64; ++i) {
    const int c = lane + 64 * i;
    const float d = c < dv ? xv[i] - mean : 0.f;
    s2 += d * d;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / dv + eps);
#pragma unroll
  for (int i = 0; i < kMaxDv / 64; ++i) {
    const int c = lane + 64 * i;
    if (c < dv) {
      float y = (xv[i] - mean) * rstd;
      if (w) y *= w[head * dv + c];
      if (b) y += b[head * dv + c];
      if (gate) y *= swishf(Elem<IN>::load(gate, off + c));
      Elem<OUT>::store(out, off + c, y);
    }
  }
}

template <int IN, int OUT>
hipError_t launch_t(int B, int H, int N, int dv, const void* x, const void* gate, const float* w,
                    const float* b, float eps, void* out, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(B) * H * N;
  dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  hipLaunchKernelGGL((gn_gate_rows<IN, OUT>), grid, dim3(256), 0, st, rows, H, N, dv, x, gate, w,
                     b, eps, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_groupnorm_gate(int B, int H, int N, int dv, int in_dt, int out_dt,
                                 const void* x, const void* gate, const float* w, const float* b,
                                 float eps, void* out, hipStream_t st) {
  if (in_dt == RN_F32)
    return out_dt == RN_F32 ? launch_t<RN_F32, RN_F32>(B, H, N, dv, x, gate, w, b, eps, out, st)
                            : launch_t<RN_F32, RN_BF16>(B, H, N, dv, x, gate, w, b, eps, out, st);
  return out_dt == RN_F32 ? launch_t<RN_BF16, RN_F32>(B, H, N, dv, x, gate, w, b, eps, out, st)
                          : launch_t<RN_BF16, RN_BF16>(B, H, N, dv, x, gate, w, b, eps, out, st);
}

}  // namespace rn
