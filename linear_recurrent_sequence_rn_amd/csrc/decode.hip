// One recurrent retention step (decode): S <- gamma S + Kh^T v in place, o = alpha Qh S
// (hwhale notes: recurrent equations and the RecurrentRetention listing). The token of
// sequence b sits at the descriptor's position, or at pos[b] when the call passes one
// position per sequence (batched decode of sequences of different lengths). With one
// decay per coordinate pair, state rows 2j and 2j+1 are scaled by pair j's decay.
//
// HBM-bound: the float32 state is read and written once per step; everything else is
// a few KB. One block owns one (b, h) state of d_k x d_v floats. Thread (group g,
// column vector c) owns columns [4c, 4c+4) of rows g, g+G, g+2G, ... so each row is
// read and written by consecutive lanes in 16-byte pieces (a wave covers 1 KB of one
// row per instruction). Non-temporal hints: the state (1 GB for batch 128 x 16 heads)
// is far larger than the last-level cache and is not re-read within the step.
//
// Main kernel (d_v in {128, 256, 512}, d_k a multiple of 8G): 512 threads, rows taken
// in batches of 8 per thread, two batches in flight: the loads of batch i+1 are issued
// before batch i is updated and stored, so the read stream never waits for the
// stores. (Measured on the 6.7B decode shape: 71% of HBM peak, against 67% for one
// batch in flight and 60% for a device-to-device copy of the same bytes.) Other
// shapes use the plain kernel below it, one batch in flight.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

constexpr int kBatch = 8;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int IN, int OUT, int VEC>
__global__ void __launch_bounds__(256) decode_step(CallArgs a, const void* q, const void* k,
                                                   const void* v, const void* gate, float* state,
                                                   void* out) {
  __shared__ float qh[kMaxDk];
  __shared__ float kh[kMaxDk];
  __shared__ float gd[kMaxDk];   // decay of each state row
  __shared__ float vv[kMaxDv];
  __shared__ float part[256 * 4];
  __shared__ float orow[kMaxDv];
  __shared__ float red[4];
  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int dk = a.dk, dv = a.dv;
  const int64_t pos = seq_pos0(a, bh / a.H);
  for (int j = threadIdx.x; j < dk / 2; j += 256) {
    float c, s;
    angle_cs(pos, a.ap.theta[j], &c, &s);
    const int64_t o = static_cast<int64_t>(bh) * dk + 2 * j;
    float q0 = Elem<IN>::load(q, o), q1 = Elem<IN>::load(q, o + 1);
    float k0 = Elem<IN>::load(k, o), k1 = Elem<IN>::load(k, o + 1);
    qh[2 * j] = q0 * c - q1 * s;
    qh[2 * j + 1] = q0 * s + q1 * c;
    kh[2 * j] = k0 * c - k1 * s;
    kh[2 * j + 1] = k0 * s + k1 * c;
    gd[2 * j] = gd[2 * j + 1] = pair_gamma(a, h, j);
  }
  for (int c = threadIdx.x; c < dv; c += 256) vv[c] = Elem<IN>::load(v, static_cast<int64_t>(bh) * dv + c);
  __syncthreads();

  const int nq = dv / VEC;                 // column vectors per row
  const int G = nq >= 256 ? 1 : 256 / nq;  // row groups
  const int tid = threadIdx.x;
  // A slot is one (row group, column vector); a thread owns one slot, or two when a
  // row has more than 256 column vectors (odd d_v above 256).
  for (int slot = tid; slot < G * nq; slot += 256) {
    const int cq = slot % nq, grp = slot / nq;
    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
    float vr[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) vr[i] = vv[cq * VEC + i];
    float* S = state + static_cast<int64_t>(bh) * dk * dv + cq * VEC;
    for (int d0 = grp; d0 < dk; d0 += G * kBatch) {
      float sv[kBatch][VEC];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d = d0 + u * G;
        if (d < dk) {
          if constexpr (VEC == 4) {
            f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + static_cast<int64_t>(d) * dv));
            sv[u][0] = x.x; sv[u][1] = x.y; sv[u][2] = x.z; sv[u][3] = x.w;
          } else {
            sv[u][0] = __builtin_nontemporal_load(S + static_cast<int64_t>(d) * dv);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int d = d0 + u * G;
        if (d < dk) {
          const float kd = kh[d], qd = qh[d], g = gd[d];
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            float s = fmaf(g, sv[u][i], kd * vr[i]);
            sv[u][i] = s;
            acc[i] = fmaf(qd, s, acc[i]);
          }
          if constexpr (VEC == 4) {
            f32x4 x = {sv[u][0], sv[u][1], sv[u][2], sv[u][3]};
            __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(S + static_cast<int64_t>(d) * dv));
          } else {
            __builtin_nontemporal_store(sv[u][0], S + static_cast<int64_t>(d) * dv);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) part[grp * dv + cq * VEC + i] = acc[i];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < dv; c += 256) {
    float s = 0.f;
    for (int gg = 0; gg < G; ++gg) s += part[gg * dv + c];
    orow[c] = a.alpha * s;
  }
  __syncthreads();
  row_epilogue256<IN, OUT>(orow, dv, a, h, gate, static_cast<int64_t>(bh) * dv, out, red);
}


constexpr int kFastThreads = 512;
constexpr int kFastBatch = 8;

// d_v = 4 * NQ; G = 512 / NQ row groups; d_k % (G * kFastBatch) == 0.
template <int IN, int OUT, int NQ>
__global__ void __launch_bounds__(kFastThreads) decode_step_pipelined(CallArgs a, const void* q,
                                                                      const void* k, const void* v,
                                                                      const void* gate,
                                                                      float* state, void* out) {
  constexpr int G = kFastThreads / NQ;
  constexpr int DV = 4 * NQ;
  __shared__ float qh[kMaxDk];
  __shared__ float kh[kMaxDk];
  __shared__ float gd[kMaxDk];   // decay of each state row
  __shared__ float part[G * DV];
  __shared__ float orow[DV];
  __shared__ float red[kFastThreads / 64];
  const int bh = blockIdx.x;
  const int h = bh % a.H;
  const int dk = a.dk;
  const int tid = threadIdx.x, cq = tid % NQ, grp = tid / NQ;
  const int64_t pos = seq_pos0(a, bh / a.H);
  for (int j = tid; j < dk / 2; j += kFastThreads) {
    float c, s;
    angle_cs(pos, a.ap.theta[j], &c, &s);
    const int64_t o = static_cast<int64_t>(bh) * dk + 2 * j;
    float q0 = Elem<IN>::load(q, o), q1 = Elem<IN>::load(q, o + 1);
    float k0 = Elem<IN>::load(k, o), k1 = Elem<IN>::load(k, o + 1);
    qh[2 * j] = q0 * c - q1 * s;
    qh[2 * j + 1] = q0 * s + q1 * c;
    kh[2 * j] = k0 * c - k1 * s;
    kh[2 * j + 1] = k0 * s + k1 * c;
    gd[2 * j] = gd[2 * j + 1] = pair_gamma(a, h, j);
  }
  float vr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vr[i] = Elem<IN>::load(v, static_cast<int64_t>(bh) * DV + 4 * cq + i);
  __syncthreads();

  const int nit = dk / (G * kFastBatch);
  float* S = state + static_cast<int64_t>(bh) * dk * DV + 4 * cq;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto load = [&](int it, f32x4* sv) {
    const int d0 = grp + it * G * kFastBatch;
#pragma unroll
    for (int u = 0; u < kFastBatch; ++u)
      sv[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + static_cast<int64_t>(d0 + u * G) * DV));
  };
  auto update = [&](int it, f32x4* sv) {
    const int d0 = grp + it * G * kFastBatch;
#pragma unroll
    for (int u = 0; u < kFastBatch; ++u) {
      const int d = d0 + u * G;
      const float kd = kh[d], qd = qh[d], g = gd[d];
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = fmaf(g, sv[u][i], kd * vr[i]);
        acc[i] = fmaf(qd, x[i], acc[i]);
      }
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(S + static_cast<int64_t>(d) * DV));
    }
  };
  f32x4 ba[kFastBatch], bb[kFastBatch];
  load(0, ba);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(it + 1, bb);
    update(it, ba);
    if (it + 2 < nit) load(it + 2, ba);
    if (it + 1 < nit) update(it + 1, bb);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[grp * DV + 4 * cq + i] = acc[i];
  __syncthreads();
  for (int c = tid; c < DV; c += kFastThreads) {
    float s = 0.f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) s += part[gg * DV + c];
    orow[c] = a.alpha * s;
  }
  __syncthreads();
  row_epilogue<IN, OUT, kFastThreads>(orow, DV, a, h, gate, static_cast<int64_t>(bh) * DV, out, red);
}

template <int IN, int OUT>
hipError_t launch_t(const CallArgs& a, const void* q, const void* k, const void* v,
                    const void* gate, float* state, void* out, hipStream_t st) {
  dim3 grid(a.B * a.H);
  const int G = a.dv > 0 && a.dv % 4 == 0 ? kFastThreads / (a.dv / 4) : 0;
  if ((a.dv == 128 || a.dv == 256 || a.dv == 512) && a.dk % (G * kFastBatch) == 0) {
    if (a.dv == 512)
      hipLaunchKernelGGL((decode_step_pipelined<IN, OUT, 128>), grid, dim3(kFastThreads), 0, st, a, q, k, v, gate, state, out);
    else if (a.dv == 256)
      hipLaunchKernelGGL((decode_step_pipelined<IN, OUT, 64>), grid, dim3(kFastThreads), 0, st, a, q, k, v, gate, state, out);
    else
      hipLaunchKernelGGL((decode_step_pipelined<IN, OUT, 32>), grid, dim3(kFastThreads), 0, st, a, q, k, v, gate, state, out);
    return hipGetLastError();
  }
  if (a.dv % 4 == 0 && a.dv / 4 <= 256)
    hipLaunchKernelGGL((decode_step<IN, OUT, 4>), grid, dim3(256), 0, st, a, q, k, v, gate, state, out);
  else
    hipLaunchKernelGGL((decode_step<IN, OUT, 1>), grid, dim3(256), 0, st, a, q, k, v, gate, state, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const CallArgs& a, int in_dt, int out_dt, const void* q,
                              const void* k, const void* v, const void* gate, float* state,
                              void* out, hipStream_t st) {
  if (in_dt == RN_F32)
    return out_dt == RN_F32 ? launch_t<RN_F32, RN_F32>(a, q, k, v, gate, state, out, st)
                            : launch_t<RN_F32, RN_BF16>(a, q, k, v, gate, state, out, st);
  return out_dt == RN_F32 ? launch_t<RN_BF16, RN_F32>(a, q, k, v, gate, state, out, st)
                          : launch_t<RN_BF16, RN_BF16>(a, q, k, v, gate, state, out, st);
}

}  // namespace rn
