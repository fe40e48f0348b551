// Plain (non-MFMA) retention kernels for float32 inputs and for shapes outside the
// MFMA kernels' tiles. They evaluate the pages' formulas directly, one 256-thread
// block per output row (parallel form) or per head (chunkwise form), with every
// product in float32 and the rotation angle reduced in float64. With one decay per
// coordinate pair (the form before the pages reduce the decay to a scalar), the decay
// of pair j enters the score inside the sum over coordinates, scales the cross term
// per coordinate and the state per row.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

constexpr int kTile = 256;  // keys per score tile

// Rotated element pair (2j, 2j+1) of row x at position p: z * e^{i p theta_j}.
template <int IN>
__device__ __forceinline__ void rot_pair(const void* x, int64_t off, int j, int64_t p,
                                         float theta, float* r0, float* r1) {
  float a = Elem<IN>::load(x, off + 2 * j), b = Elem<IN>::load(x, off + 2 * j + 1);
  float c, s;
  angle_cs(p, theta, &c, &s);
  *r0 = a * c - b * s;
  *r1 = a * s + b * c;
}

// Parallel form, one block per (t, h, b): acc = sum_{s<=t} alpha (Qh_t.Kh_s) D_ts V_s,
// rs = sum_s alpha (Qh_t.Kh_s) D_ts; O_t = c_t acc / max(c_t |rs|, 1) with the
// optional factors (hwhale notes: parallel-form equation, list of three rescalings).
template <int IN, int OUT>
__global__ void __launch_bounds__(256) generic_parallel(CallArgs a, const void* q, const void* k,
                                                        const void* v, const void* gate, void* out) {
  __shared__ float qh[kMaxDk];
  __shared__ float lgp[kMaxDk / 2];
  __shared__ float sc[kTile];
  __shared__ float orow[kMaxDv];
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int dk = a.dk, dv = a.dv;
  const int64_t bh = static_cast<int64_t>(b) * a.H + h;
  const int64_t qoff = (bh * a.N + t) * dk;
  const int64_t pt = a.pos0 + t;
  for (int j = threadIdx.x; j < dk / 2; j += 256) {
    rot_pair<IN>(q, qoff, j, pt, a.ap.theta[j], &qh[2 * j], &qh[2 * j + 1]);
    lgp[j] = pair_log2g(a, h, j);
  }
  const float lg = a.hp.log2g[h];
  const bool per_pair = a.gpair != nullptr;
  float acc0 = 0.f, acc1 = 0.f, rs = 0.f;
  const int c0 = threadIdx.x, c1 = threadIdx.x + 256;
  __syncthreads();
  for (int s0 = 0; s0 <= t; s0 += kTile) {
    const int s = s0 + threadIdx.x;
    float val = 0.f;
    if (s <= t) {
      const int64_t koff = (bh * a.N + s) * dk;
      const int64_t ps = a.pos0 + s;
      float dot = 0.f;
      for (int j = 0; j < dk / 2; ++j) {
        float k0, k1;
        rot_pair<IN>(k, koff, j, ps, a.ap.theta[j], &k0, &k1);
        const float pj = qh[2 * j] * k0 + qh[2 * j + 1] * k1;
        dot += per_pair ? pj * gpow(lgp[j], static_cast<float>(t - s)) : pj;
      }
      val = a.alpha * (per_pair ? dot : dot * gpow(lg, static_cast<float>(t - s)));
    }
    rs += val;
    sc[threadIdx.x] = val;
    __syncthreads();
    const int ns = min(kTile, t - s0 + 1);
    for (int i = 0; i < ns; ++i) {
      const int64_t voff = (bh * a.N + s0 + i) * dv;
      const float w = sc[i];
      if (c0 < dv) acc0 += w * Elem<IN>::load(v, voff + c0);
      if (c1 < dv) acc1 += w * Elem<IN>::load(v, voff + c1);
    }
    __syncthreads();
  }
  float scale = 1.0f;
  if (a.flags & (RN_NORM_D_ROW | RN_NORM_R_ROW)) {
    rs = block_sum256(rs, red);
    double ct = 1.0;
    if (a.flags & RN_NORM_D_ROW) {
      const double g = a.hp.gamma[h];
      const double G = (g == 1.0) ? static_cast<double>(t + 1) : (1.0 - pow(g, t + 1.0)) / (1.0 - g);
      ct = 1.0 / sqrt(G);
    }
    double sc_row = ct;
    if (a.flags & RN_NORM_R_ROW) sc_row = ct / fmax(fabs(ct * static_cast<double>(rs)), 1.0);
    scale = static_cast<float>(sc_row);
  }
  if (c0 < dv) orow[c0] = acc0 * scale;
  if (c1 < dv) orow[c1] = acc1 * scale;
  __syncthreads();
  row_epilogue256<IN, OUT>(orow, dv, a, h, gate, (bh * a.N + t) * dv, out, red);
}

// Chunkwise form, one block per (h, b); the state lives in the float32 workspace
// slice ws[bh] (d_k x d_v). For each chunk of length L starting at c0:
//   rows t:  O_t = alpha [ sum_{c0<=s<=t} gamma^(t-s) (Qh_t.Kh_s) V_s
//                         + gamma^(t-c0+1) Qh_t S ]
//   then     S <- gamma^L S + sum_j gamma^(L-1-j) Kh_j^T V_j
// (hwhale notes: chunkwise equation and ChunkwiseRetention listing). With one decay per
// coordinate pair, every power of gamma is taken per coordinate d inside the products
// (gamma_d^(t-s) Qh_td Kh_sd, gamma_d^(t-c0+1) Qh_td, state row d scaled by gamma_d^L,
// Kh_jd by gamma_d^(L-1-j)). Sequence b runs over its own number of tokens and from its
// own starting position when the call gives them; rows past its length are left
// untouched.
template <int IN, int OUT>
__global__ void __launch_bounds__(256) generic_chunkwise(CallArgs a, const void* q, const void* k,
                                                         const void* v, const void* gate,
                                                         const float* state_in, float* state_out,
                                                         void* out, float* ws) {
  constexpr int kJ = 16;  // key rows per state-update tile
  __shared__ float qh[kMaxDk];
  __shared__ float qx[kMaxDk];     // Qh_t scaled by the cross-term decay of each coordinate
  __shared__ float lgp[kMaxDk / 2];
  __shared__ float sc[kTile];
  __shared__ float orow[kMaxDv];
  __shared__ float kt[kJ][kMaxDk];
  __shared__ float vt[kJ][kMaxDv];
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const int dk = a.dk, dv = a.dv, N = a.N, C = a.chunk;
  const int len = seq_len(a, b);          // tokens of this sequence (rows of stride N)
  const int64_t p0 = seq_pos0(a, b);
  const int64_t bh = static_cast<int64_t>(b) * a.H + h;
  const int64_t nS = static_cast<int64_t>(dk) * dv;
  float* S = ws + bh * nS;
  for (int64_t e = threadIdx.x; e < nS; e += 256) S[e] = state_in ? state_in[bh * nS + e] : 0.f;
  for (int j = threadIdx.x; j < dk / 2; j += 256) lgp[j] = pair_log2g(a, h, j);
  __syncthreads();
  const float lg = a.hp.log2g[h];
  const bool per_pair = a.gpair != nullptr;
  const int c0 = threadIdx.x, c1 = threadIdx.x + 256;
  for (int cs = 0; cs < len; cs += C) {
    const int L = min(C, len - cs);
    for (int t = cs; t < cs + L; ++t) {
      const int64_t pt = p0 + t;
      // cross-term decay xi = gamma^(t - cs + 1), per coordinate pair
      for (int j = threadIdx.x; j < dk / 2; j += 256) {
        rot_pair<IN>(q, (bh * N + t) * dk, j, pt, a.ap.theta[j], &qh[2 * j], &qh[2 * j + 1]);
        const float xi = gpow(lgp[j], static_cast<float>(t - cs + 1));
        qx[2 * j] = qh[2 * j] * xi;
        qx[2 * j + 1] = qh[2 * j + 1] * xi;
      }
      __syncthreads();
      float acc0 = 0.f, acc1 = 0.f;
      for (int s0 = cs; s0 <= t; s0 += kTile) {
        const int s = s0 + threadIdx.x;
        float val = 0.f;
        if (s <= t) {
          const int64_t koff = (bh * N + s) * dk;
          float dot = 0.f;
          for (int j = 0; j < dk / 2; ++j) {
            float k0, k1;
            rot_pair<IN>(k, koff, j, p0 + s, a.ap.theta[j], &k0, &k1);
            const float pj = qh[2 * j] * k0 + qh[2 * j + 1] * k1;
            dot += per_pair ? pj * gpow(lgp[j], static_cast<float>(t - s)) : pj;
          }
          val = per_pair ? dot : dot * gpow(lg, static_cast<float>(t - s));
        }
        sc[threadIdx.x] = val;
        __syncthreads();
        const int ns = min(kTile, t - s0 + 1);
        for (int i = 0; i < ns; ++i) {
          const int64_t voff = (bh * N + s0 + i) * dv;
          if (c0 < dv) acc0 += sc[i] * Elem<IN>::load(v, voff + c0);
          if (c1 < dv) acc1 += sc[i] * Elem<IN>::load(v, voff + c1);
        }
        __syncthreads();
      }
      // cross-chunk term: (Qh_t ⊙ xi) S
      float x0 = 0.f, x1 = 0.f;
      for (int d = 0; d < dk; ++d) {
        if (c0 < dv) x0 += qx[d] * S[static_cast<int64_t>(d) * dv + c0];
        if (c1 < dv) x1 += qx[d] * S[static_cast<int64_t>(d) * dv + c1];
      }
      if (c0 < dv) orow[c0] = a.alpha * (acc0 + x0);
      if (c1 < dv) orow[c1] = a.alpha * (acc1 + x1);
      __syncthreads();
      row_epilogue256<IN, OUT>(orow, dv, a, h, gate, (bh * N + t) * dv, out, red);
      __syncthreads();
    }
    // state update: S <- gamma^L S + sum_j zeta_j Kh_j^T V_j, zeta_j = gamma^(L-1-j)
    for (int j0 = 0; j0 < L; j0 += kJ) {
      const int nj = min(kJ, L - j0);
      for (int e = threadIdx.x; e < nj * (dk / 2); e += 256) {
        const int jj = e / (dk / 2), p = e % (dk / 2);
        const int s = cs + j0 + jj;
        const float zeta = gpow(lgp[p], static_cast<float>(L - 1 - (j0 + jj)));
        float k0, k1;
        rot_pair<IN>(k, (bh * N + s) * dk, p, p0 + s, a.ap.theta[p], &k0, &k1);
        kt[jj][2 * p] = zeta * k0;
        kt[jj][2 * p + 1] = zeta * k1;
      }
      for (int e = threadIdx.x; e < nj * dv; e += 256) {
        const int jj = e / dv, c = e % dv;
        vt[jj][c] = Elem<IN>::load(v, (bh * N + cs + j0 + jj) * dv + c);
      }
      __syncthreads();
      for (int64_t e = threadIdx.x; e < nS; e += 256) {
        const int d = static_cast<int>(e / dv), c = static_cast<int>(e % dv);
        float s = S[e];
        if (j0 == 0) s *= gpow(lgp[d >> 1], static_cast<float>(L));
        for (int jj = 0; jj < nj; ++jj) s += kt[jj][d] * vt[jj][c];
        S[e] = s;
      }
      __syncthreads();
    }
  }
  if (state_out)
    for (int64_t e = threadIdx.x; e < nS; e += 256) state_out[bh * nS + e] = S[e];
}

template <int IN, int OUT>
hipError_t launch_parallel_t(const CallArgs& a, const void* q, const void* k, const void* v,
                             const void* gate, void* out, hipStream_t st) {
  dim3 grid(a.N, a.H, a.B);
  hipLaunchKernelGGL((generic_parallel<IN, OUT>), grid, dim3(256), 0, st, a, q, k, v, gate, out);
  return hipGetLastError();
}

template <int IN, int OUT>
hipError_t launch_chunkwise_t(const CallArgs& a, const void* q, const void* k, const void* v,
                              const void* gate, const float* s_in, float* s_out, void* out,
                              float* ws, hipStream_t st) {
  dim3 grid(a.H, a.B);
  hipLaunchKernelGGL((generic_chunkwise<IN, OUT>), grid, dim3(256), 0, st, a, q, k, v, gate,
                     s_in, s_out, out, ws);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic_parallel(const CallArgs& a, int in_dt, int out_dt, const void* q,
                                   const void* k, const void* v, const void* gate, void* out,
                                   hipStream_t st) {
  if (in_dt == RN_F32)
    return out_dt == RN_F32 ? launch_parallel_t<RN_F32, RN_F32>(a, q, k, v, gate, out, st)
                            : launch_parallel_t<RN_F32, RN_BF16>(a, q, k, v, gate, out, st);
  return out_dt == RN_F32 ? launch_parallel_t<RN_BF16, RN_F32>(a, q, k, v, gate, out, st)
                          : launch_parallel_t<RN_BF16, RN_BF16>(a, q, k, v, gate, out, st);
}

hipError_t launch_generic_chunkwise(const CallArgs& a, int in_dt, int out_dt, const void* q,
                                    const void* k, const void* v, const void* gate,
                                    const float* s_in, float* s_out, void* out, float* ws,
                                    hipStream_t st) {
  if (in_dt == RN_F32)
    return out_dt == RN_F32
               ? launch_chunkwise_t<RN_F32, RN_F32>(a, q, k, v, gate, s_in, s_out, out, ws, st)
               : launch_chunkwise_t<RN_F32, RN_BF16>(a, q, k, v, gate, s_in, s_out, out, ws, st);
  return out_dt == RN_F32
             ? launch_chunkwise_t<RN_BF16, RN_F32>(a, q, k, v, gate, s_in, s_out, out, ws, st)
             : launch_chunkwise_t<RN_BF16, RN_BF16>(a, q, k, v, gate, s_in, s_out, out, ws, st);
}

}  // namespace rn
