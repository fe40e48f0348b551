// Gradients of the chunkwise retention (with the optional GroupNorm + swish gate
// epilogue) with respect to q, k, v, the gate, the initial state and the GroupNorm
// affine parameters: plain float32 kernels for every shape.
//
// Per head, with states kept at chunk starts (chunks of kBC tokens; the gradients do not
// depend on the caller's chunk size, like the forward result):
//   S_c       state at the start of chunk c (forward scan, stored)
//   o_t       recomputed: alpha [sum_{c0<=s<=t} gamma^(t-s)(Qh_t.Kh_s) V_s + xi_t Qh_t S_c]
//   dO_t      GroupNorm and gate backward of dout_t (stored), and dgate_t
//   G_c       gradient reaching S_c (reverse scan, stored as G_{c+1} for chunk c):
//             G_c = gamma^L G_{c+1} + alpha sum_{t in c} xi_t Qh_t^T dO_t, G_end = dstate_out
//   dQh_t = alpha sum_{c0<=s<=t} gamma^(t-s)(dO_t.V_s) Kh_s + alpha xi_t S_c dO_t
//   dKh_s = alpha sum_{s<=t<c1} gamma^(t-s)(dO_t.V_s) Qh_t + zeta_s G_{c+1} V_s
//   dV_s  = alpha sum_{s<=t<c1} gamma^(t-s)(Qh_t.Kh_s) dO_t + zeta_s G_{c+1}^T Kh_s
//   dq = rot(dQh, -p), dk = rot(dKh, -p), dstate_in = G_0
// with xi_t = gamma^(t-c0+1) and zeta_s = gamma^(c1-1-s) in chunk [c0, c1). Qh and Kh are
// rotated once into the workspace (float32) by the first kernel; the row quantities are
// computed per 64-row tile of a chunk as small products through LDS. These are
// the chunkwise equation's recurrence differentiated (hwhale notes: chunkwise equation
// and ChunkwiseRetention listing; GroupNorm per head and swish gate of the multi-scale
// layer).
#include "backward_tiles.h"
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

constexpr int kTD = 32;       // state tile: d_k rows
constexpr int kTE = 64;       // state tile: d_v columns
constexpr int kTB = 64;       // tokens per scan step
constexpr int kRows = 16;     // rows per workgroup of the row kernels

// Rotated pair (2j, 2j+1) of row `off` of x at position p, times `scale`.
template <int IN>
__device__ __forceinline__ void rot_pair_s(const void* x, int64_t off, int j, int64_t p,
                                           float theta, float scale, float* r0, float* r1) {
  const float a = Elem<IN>::load(x, off + 2 * j), b = Elem<IN>::load(x, off + 2 * j + 1);
  float c, s;
  angle_cs(p, theta, &c, &s);
  *r0 = (a * c - b * s) * scale;
  *r1 = (a * s + b * c) * scale;
}

// ---- rotation pre-pass: Qh, Kh in float32 -------------------------------------------------
// Grid: (row blocks of kRows, b*H + h); 256 threads over the coordinate pairs.
template <int IN>
__global__ void __launch_bounds__(256) bw_rotate(CallArgs a, const void* q, const void* k,
                                                 float* qh, float* kh) {
  const int dk = a.dk, N = a.N;
  const int bh = blockIdx.y;
  const int64_t p0 = seq_pos0(a, bh / a.H);
  for (int r = 0; r < kRows; ++r) {
    const int t = blockIdx.x * kRows + r;
    if (t >= N) break;
    const int64_t off = (int64_t(bh) * N + t) * dk;
    for (int j = threadIdx.x; j < dk / 2; j += 256) {
      rot_pair_s<IN>(q, off, j, p0 + t, a.ap.theta[j], 1.f, &qh[off + 2 * j], &qh[off + 2 * j + 1]);
      rot_pair_s<IN>(k, off, j, p0 + t, a.ap.theta[j], 1.f, &kh[off + 2 * j], &kh[off + 2 * j + 1]);
    }
  }
}

// ---- scans --------------------------------------------------------------------------------
// REV = 0: forward state scan. X = Kh scaled by zeta, Y = v; writes S_c (the state at
//          the start of chunk c) for every chunk; starts from state_in (or zeros).
// REV = 1: gradient scan, chunks in reverse. X = alpha Qh scaled by xi, Y = dO (float32
//          workspace); writes G_{c+1} (the gradient reaching the end of chunk c) for every
//          chunk and the final G_0 to dstate_in; starts from dstate_out (or zeros).
// Grid: (state tiles of 32 x 64, b*H + h); 256 threads, 8 elements each.
template <int IN, int REV>
__global__ void __launch_bounds__(256) bw_scan(CallArgs a, const float* xsrc, const void* ysrc,
                                               const float* init, float* store, float* final_out) {
  __shared__ float xs[kTB][kTD];
  __shared__ float ys[kTB][kTE];
  const int dk = a.dk, dv = a.dv, N = a.N;
  const int ntE = (dv + kTE - 1) / kTE;
  const int d0 = kTD * (blockIdx.x / ntE), e0 = kTE * (blockIdx.x % ntE);
  const int bh = blockIdx.y, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const int64_t nS = int64_t(dk) * dv;
  const int te = threadIdx.x & 63, tr = threadIdx.x >> 6;
  const int e = e0 + te;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = d0 + tr + 4 * i;
    acc[i] = (init && d < dk && e < dv) ? init[bh * nS + int64_t(d) * dv + e] : 0.f;
  }
  for (int step = 0; step < nch; ++step) {
    const int c = REV ? nch - 1 - step : step;
    const int c0 = c * kBC, c1 = min(N, c0 + kBC), L = c1 - c0;
    // store this chunk's boundary value, then apply the chunk
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = d0 + tr + 4 * i;
      if (d < dk && e < dv) store[(bh * nch + c) * nS + int64_t(d) * dv + e] = acc[i];
    }
    const float gL = gpow(lg, float(L));
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= gL;
    for (int t0 = c0; t0 < c1; t0 += kTB) {
      const int nt = min(kTB, c1 - t0);
      __syncthreads();
      // X rows: kTD/2 pairs x nt tokens
      for (int idx = threadIdx.x; idx < kTB * (kTD / 2); idx += 256) {
        const int tt = idx / (kTD / 2), pr = idx % (kTD / 2), j = d0 / 2 + pr;
        float r0 = 0.f, r1 = 0.f;
        if (tt < nt && 2 * j < dk) {
          const int t = t0 + tt, jc = t - c0;
          const float w = REV ? a.alpha * gpow(lg, float(jc + 1)) : gpow(lg, float(L - 1 - jc));
          const int64_t off = (int64_t(bh) * N + t) * dk + 2 * j;
          r0 = xsrc[off] * w;
          r1 = xsrc[off + 1] * w;
        }
        xs[tt][2 * pr] = r0;
        xs[tt][2 * pr + 1] = r1;
      }
      for (int idx = threadIdx.x; idx < kTB * kTE; idx += 256) {
        const int tt = idx / kTE, ee = e0 + idx % kTE;
        float y = 0.f;
        if (tt < nt && ee < dv) {
          const int64_t off = (int64_t(bh) * N + t0 + tt) * dv + ee;
          y = REV ? static_cast<const float*>(ysrc)[off] : Elem<IN>::load(ysrc, off);
        }
        ys[tt][idx % kTE] = y;
      }
      __syncthreads();
      for (int tt = 0; tt < nt; ++tt) {
        const float y = ys[tt][te];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(xs[tt][tr + 4 * i], y, acc[i]);
      }
    }
  }
  if (final_out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = d0 + tr + 4 * i;
      if (d < dk && e < dv) final_out[bh * nS + int64_t(d) * dv + e] = acc[i];
    }
  }
}

// ---- tiled products ---------------------------------------------------------------------
// Grid: (64-row tiles, b*H + h). o_R = alpha (Qh_R Kh_C^T (.) D) V_C + alpha xi Qh_R S_c, then
// the GroupNorm / gate backward per row: dO (float32 workspace), dgate, and the tile's
// sums added to dgn_w / dgn_b.
template <int IN, int OUTD>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bw_dout(CallArgs a, const float* Qh, const float* Kh,
                                               const void* v, const void* gate, const void* dout,
                                               const float* S, float* dO, void* dgate,
                                               float* dgn_w, float* dgn_b) {
  __shared__ typename TileOf<IN>::type sm;
  const int dk = a.dk, dv = a.dv, N = a.N;
  const TileRows T = tile_rows(N);
  if (T.r0 >= T.r1) return;
  const int bh = blockIdx.y, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const float* Qb = Qh + int64_t(bh) * N * dk;
  const float* Kb = Kh + int64_t(bh) * N * dk;
  const float* Sc = S + (int64_t(bh) * nch + T.c) * int64_t(dk) * dv;
  const int nkey = T.r1 - T.c0;   // keys c0 .. r1-1
  float m[4][16];
  zero_acc(m);
  tmm<IN, 16, false, kBCols>(m, dk, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          return (T.r0 + row < T.r1 && kk < dk) ? Qb[int64_t(T.r0 + row) * dk + kk] : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < nkey && kk < dk) ? Kb[int64_t(T.c0 + col) * dk + kk] : 0.f; });
  store_scores<true>(sm, m, T.r0, T.r1, T.c0, T.r1, lg, a.alpha);
  float o[4][32];
  zero_acc(o);
  tmm<IN, 32, true, kBRows>(o, (nkey + kKS - 1) / kKS * kKS, sm, [](int, int) { return 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < nkey && col < dv) ? Elem<IN>::load(v, (int64_t(bh) * N + T.c0 + kk) * dv + col) : 0.f; });
  tmm<IN, 32, false, kBRows>(o, dk, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          const int t = T.r0 + row;
          return (t < T.r1 && kk < dk) ? a.alpha * gpow(lg, float(t - T.c0 + 1)) * Qb[int64_t(t) * dk + kk] : 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < dk && col < dv) ? Sc[int64_t(kk) * dv + col] : 0.f; });
  gn_backward_tile<IN, OUTD>(sm, o, a, h, bh, T.r0, T.r1, gate, dout, dgate, dgn_w, dgn_b,
      [&](int64_t hoff, int i, bool ok, float x, int, int) __attribute__((always_inline)) {
        if (ok) dO[hoff + i] = x;
      });
}

// ---- dq -----------------------------------------------------------------------------------
// dQh_R = [alpha (dO_R V_C^T) (.) D] Kh_C + alpha xi dO_R S_c^T, rotated back.
template <int IN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bw_dq(CallArgs a, const float* Kh, const void* v,
                                             const float* dO, const float* S, void* dq) {
  __shared__ typename TileOf<IN>::type sm;
  const int dk = a.dk, dv = a.dv, N = a.N;
  const TileRows T = tile_rows(N);
  if (T.r0 >= T.r1) return;
  const int bh = blockIdx.y, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const float* Kb = Kh + int64_t(bh) * N * dk;
  const float* Db = dO + int64_t(bh) * N * dv;
  const float* Sc = S + (int64_t(bh) * nch + T.c) * int64_t(dk) * dv;
  const int nkey = T.r1 - T.c0;
  float m[4][16];
  zero_acc(m);
  tmm<IN, 16, false, kBCols>(m, dv, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          return (T.r0 + row < T.r1 && kk < dv) ? Db[int64_t(T.r0 + row) * dv + kk] : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < nkey && kk < dv) ? Elem<IN>::load(v, (int64_t(bh) * N + T.c0 + col) * dv + kk) : 0.f; });
  store_scores<true>(sm, m, T.r0, T.r1, T.c0, T.r1, lg, a.alpha);
  float g[4][16];
  zero_acc(g);
  tmm<IN, 16, true, kBRows>(g, (nkey + kKS - 1) / kKS * kKS, sm, [](int, int) { return 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < nkey && col < dk) ? Kb[int64_t(T.c0 + kk) * dk + col] : 0.f; });
  tmm<IN, 16, false, kBCols>(g, dv, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          const int t = T.r0 + row;
          return (t < T.r1 && kk < dv) ? a.alpha * gpow(lg, float(t - T.c0 + 1)) * Db[int64_t(t) * dv + kk] : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < dk && kk < dv) ? Sc[int64_t(col) * dv + kk] : 0.f; });
  store_rotated<IN>(sm, g, a, seq_pos0(a, bh / a.H), bh, T.r0, T.r1, dq);
}

// ---- dk ------------------------------------------------------------------------------------
// Tile rows are keys s; later rows t in [s, c1): dKh_R = [alpha (V_R dO_T^T) (.) D'] Qh_T
// + zeta_s V_R G_{c+1}^T, rotated back.
template <int IN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bw_dk(CallArgs a, const float* Qh, const void* v,
                                             const float* dO, const float* G, void* dk_) {
  __shared__ typename TileOf<IN>::type sm;
  const int dk = a.dk, dv = a.dv, N = a.N;
  const TileRows T = tile_rows(N);
  if (T.r0 >= T.r1) return;
  const int bh = blockIdx.y, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const float* Qb = Qh + int64_t(bh) * N * dk;
  const float* Db = dO + int64_t(bh) * N * dv;
  const float* Gc = G + (int64_t(bh) * nch + T.c) * int64_t(dk) * dv;
  const int nlater = T.c1 - T.r0;   // rows r0 .. c1-1
  float m[4][16];
  zero_acc(m);
  tmm<IN, 16, false, kBCols>(m, dv, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          return (T.r0 + row < T.r1 && kk < dv) ? Elem<IN>::load(v, (int64_t(bh) * N + T.r0 + row) * dv + kk) : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < nlater && kk < dv) ? Db[int64_t(T.r0 + col) * dv + kk] : 0.f; });
  store_scores<false>(sm, m, T.r0, T.r1, T.r0, T.c1, lg, a.alpha);
  float g[4][16];
  zero_acc(g);
  tmm<IN, 16, true, kBRows>(g, (nlater + kKS - 1) / kKS * kKS, sm, [](int, int) { return 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < nlater && col < dk) ? Qb[int64_t(T.r0 + kk) * dk + col] : 0.f; });
  tmm<IN, 16, false, kBCols>(g, dv, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          const int s = T.r0 + row;
          return (s < T.r1 && kk < dv) ? gpow(lg, float(T.c1 - 1 - s)) * Elem<IN>::load(v, (int64_t(bh) * N + s) * dv + kk) : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < dk && kk < dv) ? Gc[int64_t(col) * dv + kk] : 0.f; });
  store_rotated<IN>(sm, g, a, seq_pos0(a, bh / a.H), bh, T.r0, T.r1, dk_);
}

// ---- dv ------------------------------------------------------------------------------------
// dV_R = [alpha (Kh_R Qh_T^T) (.) D'] dO_T + zeta_s Kh_R G_{c+1}.
template <int IN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bw_dv(CallArgs a, const float* Qh, const float* Kh,
                                             const float* dO, const float* G, void* dv_) {
  __shared__ typename TileOf<IN>::type sm;
  const int dk = a.dk, dv = a.dv, N = a.N;
  const TileRows T = tile_rows(N);
  if (T.r0 >= T.r1) return;
  const int bh = blockIdx.y, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const float* Qb = Qh + int64_t(bh) * N * dk;
  const float* Kb = Kh + int64_t(bh) * N * dk;
  const float* Db = dO + int64_t(bh) * N * dv;
  const float* Gc = G + (int64_t(bh) * nch + T.c) * int64_t(dk) * dv;
  const int nlater = T.c1 - T.r0;
  float m[4][16];
  zero_acc(m);
  tmm<IN, 16, false, kBCols>(m, dk, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          return (T.r0 + row < T.r1 && kk < dk) ? Kb[int64_t(T.r0 + row) * dk + kk] : 0.f; },
      [&](int col, int kk) __attribute__((always_inline)) {
          return (col < nlater && kk < dk) ? Qb[int64_t(T.r0 + col) * dk + kk] : 0.f; });
  store_scores<false>(sm, m, T.r0, T.r1, T.r0, T.c1, lg, a.alpha);
  float o[4][32];
  zero_acc(o);
  tmm<IN, 32, true, kBRows>(o, (nlater + kKS - 1) / kKS * kKS, sm, [](int, int) { return 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < nlater && col < dv) ? Db[int64_t(T.r0 + kk) * dv + col] : 0.f; });
  tmm<IN, 32, false, kBRows>(o, dk, sm,
      [&](int row, int kk) __attribute__((always_inline)) {
          const int s = T.r0 + row;
          return (s < T.r1 && kk < dk) ? gpow(lg, float(T.c1 - 1 - s)) * Kb[int64_t(s) * dk + kk] : 0.f; },
      [&](int kk, int col) __attribute__((always_inline)) {
          return (kk < dk && col < dv) ? Gc[int64_t(kk) * dv + col] : 0.f; });
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = T.r0 + 4 * ty + r;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int col = tx + 16 * j;
      if (s < T.r1 && col < dv) Elem<IN>::store(dv_, (int64_t(bh) * N + s) * dv + col, o[r][j]);
    }
  }
}

__global__ void fill_zero(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

size_t align256b(size_t x) { return (x + 255) & ~size_t(255); }

struct BwLayout {
  size_t S, G, dO, Qh, Kh, total;
};
BwLayout bw_layout(const CallArgs& a) {
  const size_t nch = (a.N + kBC - 1) / kBC;
  const size_t heads = size_t(a.B) * a.H;
  const size_t states = align256b(heads * nch * a.dk * a.dv * sizeof(float));
  const size_t rows_k = align256b(heads * size_t(a.N) * a.dk * sizeof(float));
  BwLayout L;
  L.S = 0;
  L.G = L.S + states;
  L.dO = L.G + states;
  L.Qh = L.dO + align256b(heads * size_t(a.N) * a.dv * sizeof(float));
  L.Kh = L.Qh + rows_k;
  L.total = L.Kh + rows_k;
  return L;
}

template <int IN, int OUTD>
hipError_t launch_bw_t(const CallArgs& a, const BwArgs& x, void* ws, hipStream_t st) {
  const BwLayout L = bw_layout(a);
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* S = reinterpret_cast<float*>(w + L.S);
  float* G = reinterpret_cast<float*>(w + L.G);
  float* dO = reinterpret_cast<float*>(w + L.dO);
  float* Qh = reinterpret_cast<float*>(w + L.Qh);
  float* Kh = reinterpret_cast<float*>(w + L.Kh);
  const int BH = a.B * a.H;
  const dim3 gscan(((a.dk + kTD - 1) / kTD) * ((a.dv + kTE - 1) / kTE), BH);
  const dim3 grows((a.N + kRows - 1) / kRows, BH);
  const dim3 gtiles(((a.N + kBC - 1) / kBC) * (kBC / kR), BH);
  hipLaunchKernelGGL((bw_rotate<IN>), grows, dim3(256), 0, st, a, x.q, x.k, Qh, Kh);
  hipLaunchKernelGGL((bw_scan<IN, 0>), gscan, dim3(256), 0, st, a, static_cast<const float*>(Kh),
                     x.v, x.state_in, S, static_cast<float*>(nullptr));
  const bool gn = a.flags & RN_EPI_GN;
  if (gn) {
    if (x.dgn_w) hipLaunchKernelGGL(fill_zero, dim3(8), dim3(256), 0, st, x.dgn_w, int64_t(a.H) * a.dv);
    if (x.dgn_b) hipLaunchKernelGGL(fill_zero, dim3(8), dim3(256), 0, st, x.dgn_b, int64_t(a.H) * a.dv);
  }
  hipLaunchKernelGGL((bw_dout<IN, OUTD>), gtiles, dim3(256), 0, st, a, static_cast<const float*>(Qh),
                     static_cast<const float*>(Kh), x.v, x.gate, x.dout, S, dO, x.dgate, x.dgn_w,
                     x.dgn_b);
  hipLaunchKernelGGL((bw_scan<IN, 1>), gscan, dim3(256), 0, st, a, static_cast<const float*>(Qh),
                     static_cast<const void*>(dO), x.dstate_out, G, x.dstate_in);
  hipLaunchKernelGGL((bw_dq<IN>), gtiles, dim3(256), 0, st, a, static_cast<const float*>(Kh), x.v,
                     static_cast<const float*>(dO), static_cast<const float*>(S), x.dq);
  hipLaunchKernelGGL((bw_dk<IN>), gtiles, dim3(256), 0, st, a, static_cast<const float*>(Qh), x.v,
                     static_cast<const float*>(dO), static_cast<const float*>(G), x.dk);
  hipLaunchKernelGGL((bw_dv<IN>), gtiles, dim3(256), 0, st, a, static_cast<const float*>(Qh),
                     static_cast<const float*>(Kh), static_cast<const float*>(dO),
                     static_cast<const float*>(G), x.dv);
  return hipGetLastError();
}

}  // namespace

size_t backward_ws_bytes(const CallArgs& a) { return bw_layout(a).total; }

hipError_t launch_backward(const CallArgs& a, int in_dt, int out_dt, const BwArgs& x, void* ws,
                           hipStream_t st) {
  if (in_dt == RN_F32)
    return out_dt == RN_F32 ? launch_bw_t<RN_F32, RN_F32>(a, x, ws, st)
                            : launch_bw_t<RN_F32, RN_BF16>(a, x, ws, st);
  return out_dt == RN_F32 ? launch_bw_t<RN_BF16, RN_F32>(a, x, ws, st)
                          : launch_bw_t<RN_BF16, RN_BF16>(a, x, ws, st);
}

}  // namespace rn
