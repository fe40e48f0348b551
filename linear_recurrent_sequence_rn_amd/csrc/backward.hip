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
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

constexpr int kBC = 256;      // tokens per stored state
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

// ---- tiled products ------------------------------------------------------------------------
// The row kernels work on 64-row tiles of one chunk. 256 threads, (ty, tx) = (tid >> 4,
// tid & 15); a 64 x NC product tile is held as acc[r][j] = C[4 ty + r][tx + 16 j]. The
// reduction dimension streams through LDS in slices of 16: As[k][row], Bs[k][col]; a
// decayed score tile waits in LDS transposed (P[key][row]) to be the next product's A.
constexpr int kR = 64;      // rows per tile
constexpr int kKS = 16;     // reduction slice
constexpr int kLdA = 68;    // LDS pitch (floats) of As and P: rows stay 16-byte aligned
constexpr int kLdB = kMaxDv + 4;

struct alignas(16) TileShared {
  float As[kKS][kLdA];
  float Bs[kKS][kLdB];
  float P[kBC][kLdA];
};

// acc += A (64 x K) B (K x 16 NCT). ga(row, k) and gb(...) return operand elements (zero
// outside the operand); B is addressed gb(k, col) for BM = kBRows (reduction along the
// source's rows) or gb(col, k) for BM = kBCols. With FROMP, A is read from P (whose rows are
// the reduction index) and ga is unused. Each slice's elements are fetched into registers
// one slice ahead, so their global loads overlap the previous slice's arithmetic.
enum { kBRows = 0, kBCols = 1 };
template <int NCT, bool FROMP, int BM, class GA, class GB>
__device__ __forceinline__ void tile_mm(float (&acc)[4][NCT], int K, TileShared& sm, GA ga, GB gb) {
  constexpr int NCB = 16 * NCT;        // B columns
  constexpr int NBE = NCB / 16;        // B elements per thread and slice
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float ra[4], rb[NBE];
  auto fetch = [&](int k0) __attribute__((always_inline)) {
    if constexpr (!FROMP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        ra[i] = ga(e >> 4, k0 + (e & 15));
      }
    }
#pragma unroll
    for (int i = 0; i < NBE; ++i) {
      const int e = tid + 256 * i;
      if constexpr (BM == kBRows) rb[i] = gb(k0 + e / NCB, e % NCB);
      else rb[i] = gb(e >> 4, k0 + (e & 15));
    }
  };
  auto put = [&]() __attribute__((always_inline)) {
    if constexpr (!FROMP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        sm.As[e & 15][e >> 4] = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NBE; ++i) {
      const int e = tid + 256 * i;
      if constexpr (BM == kBRows) sm.Bs[e / NCB][e % NCB] = rb[i];
      else sm.Bs[e & 15][e >> 4] = rb[i];
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += kKS) {
    __syncthreads();   // the previous slice's reads of As / Bs are done
    put();
    __syncthreads();
    if (k0 + kKS < K) fetch(k0 + kKS);
#pragma unroll 4
    for (int kk = 0; kk < kKS; ++kk) {
      float4 av;
      if constexpr (FROMP) av = *reinterpret_cast<const float4*>(&sm.P[k0 + kk][4 * ty]);
      else av = *reinterpret_cast<const float4*>(&sm.As[kk][4 * ty]);
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const float b = sm.Bs[kk][tx + 16 * j];
        acc[0][j] = fmaf(av.x, b, acc[0][j]);
        acc[1][j] = fmaf(av.y, b, acc[1][j]);
        acc[2][j] = fmaf(av.z, b, acc[2][j]);
        acc[3][j] = fmaf(av.w, b, acc[3][j]);
      }
    }
  }
}

template <int NCT>
__device__ __forceinline__ void zero_acc(float (&acc)[4][NCT]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < NCT; ++j) acc[r][j] = 0.f;
}

// ---- the same tile products on matrix cores (bf16 inputs) ------------------------------
// 16x16x32 f16 MFMA with float32 accumulation. The accumulator layout of a 16x16 tile
// (lane: column l16, rows 4g..4g+3) is the layout above: thread 64w + 16g + l16 holds
// rows 16w + 4g + r, i.e. ty = 4w + g, tx = l16. Operands are rounded to IEEE half when
// they are staged: A as As[row][k], B as Bs[col][k] (32 k-values per slice, 8 per lane
// and 16 bytes per read), a score tile as P[row][key].
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kKH = 32;             // reduction slice
constexpr int kLdH = kKH + 8;       // LDS pitch (half) of As and Bs rows
constexpr int kLdPH = kBC + 8;      // LDS pitch (half) of P rows

struct alignas(16) TileSharedH {
  union {
    struct {
      _Float16 As[kR][kLdH];
      _Float16 Bs[kMaxDv][kLdH];
      _Float16 P[kR][kLdPH];
    } m;
    float rot[kR][kMaxDk + 4];             // rows rotated back before their store
    struct {
      float sw[16][kLdB];                  // per-thread sums of the GroupNorm backward
      float sb[16][kLdB];
    } gn;
  };
};

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v;
  v[0] = static_cast<_Float16>(lo);
  v[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// acc += A (64 x K) B (K x 16 NCT) as in tile_mm. Each thread stages runs of 8 consecutive
// k-values: A row tid/4, k 8 (tid%4) ..; B runs are spread so that consecutive threads
// read consecutive source addresses (for BM = kBRows consecutive columns, for kBCols the
// four runs of one column). The next slice is fetched into registers while the MFMAs of
// the current one run.
template <int NCT, bool FROMP, int BM, class GA, class GB>
__device__ __forceinline__ void tile_mm_h(float (&acc)[4][NCT], int K, TileSharedH& sm, GA ga, GB gb) {
  constexpr int NCB = 16 * NCT;            // B columns
  constexpr int NRUN = NCB * 4 / 256;      // B runs of 8 per thread and slice
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  float ra[8], rb[NRUN][8];
  auto bcol = [&](int u) { const int run = tid + 256 * u; return BM == kBRows ? run % NCB : run >> 2; };
  auto bq = [&](int u) { const int run = tid + 256 * u; return BM == kBRows ? run / NCB : run & 3; };
  auto fetch = [&](int k0) __attribute__((always_inline)) {
    if constexpr (!FROMP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = ga(tid >> 2, k0 + 8 * (tid & 3) + i);
    }
#pragma unroll
    for (int u = 0; u < NRUN; ++u) {
      const int col = bcol(u), kq = k0 + 8 * bq(u);
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[u][i] = BM == kBRows ? gb(kq + i, col) : gb(col, kq + i);
    }
  };
  auto put = [&]() __attribute__((always_inline)) {
    if constexpr (!FROMP)
      *reinterpret_cast<u32x4*>(&sm.m.As[tid >> 2][8 * (tid & 3)]) =
          u32x4{pack_h2(ra[0], ra[1]), pack_h2(ra[2], ra[3]), pack_h2(ra[4], ra[5]), pack_h2(ra[6], ra[7])};
#pragma unroll
    for (int u = 0; u < NRUN; ++u)
      *reinterpret_cast<u32x4*>(&sm.m.Bs[bcol(u)][8 * bq(u)]) =
          u32x4{pack_h2(rb[u][0], rb[u][1]), pack_h2(rb[u][2], rb[u][3]), pack_h2(rb[u][4], rb[u][5]),
                pack_h2(rb[u][6], rb[u][7])};
  };
  f32x4 t[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += kKH) {
    __syncthreads();   // the previous slice's reads of As / Bs are done
    put();
    __syncthreads();
    if (k0 + kKH < K) fetch(k0 + kKH);
    f16x8 av;
    if constexpr (FROMP) av = *reinterpret_cast<const f16x8*>(&sm.m.P[16 * w + l16][k0 + 8 * g]);
    else av = *reinterpret_cast<const f16x8*>(&sm.m.As[16 * w + l16][8 * g]);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const f16x8 bv = *reinterpret_cast<const f16x8*>(&sm.m.Bs[16 * j + l16][8 * g]);
      t[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, t[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][j] += t[j][r];
}

// Shared memory and the tile product of one input type: float32 VALU for float32 inputs,
// matrix cores for bf16 inputs.
template <int IN> struct TileOf { using type = TileShared; };
template <> struct TileOf<RN_BF16> { using type = TileSharedH; };

template <int IN, int NCT, bool FROMP, int BM, class SM, class GA, class GB>
__device__ __forceinline__ void tmm(float (&acc)[4][NCT], int K, SM& sm, GA ga, GB gb) {
  if constexpr (IN == RN_BF16) tile_mm_h<NCT, FROMP, BM>(acc, K, sm, ga, gb);
  else tile_mm<NCT, FROMP, BM>(acc, K, sm, ga, gb);
}
__device__ __forceinline__ float* rot_buf(TileShared& sm) { return &sm.P[0][0]; }
__device__ __forceinline__ float* rot_buf(TileSharedH& sm) { return &sm.rot[0][0]; }
__device__ __forceinline__ float* gn_sw(TileShared& sm) { return &sm.Bs[0][0]; }
__device__ __forceinline__ float* gn_sw(TileSharedH& sm) { return &sm.gn.sw[0][0]; }
__device__ __forceinline__ float* gn_sb(TileShared& sm) { return &sm.P[0][0]; }
__device__ __forceinline__ float* gn_sb(TileSharedH& sm) { return &sm.gn.sb[0][0]; }

// Decayed, masked score tile -> P (transposed): P[key - key0][row] for the tile's rows
// row0 + 4ty + r and keys key0 + tx + 16 j < key_end. FORWARD: keys s <= t (o, dq);
// otherwise later rows t >= s (dk, dv: the tile's rows are the keys s).
template <bool FORWARD, class SM>
__device__ __forceinline__ void store_scores(SM& sm, const float (&m)[4][16], int row0,
                                             int row_end, int key0, int key_end, float lg,
                                             float alpha) {
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  __syncthreads();   // the previous product's reads of P are done
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = row0 + 4 * ty + r, key = key0 + tx + 16 * j;
      const int dist = FORWARD ? row - key : key - row;
      const bool ok = row < row_end && key < key_end && dist >= 0;
      const float x = ok ? alpha * m[r][j] * gpow(lg, float(dist)) : 0.f;
      if constexpr (__is_same(SM, TileSharedH)) sm.m.P[4 * ty + r][tx + 16 * j] = static_cast<_Float16>(x);
      else sm.P[tx + 16 * j][4 * ty + r] = x;
    }
}

// Sum over the 16 threads (tx) that share a row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

// Tile of grid.x: chunk c = [c0, c1), rows [r0, r1) (64-row tile within the chunk).
struct TileRows {
  int c, c0, c1, r0, r1;
};
__device__ __forceinline__ TileRows tile_rows(int N) {
  TileRows t;
  t.c = blockIdx.x / (kBC / kR);
  t.c0 = t.c * kBC;
  t.c1 = min(N, t.c0 + kBC);
  t.r0 = t.c0 + kR * (blockIdx.x % (kBC / kR));
  t.r1 = min(t.c1, t.r0 + kR);
  return t;
}

// Rotates a row tile of gradients back by -p and stores it: the tile goes through LDS
// (P, free after the products) so that each thread then takes whole coordinate pairs.
template <int IN, class SM>
__device__ __forceinline__ void store_rotated(SM& sm, const float (&g)[4][16], const CallArgs& a,
                                              int64_t p0, int bh, int r0, int r1, void* dst) {
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15, dk = a.dk;
  float* buf = rot_buf(sm);   // [64 rows][kMaxDk + 4]
  constexpr int ld = kMaxDk + 4;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 16; ++j) buf[(4 * ty + r) * ld + tx + 16 * j] = g[r][j];
  __syncthreads();
  for (int e = threadIdx.x; e < kR * (dk / 2); e += 256) {
    const int row = e / (dk / 2), jp = e % (dk / 2), t = r0 + row;
    if (t >= r1) continue;
    float cs, sn;
    angle_cs(p0 + t, a.ap.theta[jp], &cs, &sn);
    const float g0 = buf[row * ld + 2 * jp], g1 = buf[row * ld + 2 * jp + 1];
    const int64_t off = (int64_t(bh) * a.N + t) * dk + 2 * jp;
    Elem<IN>::store(dst, off, g0 * cs + g1 * sn);
    Elem<IN>::store(dst, off + 1, -g0 * sn + g1 * cs);
  }
}

// ---- recompute o, then the epilogue backward --------------------------------------------
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
  const bool gn = a.flags & RN_EPI_GN, gt = a.flags & RN_EPI_GATE;
  if (!gn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = T.r0 + 4 * ty + r;
      if (t >= T.r1) continue;
      const int64_t roff = (int64_t(bh) * N + t) * dv;
      for (int col = tx; col < dv; col += 16) dO[roff + col] = Elem<OUTD>::load(dout, roff + col);
    }
    return;
  }
  // GroupNorm / gate backward, row by row. Per-column sums of dy * xh and dy (for dgn_w,
  // dgn_b) gather in this thread's own LDS cells: Bs[ty][col] and P viewed as [16][kLdB].
  float* sw = gn_sw(sm);
  float* sb = gn_sb(sm);
  __syncthreads();
#pragma clang loop unroll(full)
  for (int j = 0; j < 32; ++j) {
    sw[ty * kLdB + tx + 16 * j] = 0.f;
    sb[ty * kLdB + tx + 16 * j] = 0.f;
  }
  auto gnw = [&](int col) { return a.gn_w ? a.gn_w[h * dv + col] : 1.f; };
  auto gnb = [&](int col) { return a.gn_b ? a.gn_b[h * dv + col] : 0.f; };
#pragma clang loop unroll(full)
  for (int r = 0; r < 4; ++r) {
    const int t = T.r0 + 4 * ty + r;
    const bool live = t < T.r1;
    const int64_t roff = (int64_t(bh) * N + (live ? t : T.r0)) * dv;
    float s1 = 0.f;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) s1 += (tx + 16 * j < dv) ? o[r][j] : 0.f;
    const float mean = row16_sum(s1) / dv;
    float s2 = 0.f;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      const float dd = o[r][j] - mean;
      s2 += (tx + 16 * j < dv) ? dd * dd : 0.f;
    }
    const float rstd = 1.0f / sqrtf(row16_sum(s2) / dv + a.eps);
    // dy = dout (* swish(g)); dxh = dy * w; the row means of dxh and dxh * xh
    auto dy_of = [&](int j, float xh) {
      const int col = tx + 16 * j;
      float dy = Elem<OUTD>::load(dout, roff + col);
      if (gt) {
        const float g = Elem<IN>::load(gate, roff + col);
        const float sg = 1.0f / (1.0f + expf(-g));
        dy *= g * sg;
      }
      (void)xh;
      return dy;
    };
    float m1 = 0.f, m2 = 0.f;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      const int col = tx + 16 * j;
      if (live && col < dv) {
      const float xh = (o[r][j] - mean) * rstd;
      const float dy = dy_of(j, xh);
      const float dxh = dy * gnw(col);
      m1 += dxh;
      m2 += dxh * xh;
      sw[ty * kLdB + col] += dy * xh;
      sb[ty * kLdB + col] += dy;
      if (gt) {
        const float g = Elem<IN>::load(gate, roff + col);
        const float sg = 1.0f / (1.0f + expf(-g));
        const float d0 = Elem<OUTD>::load(dout, roff + col);
        Elem<IN>::store(dgate, roff + col, d0 * (xh * gnw(col) + gnb(col)) * sg * (1.0f + g * (1.0f - sg)));
      }
      }
    }
    m1 = row16_sum(m1) / dv;
    m2 = row16_sum(m2) / dv;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      const int col = tx + 16 * j;
      if (live && col < dv) {
        const float xh = (o[r][j] - mean) * rstd;
        const float dxh = dy_of(j, xh) * gnw(col);
        dO[roff + col] = rstd * (dxh - m1 - xh * m2);
      }
    }
  }
  if (dgn_w || dgn_b) {
    __syncthreads();
    for (int col = threadIdx.x; col < dv; col += 256) {
      float xw = 0.f, xb = 0.f;
      for (int y = 0; y < 16; ++y) {
        xw += sw[y * kLdB + col];
        xb += sb[y * kLdB + col];
      }
      if (dgn_w) atomicAdd(&dgn_w[h * dv + col], xw);
      if (dgn_b) atomicAdd(&dgn_b[h * dv + col], xb);
    }
  }
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
