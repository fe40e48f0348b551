// Tile machinery shared by the backward kernels (internal): 64-row tiles of one 256-token
// chunk, products through LDS in float32 (VALU) or on matrix cores (f16 operands, float32
// accumulation), score tiles with the decay and the causal mask, rows rotated back before
// their store. The accumulator of a 64 x 16 NCT product is held as acc[r][j] =
// C[4 ty + r][tx + 16 j] with (ty, tx) = (tid >> 4, tid & 15), which is also the layout of a
// 16x16 MFMA tile (lane: column l16, rows 4g..4g+3; ty = 4 wave + g, tx = l16).
#pragma once
#include "rn_device.h"

namespace rn {
namespace {

constexpr int kBC = 256;      // tokens per stored state (chunk of the backward)

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
constexpr int kLdPH = kBC + 16;     // LDS pitch (half) of P rows: 34 16-byte units, so the
                                    // 16-byte reads of 16 rows x 4 runs are conflict-free

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
      if constexpr (!__is_same(SM, TileShared)) sm.m.P[4 * ty + r][tx + 16 * j] = static_cast<_Float16>(x);
      else sm.P[tx + 16 * j][4 * ty + r] = x;
    }
}

// Buffer offset `off` when `live`, else one past every buffer range (bit 31 set: loads
// return zero, stores are dropped). Formed without a select: the compiler turned selects
// on load offsets into branches around the loads, and at each join it waits for every
// load in flight. (The empty statement only hides the value from the optimizer.)
__device__ __forceinline__ uint32_t live_off(uint32_t off, bool live) {
  uint32_t hi = static_cast<uint32_t>(!live) << 31;
  __asm__("" : "+v"(hi));
  return off | hi;
}

// Sum over the 16 threads (tx = lanes 16k .. 16k+15) that share a row, every lane
// receiving it: DPP moves (VALU only) swap neighbours, swap pairs, mirror within 8 lanes,
// mirror within 16.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);    // lane ^ 1
  x += dpp_mov<0x4E>(x);    // lane ^ 2
  x += dpp_mov<0x141>(x);   // lane i <-> 7 - i within 8
  x += dpp_mov<0x140>(x);   // lane i <-> 15 - i within 16
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


// GroupNorm / gate backward of a 64-row tile whose pre-GroupNorm output o (64 x d_v, in
// the accumulator layout) has been recomputed: per row the gradient before GroupNorm,
// dO = rstd (dxh - mean(dxh) - xh mean(dxh xh)) with dxh = dy w and dy = dout (* swish(g)),
// is passed to store_dO(head offset, element offset within the head, whether the element
// exists, value, row within the tile, column); the gate's gradient is stored; the tile's
// per-column sums of dy xh and dy are added to dgn_w and dgn_b. Without GroupNorm dO is
// dout.
// Element stores through a buffer resource over one head's rows: a store with ok false
// goes to an offset past the range and is dropped, so the stores of a row need no branch
// (a branch would make every later wait also wait for the stores already issued).
constexpr uint32_t kGnSink = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes), 0x00020000);
}
template <int DT>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int i, bool ok, float x) {
  if constexpr (DT == RN_F32) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, live_off(static_cast<uint32_t>(i) * 4, ok), 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, live_off(static_cast<uint32_t>(i) * 2, ok), 0, 0);
  }
}

// dout (and gate) of one row at columns tx + 16 j: all 32 (64) loads are issued before any
// is used, at addresses clamped into the row (columns past d_v read a valid element that
// the caller discards), so no branch separates a load from the others in flight.
template <int DT>
__device__ __forceinline__ float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t voff, int j) {
  if constexpr (DT == RN_F32)
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff * 4 + 64 * j, 0, 0));
  else
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff * 2 + 32 * j, 0, 0));
}
// dout (and gate) of one row (elements roff + tx + 16 j of the head; the row differs
// between the lane groups of a wave): all 32 (64) loads are issued before any is used,
// through buffer resources over the head with one per-lane offset and the column step in
// the immediate, so no branch and no per-element address separates a load from the
// others in flight. Columns past d_v (d_v < 512) read an element of the next row or past
// the range (0); the caller discards them.
template <int IN, int OUTD>
__device__ __forceinline__ void gn_load_row(float (&dov)[32], float (&gav)[32], __amdgpu_buffer_rsrc_t rdo,
                                            __amdgpu_buffer_rsrc_t rga, bool gt, int roff, int tx) {
  const uint32_t voff = static_cast<uint32_t>(roff + tx);
  if (gt) {
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      dov[j] = load_elem<OUTD>(rdo, voff, j);
      gav[j] = load_elem<IN>(rga, voff, j);
    }
  } else {
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      dov[j] = load_elem<OUTD>(rdo, voff, j);
      gav[j] = 0.f;
    }
  }
}

// AFF: the GroupNorm has an affine weight or bias, or their gradients are asked for;
// without it the weights are 1 and 0 and no column sums are kept (128 fewer registers).
template <int IN, int OUTD, bool AFF = true, class SM, class STORE>
__device__ __forceinline__ void gn_backward_tile(SM& sm, const float (&o)[4][32], const CallArgs& a,
                                                 int h, int bh, int r0, int r1, const void* gate,
                                                 const void* dout, void* dgate, float* dgn_w,
                                                 float* dgn_b, STORE store_dO) {
  const int dv = a.dv, N = a.N;
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const struct { int r0, r1; } T{r0, r1};
  const bool gn = a.flags & RN_EPI_GN, gt = a.flags & RN_EPI_GATE;
  // the head's rows (uniform bases: element offsets within a head fit 32 bits)
  const int64_t hoff = int64_t(bh) * N * dv;
  dout = static_cast<const char*>(dout) + hoff * (OUTD == RN_F32 ? 4 : 2);
  if (gate) gate = static_cast<const char*>(gate) + hoff * (IN == RN_F32 ? 4 : 2);
  if (dgate) dgate = static_cast<char*>(dgate) + hoff * (IN == RN_F32 ? 4 : 2);
  const __amdgpu_buffer_rsrc_t rdg = head_rsrc(dgate, int64_t(N) * dv * (IN == RN_F32 ? 4 : 2));
  const __amdgpu_buffer_rsrc_t rdo = head_rsrc(dout, int64_t(N) * dv * (OUTD == RN_F32 ? 4 : 2));
  const __amdgpu_buffer_rsrc_t rga = head_rsrc(gate, int64_t(N) * dv * (IN == RN_F32 ? 4 : 2));
  if (!gn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = T.r0 + 4 * ty + r;
      const bool live = t < T.r1;
      const int roff = (live ? t : T.r0) * dv;
      for (int col = tx; col < dv; col += 16)
        store_dO(hoff, roff + col, live, live ? Elem<OUTD>::load(dout, roff + col) : 0.f, 4 * ty + r, col);
    }
    return;
  }
  // GroupNorm / gate backward, row by row. Per-column sums of dy * xh and dy (for dgn_w,
  // dgn_b) gather in registers over this thread's four rows, then in its own LDS cells
  // (two [16][kLdB] float arrays) for the reduction over the tile.
  const bool sums = AFF && (dgn_w || dgn_b);
  float swa[32], sba[32];
#pragma clang loop unroll(full)
  for (int j = 0; j < 32; ++j) swa[j] = sba[j] = 0.f;
  // affine parameters of this thread's 32 columns; dout, gate and the sigmoid are taken
  // once per element
  float wv[32], bv[32];
#pragma clang loop unroll(full)
  for (int j = 0; j < 32; ++j) {
    const int col = tx + 16 * j;
    if constexpr (!AFF) {
      wv[j] = 1.f;
      bv[j] = 0.f;
      continue;
    }
    wv[j] = (a.gn_w && col < dv) ? a.gn_w[h * dv + col] : 1.f;
    bv[j] = (a.gn_b && col < dv) ? a.gn_b[h * dv + col] : 0.f;
  }
#pragma clang loop unroll(full)
  for (int r = 0; r < 4; ++r) {
    const int t = T.r0 + 4 * ty + r;
    const bool live = t < T.r1;
    const int roff = (live ? t : T.r0) * dv;
    float dov[32], gav[32];
    gn_load_row<IN, OUTD>(dov, gav, rdo, rga, gt, roff, tx);
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
    // dy = dout (* swish(g)); dgate = dout y swish'(g); the row means of dxh = dy w and
    // of dxh xh
    // (all of the row's loads were issued above, so the stores here cost at most one wait)
    float dyv[32];
    float m1 = 0.f, m2 = 0.f;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      const bool ok = live && tx + 16 * j < dv;
      const float xh = (o[r][j] - mean) * rstd;
      const float d0 = dov[j];
      float dy = d0;
      if (gt) {
        const float g = gav[j];
        const float sg = 1.0f / (1.0f + expf(-g));
        dy = d0 * g * sg;
        store_elem<IN>(rdg, roff + tx + 16 * j, ok, d0 * (xh * wv[j] + bv[j]) * sg * (1.0f + g * (1.0f - sg)));
      }
      dy = ok ? dy : 0.f;
      dyv[j] = dy;
      const float dxh = dy * wv[j];
      m1 += dxh;
      m2 += dxh * xh;
      if constexpr (AFF) {
        swa[j] += dy * xh;
        sba[j] += dy;
      }
    }
    m1 = row16_sum(m1) / dv;
    m2 = row16_sum(m2) / dv;
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      const int col = tx + 16 * j;
      const float xh = (o[r][j] - mean) * rstd;
      store_dO(hoff, roff + col, live && col < dv, rstd * (dyv[j] * wv[j] - m1 - xh * m2), 4 * ty + r, col);
    }
  }
  if (sums) {
    float* sw = gn_sw(sm);
    float* sb = gn_sb(sm);
    __syncthreads();   // the products' reads of shared memory are done
#pragma clang loop unroll(full)
    for (int j = 0; j < 32; ++j) {
      sw[ty * kLdB + tx + 16 * j] = swa[j];
      sb[ty * kLdB + tx + 16 * j] = sba[j];
    }
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

}  // namespace
}  // namespace rn
