// Matrix-core path of the chunkwise backward for bf16 inputs with d_k and d_v multiples of
// 8: the same gradients as the float32 path (the chunkwise recurrence differentiated; hwhale
// notes: chunkwise equation and ChunkwiseRetention listing; GroupNorm per head and swish
// gate of the multi-scale layer), with every product on 16x16x32 f16 MFMA and float32
// accumulation.
//
// Every product operand is a row-major half matrix whose reduction index is contiguous,
// so that each lane stages 8 consecutive values with one 16-byte load. The reductions run
// over d_k, d_v or tokens, so a prep pass writes the rotated rows of q and k in half both
// row-major ([N][d_k]) and transposed ([d_k][Np], tokens contiguous), and v transposed;
// the GroupNorm backward writes dO row-major and a second pass transposes it; the state
// scans write each chunk's state in both orientations. Np is N rounded up to 64 and the
// transposed copies are zero past N, so a reduction over tokens may read up to the next
// multiple of 32 (the scores or weights there are zero).
//
// Per head (chunks of 256 tokens, c0 its first token, c1 one past its last):
//   scan (forward)  S_c for every chunk: S <- gamma^L S + sum_s gamma^(c1-1-s) Kh_s^T V_s
//   dout            o recomputed per 64-row tile, then the GroupNorm / gate backward -> dO
//   scan (reverse)  G_{c+1} for every chunk: G <- gamma^L G + alpha sum_t gamma^(t-c0+1) Qh_t^T dO_t
//   dq  = [alpha (dO V^T) (.) D] Kh + alpha xi dO S_c^T,   rotated back
//   dk  = [alpha (V dO^T) (.) D'] Qh + zeta V G_{c+1}^T,   rotated back
//   dv  = [alpha (Kh Qh^T) (.) D'] dO + zeta Kh G_{c+1}
#include "backward_tiles.h"
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Row-major source of half (or, for the input v, bf16) values: element (r, c) at
// p[r * pitch + c]; rows at or past `rows` read as zeros.
struct Src {
  const uint16_t* p;
  int64_t pitch;
  int rows;
  bool bf;
};

__device__ __forceinline__ uint16_t h_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t x) {
  return pack_h2(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
}
__device__ __forceinline__ u32x4 bf8_to_h8(u32x4 x) {
  const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
  return u32x4{bf2_to_h2(x0), bf2_to_h2(x1), bf2_to_h2(x2), bf2_to_h2(x3)};
}
// (The halves are taken apart with integer shifts: a bit_cast of each vector element to a
// pair of halves, in an unrolled loop, was compiled to reuse element 0 for all four.)
__device__ __forceinline__ float h_to_f(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xffffu)));
}
__device__ __forceinline__ u32x4 scale8(u32x4 x, const float* f) {
  const uint32_t x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
  return u32x4{pack_h2(h_to_f(x0) * f[0], h_to_f(x0 >> 16) * f[1]),
               pack_h2(h_to_f(x1) * f[2], h_to_f(x1 >> 16) * f[3]),
               pack_h2(h_to_f(x2) * f[4], h_to_f(x2 >> 16) * f[5]),
               pack_h2(h_to_f(x3) * f[6], h_to_f(x3 >> 16) * f[7])};
}
// 8 values (r, c .. c+7) as half; zero for rows past the source or when `live` is false.
__device__ __forceinline__ u32x4 run8(const Src& s, int r, int64_t c, bool live = true) {
  if (!live || r >= s.rows) return u32x4{0u, 0u, 0u, 0u};
  const u32x4 x = *reinterpret_cast<const u32x4*>(s.p + r * s.pitch + c);
  return s.bf ? bf8_to_h8(x) : x;
}
// Raw 16 bytes (r, c .. c+7) through a buffer resource over the source: rows past it read
// as zero, and so does a run that is not `live` (sent past the range). No branch, so the
// loads of a slice stay in flight together; the bf16 -> half conversion is the caller's.
constexpr uint32_t kRunSink = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t src_rsrc(const Src& s) {
  const int64_t bytes = int64_t(s.rows) * s.pitch * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(s.p), 0,
                                           static_cast<int>(bytes > 0x7fffffff ? 0x7fffffff : bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 raw8(__amdgpu_buffer_rsrc_t r, int64_t pitch, int row, int64_t c, bool live) {
  const uint32_t off = live_off(static_cast<uint32_t>((row * pitch + c) * 2), live);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// acc += A B over k < K, A (64 x K) either P (FROMP) or rows ar0 + i of A scaled by
// amul * gamma^(ae0 + aesg i) (log2 gamma = alg), B (K x 16 NCT) given by its columns:
// column n is row br0 + n of B, read from column bc0 on. Without FROMP, K is a multiple of
// 8 and runs at or past K read as zeros; with FROMP the scores past the product's extent
// are zero. The next slice is fetched into registers while the MFMAs of the current run.
template <int NCT, bool FROMP, int NSET = 1, class SM>
__device__ __forceinline__ void tmm16(float (&acc)[4][NCT], int K, SM& sm, const Src& A,
                                      int ar0, float amul, float alg, int ae0, int aesg,
                                      const Src& B, int br0, int bc0) {
  constexpr int NRUN = NCT / 4;   // B runs of 8 per thread and slice (16 NCT columns x 4 runs)
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const int arow = tid >> 2, aq = tid & 3;
  const bool scaled = !FROMP && (aesg != 0 || amul != 1.f);
  float af[8];
  {
    const float f = amul * exp2f(alg * float(ae0 + aesg * arow));
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = f;
  }
  // NSET register sets: the NSET slices after slice k0 are in flight while it computes
  static_assert(NSET == 1 || NSET == 2, "one or two register sets");
  u32x4 ra[NSET], rb[NSET][NRUN];
#pragma unroll
  for (int i = 0; i < NSET; ++i) ra[i] = u32x4{0u, 0u, 0u, 0u};
  const __amdgpu_buffer_rsrc_t rsa = src_rsrc(A), rsb = src_rsrc(B);
  auto fetch = [&](int k0, int set) __attribute__((always_inline)) {
    if constexpr (!FROMP) ra[set] = raw8(rsa, A.pitch, ar0 + arow, k0 + 8 * aq, k0 + 8 * aq < K);
#pragma unroll
    for (int u = 0; u < NRUN; ++u) {
      const int run = tid + 256 * u, n = run >> 2, kq = k0 + 8 * (run & 3);
      rb[set][u] = raw8(rsb, B.pitch, br0 + n, int64_t(bc0) + kq, kq < K);
    }
  };
  auto put = [&](int set) __attribute__((always_inline)) {
    if constexpr (!FROMP) {
      const u32x4 x = A.bf ? bf8_to_h8(ra[set]) : ra[set];
      *reinterpret_cast<u32x4*>(&sm.m.As[arow][8 * aq]) = scaled ? scale8(x, af) : x;
    }
#pragma unroll
    for (int u = 0; u < NRUN; ++u) {
      const int run = tid + 256 * u;
      *reinterpret_cast<u32x4*>(&sm.m.Bs[run >> 2][8 * (run & 3)]) = B.bf ? bf8_to_h8(rb[set][u]) : rb[set][u];
    }
  };
  f32x4 t[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one slice: stage the set, refill it with the slice NSET ahead, multiply
  auto slice = [&](int k0, int set) __attribute__((always_inline)) {
    __syncthreads();   // the previous slice's reads of As / Bs are done
    put(set);
    __syncthreads();
    fetch(k0 + NSET * kKH, set);
    f16x8 av;
    if constexpr (FROMP) av = *reinterpret_cast<const f16x8*>(&sm.m.P[16 * w + l16][k0 + 8 * g]);
    else av = *reinterpret_cast<const f16x8*>(&sm.m.As[16 * w + l16][8 * g]);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const f16x8 bv = *reinterpret_cast<const f16x8*>(&sm.m.Bs[16 * j + l16][8 * g]);
      t[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, t[j], 0, 0, 0);
    }
  };
  // with two sets, slices go in pairs with no branch between them: K is rounded up to 64,
  // the runs past K read as zeros (and, with FROMP, so do the scores past the product's
  // extent)
  fetch(0, 0);
  if constexpr (NSET == 2) {
    fetch(kKH, 1);
    for (int k0 = 0; k0 < K; k0 += 2 * kKH) {
      slice(k0, 0);
      slice(k0 + kKH, 1);
    }
  } else {
    for (int k0 = 0; k0 < K; k0 += kKH) slice(k0, 0);
  }
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][j] += t[j][r];
}

// ---- products with both operands copied straight into LDS -------------------------------
// Shared memory of the tile kernels. A ring of NSLOT product slices (the copy path): a
// slot holds A's 64 rows x 32 k-values (256 units of 16 bytes) and then B's columns x 32
// k-values (up to BUNITS units), as 16-byte runs copied from the half sources by buffer
// loads into LDS. Run q (k-values 8q..8q+7) of row (column) n sits at unit
// 4n + (q ^ ring_swz(n)). A 16-byte LDS read serves 16 lanes at a time, lanes
// {0-3, 12-15, 20-23, 24-27} together (and the sets derived from them: lane bit 5 and
// bits 2 ^ 3 ^ 4 fixed), over 64 banks of 4 bytes; with ring_swz(n) = 0, 2, 3, 1 for
// (n >> 2) & 3 = 0..3 the 16 rows and four runs such a set reads at one q fall into 16
// different 4-bank groups. The ring shares its space with the staging buffers of the
// register path (As, Bs: operands that need a conversion), and, after the products, with
// the rotation buffer and the GroupNorm backward's sums and dO tile.
template <int NSLOT, int BUNITS, int DTROWS = 1>
struct alignas(16) TileSharedD {
  union {
    struct {
      union {
        u32x4 ring[NSLOT][256 + BUNITS];
        struct {
          _Float16 As[kR][kLdH];
          _Float16 Bs[kMaxDv][kLdH];
        };
      };
      _Float16 P[kR][kLdPH];
    } m;
    float rot[kR][kMaxDk + 4];
    struct {
      float sw[16][kLdB];
      float sb[16][kLdB];
      uint16_t dtile[DTROWS][kMaxDv + 8];   // (bm_dout only: kR rows)
    } gn;
  };
};
template <int NS, int BU, int DT> __device__ __forceinline__ float* rot_buf(TileSharedD<NS, BU, DT>& sm) { return &sm.rot[0][0]; }
template <int NS, int BU, int DT> __device__ __forceinline__ float* gn_sw(TileSharedD<NS, BU, DT>& sm) { return &sm.gn.sw[0][0]; }
template <int NS, int BU, int DT> __device__ __forceinline__ float* gn_sb(TileSharedD<NS, BU, DT>& sm) { return &sm.gn.sb[0][0]; }

__device__ __forceinline__ int ring_swz(int n) { return (0x78 >> (2 * ((n >> 2) & 3))) & 3; }
__device__ __forceinline__ int ring_unit(int n, int q) { return 4 * n + (q ^ ring_swz(n)); }

// Barrier for LDS traffic only: this wave's LDS operations are complete; copies into LDS
// that are still in flight stay in flight (__syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | (((VM >> 4) & 3) << 14));
  __asm__ volatile("" ::: "memory");
}

// acc += A B as tmm16 does, for half sources only (no conversion): both operands of slice
// k (32 k-values) are copied into ring slot k % NSLOT while slices k - NSLOT + 1 .. k - 1
// are multiplied, one barrier per slice. A's row scaling amul * gamma^(ae0 + aesg i) is
// applied to the product's rows instead of A's (C = diag(f) A B). The caller has issued no
// store that is still in flight (the copies are waited for by count, in issue order).
template <int NCT, bool FROMP, int NSLOT, class SM>
__device__ __forceinline__ void tmm16d(float (&acc)[4][NCT], int K, SM& sm, const Src& A,
                                       int ar0, float amul, float alg, int ae0, int aesg,
                                       const Src& B, int br0, int bc0) {
  constexpr int NRUN = NCT / 4;                    // B copies per wave and slice
  constexpr int NOPS = NRUN + (FROMP ? 0 : 1);     // copies per wave and slice
  static_assert(NSLOT >= 2 && (NSLOT - 2) * NOPS <= 63, "ring depth");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const __amdgpu_buffer_rsrc_t rsa = src_rsrc(A), rsb = src_rsrc(B);
  const int nsl = (K + kKH - 1) / kKH;
  // A copy of this lane: unit 64 w + l of the slot's A part
  const int ap = 64 * w + l, arow = ap >> 2, aq = (ap & 3) ^ ring_swz(arow);
  auto issue = [&](int k, int slot) __attribute__((always_inline)) {
    const int k0 = k * kKH;
    if constexpr (!FROMP) {
      const int kq = k0 + 8 * aq;
      const uint32_t off = live_off(static_cast<uint32_t>(((ar0 + arow) * A.pitch + kq) * 2), kq < K);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsa, (__attribute__((address_space(3))) void*)(&sm.m.ring[slot][64 * w]), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NRUN; ++u) {
      const int p = (NRUN * w + u) * 64 + l, n = p >> 2, q = (p & 3) ^ ring_swz(n);
      const int kq = k0 + 8 * q;
      const uint32_t off = live_off(static_cast<uint32_t>(((br0 + n) * B.pitch + bc0 + kq) * 2), kq < K);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsb, (__attribute__((address_space(3))) void*)(&sm.m.ring[slot][256 + (NRUN * w + u) * 64]), 16,
          off, 0, 0, 0);
    }
  };
  f32x4 t[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();   // earlier reads of the ring (and of P's writes) are done
#pragma unroll
  for (int k = 0; k < NSLOT - 1; ++k)
    if (k < nsl) issue(k, k);
  int slot = 0;
  for (int k = 0; k < nsl; ++k) {
    // this wave's copies of slice k are complete (those of the next NSLOT-2 slices, when
    // issued, may stay in flight)
    if (k + NSLOT - 2 < nsl) wait_vm<(NSLOT - 2) * NOPS>();
    else wait_vm<0>();
    lds_barrier();   // every wave's copies of slice k landed; slice k-1's reads are done
    if (k + NSLOT - 1 < nsl) issue(k + NSLOT - 1, slot == 0 ? NSLOT - 1 : slot - 1);
    const u32x4* rs = sm.m.ring[slot];
    f16x8 av;
    if constexpr (FROMP) av = *reinterpret_cast<const f16x8*>(&sm.m.P[16 * w + l16][k * kKH + 8 * g]);
    else av = __builtin_bit_cast(f16x8, rs[ring_unit(16 * w + l16, g)]);
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const f16x8 bv = __builtin_bit_cast(f16x8, rs[256 + ring_unit(16 * j + l16, g)]);
      t[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, t[j], 0, 0, 0);
    }
    slot = slot + 1 == NSLOT ? 0 : slot + 1;
  }
  float f[4] = {1.f, 1.f, 1.f, 1.f};
  if (!FROMP && (aesg != 0 || amul != 1.f)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) f[r] = amul * exp2f(alg * float(ae0 + aesg * (16 * w + 4 * g + r)));
  }
#pragma unroll
  for (int j = 0; j < NCT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r][j] += f[r] * t[j][r];
}

// Workspace (half), per head: row-major rotated q and k, their transposes, v transposed,
// dO row-major and transposed, and the chunk states S and G in both orientations.
struct MLayout {
  int Np, nch;
  size_t QR, KR, QT, KT, VT, DR, DT, S, ST, G, GT, total;   // byte offsets
};
size_t a256(size_t x) { return (x + 255) & ~size_t(255); }
MLayout m_layout(const CallArgs& a) {
  MLayout L;
  L.Np = (a.N + 63) / 64 * 64;
  L.nch = (a.N + kBC - 1) / kBC;
  const size_t BH = size_t(a.B) * a.H;
  const size_t rowk = a256(BH * a.N * a.dk * 2), rowv = a256(BH * a.N * a.dv * 2);
  const size_t tk = a256(BH * a.dk * L.Np * 2), tv = a256(BH * a.dv * L.Np * 2);
  const size_t st = a256(BH * L.nch * a.dk * a.dv * 2);
  size_t o = 0;
  L.QR = o; o += rowk;
  L.KR = o; o += rowk;
  L.QT = o; o += tk;
  L.KT = o; o += tk;
  L.VT = o; o += tv;
  L.DR = o; o += rowv;
  L.DT = o; o += tv;
  L.S = o; o += st;
  L.ST = o; o += st;
  L.G = o; o += st;
  L.GT = o; o += st;
  L.total = o;
  return L;
}

// ---- prep: rotated q, k (row-major and transposed) and v transposed, per 64 tokens ------
// Grid (Np/64, b*H + h); the transposes go through LDS, [column][token].
// Transposed tile of a 64-token block: row c (a coordinate) holds the 64 tokens as eight
// 16-byte pieces, piece j stored at slot j ^ ((c >> 3) & 7). The swizzle spreads the
// 2-byte writes of a wave (coordinates 8 rows apart in consecutive lanes) over the banks
// and leaves the 16-byte read-out conflict free.
constexpr int kTp = 64;
__device__ __forceinline__ int tswz(int c, int tt) { return tt ^ (((c >> 3) & 7) << 3); }
__device__ __forceinline__ void store_t_rows(uint16_t (*tb)[kTp], int rows, uint16_t* T, int Np, int t0) {
  for (int e = threadIdx.x; e < rows * 8; e += 256) {
    const int c = e >> 3, pc = e & 7;
    *reinterpret_cast<u32x4*>(T + int64_t(c) * Np + t0 + 8 * pc) =
        *reinterpret_cast<const u32x4*>(&tb[c][8 * (pc ^ ((c >> 3) & 7))]);
  }
}
__global__ void __launch_bounds__(256) bm_prep(CallArgs a, const uint16_t* q, const uint16_t* k,
                                               const uint16_t* v, uint16_t* QR, uint16_t* KR,
                                               uint16_t* QT, uint16_t* KT, uint16_t* VT, int Np) {
  __shared__ __attribute__((aligned(16))) uint16_t tb[kMaxDv][kTp];
  const int dk = a.dk, dv = a.dv, N = a.N;
  const int t0 = blockIdx.x * 64, bh = blockIdx.y;
  const int64_t p0 = seq_pos0(a, bh / a.H);
  // The block's rows of q, k and v are contiguous in memory: element run e (16 bytes) of
  // a tile is token e / runs-per-row, coordinates 8 (e % runs-per-row) .. +8, so a wave
  // reads and writes one contiguous 1 KB span. All of a thread's loads are issued before
  // the first is used (8 runs each of q and k, 16 of v at the 6.7B shape).
  constexpr int kMaxRunsK = 64 * (kMaxDk / 8) / 256;
  constexpr int kMaxRunsV = 64 * (kMaxDv / 8) / 256;
  {
    // q and k together: one angle per (token, pair); rotated q goes to tile rows
    // 0..dk-1, rotated k to rows dk..2dk-1 (2 dk <= kMaxDv)
    const int rpr = dk >> 3, nrun = 64 * rpr;
    const uint16_t* xq = q + (int64_t(bh) * N + t0) * dk;
    const uint16_t* xk = k + (int64_t(bh) * N + t0) * dk;
    const int nval = (min(N - t0, 64)) * rpr;   // runs inside the sequence
    u32x4 rq[kMaxRunsK], rk[kMaxRunsK];
#pragma unroll
    for (int i = 0; i < kMaxRunsK; ++i) {
      const int e = threadIdx.x + 256 * i;
      const bool in = e < nval;
      rq[i] = in ? *reinterpret_cast<const u32x4*>(xq + 8 * e) : u32x4{0u, 0u, 0u, 0u};
      rk[i] = in ? *reinterpret_cast<const u32x4*>(xk + 8 * e) : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* Rq = QR + (int64_t(bh) * N + t0) * dk;
    uint16_t* Rk = KR + (int64_t(bh) * N + t0) * dk;
#pragma unroll
    for (int i = 0; i < kMaxRunsK; ++i) {
      const int e = threadIdx.x + 256 * i;
      if (e >= nrun) break;
      const int tt = e / rpr, cq = e - tt * rpr;
      uint32_t oq[4], ok[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float c, sn;
        angle_cs(p0 + t0 + tt, a.ap.theta[4 * cq + m], &c, &sn);
        const float q0 = __uint_as_float(rq[i][m] << 16), q1 = __uint_as_float(rq[i][m] & 0xffff0000u);
        const float k0 = __uint_as_float(rk[i][m] << 16), k1 = __uint_as_float(rk[i][m] & 0xffff0000u);
        oq[m] = pack_h2(q0 * c - q1 * sn, q0 * sn + q1 * c);
        ok[m] = pack_h2(k0 * c - k1 * sn, k0 * sn + k1 * c);
        const int r0 = 8 * cq + 2 * m, r1 = dk + r0;
        tb[r0][tswz(r0, tt)] = uint16_t(oq[m] & 0xffffu);
        tb[r0 + 1][tswz(r0 + 1, tt)] = uint16_t(oq[m] >> 16);
        // (the k tile is read out from row dk on, so it swizzles by its own row index)
        tb[r1][tswz(r0, tt)] = uint16_t(ok[m] & 0xffffu);
        tb[r1 + 1][tswz(r0 + 1, tt)] = uint16_t(ok[m] >> 16);
      }
      if (e < nval) {
        *reinterpret_cast<u32x4*>(Rq + 8 * e) = u32x4{oq[0], oq[1], oq[2], oq[3]};
        *reinterpret_cast<u32x4*>(Rk + 8 * e) = u32x4{ok[0], ok[1], ok[2], ok[3]};
      }
    }
    __syncthreads();
    store_t_rows(tb, dk, QT + int64_t(bh) * dk * Np, Np, t0);
    store_t_rows(tb + dk, dk, KT + int64_t(bh) * dk * Np, Np, t0);
    __syncthreads();
  }
  const int rpv = dv >> 3, nrun = 64 * rpv;
  const int nval = (min(N - t0, 64)) * rpv;
  const uint16_t* xv = v + (int64_t(bh) * N + t0) * dv;
  u32x4 raw[kMaxRunsV];
#pragma unroll
  for (int i = 0; i < kMaxRunsV; ++i) {
    const int e = threadIdx.x + 256 * i;
    raw[i] = e < nval ? *reinterpret_cast<const u32x4*>(xv + 8 * e) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kMaxRunsV; ++i) {
    const int e = threadIdx.x + 256 * i;
    if (e >= nrun) break;
    const int tt = e / rpv, cq = e - tt * rpv;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t hh = bf2_to_h2(raw[i][m]);
      const int r0 = 8 * cq + 2 * m;
      tb[r0][tswz(r0, tt)] = uint16_t(hh & 0xffffu);
      tb[r0 + 1][tswz(r0 + 1, tt)] = uint16_t(hh >> 16);
    }
  }
  __syncthreads();
  store_t_rows(tb, dv, VT + int64_t(bh) * dv * Np, Np, t0);
}

// ---- state scans on matrix cores ---------------------------------------------------------
// REV = 0: S (chunk states) from X = Kh^T weighted by zeta, Y = V^T, from state_in.
// REV = 1: G (gradients reaching the chunk ends) from X = Qh^T weighted by alpha xi, Y = dO^T,
//          chunks in reverse, from dstate_out; the final value goes to dstate_in.
// Workgroup: a 64 (d_k) x 128 (d_v) tile of the state in MFMA accumulators, wave w rows
// 16w.. of the tile. Per 64-token slice: X^T rows (tokens weighted on staging) times Y^T
// rows, staged in one of two LDS buffers (one barrier per slice). Each chunk's boundary
// value is stored in half as [d_k][d_v] and [d_v][d_k].
constexpr int kSK = 64;            // tokens per slice
constexpr int kLdS = kSK + 8;      // LDS pitch (half) of a staged row
constexpr int kLdT = 128 + 8;   // LDS pitch (half) of the staged boundary value
struct alignas(16) ScanShared {
  _Float16 As[2][64][kLdS];
  _Float16 Bs[2][128][kLdS];
  float wt[2][kBC];               // token weights of a chunk (by chunk parity)
  uint16_t bv[64][kLdT];          // the chunk's boundary value (half), for 16-byte row stores
};

template <int REV>
__global__ void __launch_bounds__(256) bm_scan(CallArgs a, const uint16_t* XT, const uint16_t* YT,
                                               const float* init, uint16_t* Sr, uint16_t* St,
                                               float* final_out, int Np) {
  __shared__ ScanShared sm;
  const int dk = a.dk, dv = a.dv, N = a.N;
  // 1-D grid: the state tiles of a head all run on one XCD (id mod 8), where the tiles that
  // share rows of X^T or Y^T find them in L2
  const int nte = (dv + 127) / 128, ntiles = ((dk + 63) / 64) * nte;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int bh = 8 * (jx / ntiles) + xcd, tile = jx % ntiles;
  if (bh >= a.B * a.H) return;
  const int d0 = 64 * (tile / nte), e0 = 128 * (tile % nte);
  const int h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int nch = (N + kBC - 1) / kBC;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const Src X{XT + int64_t(bh) * dk * Np, Np, dk, false};
  const Src Y{YT + int64_t(bh) * dv * Np, Np, dv, false};
  const int64_t nS = int64_t(dk) * dv;
  f32x4 t[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = d0 + 16 * w + 4 * g + r, e = e0 + 16 * j + l16;
      t[j][r] = (init && d < dk && e < dv) ? init[bh * nS + int64_t(d) * dv + e] : 0.f;
    }
  // Slices of 64 tokens are numbered across chunks (slice u: chunk u >> 2 in scan order,
  // tokens 64 (u & 3) .. of it) and loaded four ahead through a ring of register sets,
  // branch-free: runs past a chunk's end or past the last chunk read as zeros. Thread tid
  // stages runs tid + 256 v: X^T row (run >> 3) (two runs), Y^T row (run >> 3) (four
  // runs), tokens 8 (run & 7) .. of the slice.
  constexpr int kSets = 4;
  const __amdgpu_buffer_rsrc_t rx = src_rsrc(X), ry = src_rsrc(Y);
  u32x4 ra[kSets][2], rb[kSets][4];
  auto fetch = [&](int u, int set) __attribute__((always_inline)) {
    const int ci = u >> 2;
    const int cu = REV ? nch - 1 - ci : ci;
    const int c0u = cu * kBC, Lu = ci < nch ? min(N, c0u + kBC) - c0u : 0;
    const int k = kSK * (u & 3);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int run = tid + 256 * v, kq = k + 8 * (run & 7);
      ra[set][v] = raw8(rx, X.pitch, d0 + (run >> 3), int64_t(c0u) + kq, kq < Lu);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int run = tid + 256 * v, kq = k + 8 * (run & 7);
      rb[set][v] = raw8(ry, Y.pitch, e0 + (run >> 3), int64_t(c0u) + kq, kq < Lu);
    }
  };
  // chunk boundary values through buffer resources over the head's states: lanes past
  // d_k or d_v store to a dropped offset (no branch)
  const __amdgpu_buffer_rsrc_t rS = src_rsrc(Src{Sr + int64_t(bh) * nch * nS, 1, int(nch * nS), false});
  const __amdgpu_buffer_rsrc_t rST = src_rsrc(Src{St + int64_t(bh) * nch * nS, 1, int(nch * nS), false});
  for (int u = 0; u < kSets; ++u) fetch(u, u);
  // token weights of chunk `step` (scan order): zeta_s = gamma^(L-1-s) for the states,
  // alpha xi_s = alpha gamma^(s+1) for the gradients, zero past the chunk's end
  auto weights = [&](int step, float* wt) {
    const int cw = REV ? nch - 1 - step : step;
    const int Lw = (step < nch) ? min(N, cw * kBC + kBC) - cw * kBC : 0;
    for (int jj = tid; jj < kBC; jj += 256)
      wt[jj] = jj < Lw ? (REV ? a.alpha * gpow(lg, float(jj + 1)) : gpow(lg, float(Lw - 1 - jj))) : 0.f;
  };
  weights(0, sm.wt[0]);
  __syncthreads();
  for (int step = 0; step < nch; ++step) {
    const int c = REV ? nch - 1 - step : step;
    const int c0 = c * kBC, L = min(N, c0 + kBC) - c0;
    // the chunk's boundary value, in both orientations
    const uint32_t cbase = static_cast<uint32_t>(int64_t(c) * nS);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + 16 * j + l16, d = d0 + 16 * w + 4 * g;
      const bool ok = e < dv && d < dk;
      const uint32_t ot = live_off((cbase + uint32_t(e) * dk + d) * 2, ok);
      __builtin_amdgcn_raw_buffer_store_b64(
          __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int,
                             u32x2{pack_h2(t[j][0], t[j][1]), pack_h2(t[j][2], t[j][3])}),
          rST, ot, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.bv[16 * w + 4 * g + r][16 * j + l16] = h_bits(t[j][r]);
    }
    // (the weights of the next chunk go in while the boundary value is staged)
    weights(step + 1, sm.wt[(step + 1) & 1]);
    __syncthreads();   // the staged boundary value is complete
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int run = tid + 256 * v, row = run >> 4, q = run & 15;
      const bool ok = d0 + row < dk && e0 + 8 * q < dv;
      const uint32_t orow = live_off((cbase + uint32_t(d0 + row) * dv + e0 + 8 * q) * 2, ok);
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int,
                             *reinterpret_cast<const u32x4*>(&sm.bv[row][8 * q])),
          rS, orow, 0, 0);
    }
    const float gL = gpow(lg, float(L));
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] *= gL;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int buf = i & 1, k0 = kSK * i;
      // stage slice i of the chunk: X^T runs weighted per token
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int run = tid + 256 * v, kq = k0 + 8 * (run & 7);
        float f[8];
        {
          const float4 f0 = *reinterpret_cast<const float4*>(&sm.wt[step & 1][kq]);
          const float4 f1 = *reinterpret_cast<const float4*>(&sm.wt[step & 1][kq + 4]);
          f[0] = f0.x; f[1] = f0.y; f[2] = f0.z; f[3] = f0.w;
          f[4] = f1.x; f[5] = f1.y; f[6] = f1.z; f[7] = f1.w;
        }
        *reinterpret_cast<u32x4*>(&sm.As[buf][run >> 3][8 * (run & 7)]) = scale8(ra[i][v], f);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int run = tid + 256 * v;
        *reinterpret_cast<u32x4*>(&sm.Bs[buf][run >> 3][8 * (run & 7)]) = rb[i][v];
      }
      // the buffer staged here was last read two slices ago, before every wave's
      // previous barrier
      __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      fetch(4 * step + i + kSets, i);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f16x8 av = *reinterpret_cast<const f16x8*>(&sm.As[buf][16 * w + l16][32 * e + 8 * g]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f16x8 bv = *reinterpret_cast<const f16x8*>(&sm.Bs[buf][16 * j + l16][32 * e + 8 * g]);
          t[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, t[j], 0, 0, 0);
        }
      }
    }
  }
  if (final_out) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = d0 + 16 * w + 4 * g + r, e = e0 + 16 * j + l16;
        if (d < dk && e < dv) final_out[bh * nS + int64_t(d) * dv + e] = t[j][r];
      }
  }
}

// ---- tile kernels (1-D grid over (head, chunk, 64-row tile)) ----------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (id mod 8). The four row tiles of
// a chunk read the same chunk operands (its keys, values, state), so they are numbered to
// run one after the other on one XCD, where the later ones find those operands in L2:
// id = 8 (4 (P / 8) + tile) + P % 8 for chunk P = bh * nch + c.
struct TileAt {
  TileRows T;
  int bh;
  bool valid;
};
__device__ __forceinline__ TileAt tile_at(int N, int BH, int nch) {
  const int id = blockIdx.x, j = id >> 3;
  const int P = 8 * (j >> 2) + (id & 7), tile = j & 3;
  TileAt r;
  r.valid = P < BH * nch;
  r.bh = r.valid ? P / nch : 0;
  const int c = r.valid ? P % nch : 0;
  r.T.c = c;
  r.T.c0 = c * kBC;
  r.T.c1 = min(N, r.T.c0 + kBC);
  r.T.r0 = r.T.c0 + kR * tile;
  r.T.r1 = min(r.T.c1, r.T.r0 + kR);
  return r;
}
struct Heads {
  const uint16_t *QR, *KR, *QT, *KT, *VT, *DR, *DT, *S, *ST, *G, *GT;
  int Np, nch;
};

// ---- GroupNorm / gate backward of a bm_dout tile ----------------------------------------
// Each wave takes the 16 rows it holds in its accumulators (rows 16w + 4g + r, columns
// l16 + 16 j), staged through LDS in float32, and works through them one row at a time with
// 8 consecutive columns per lane, so that dout, gate and dgate move in 16-byte pieces.
// Per row: dO = rstd (dxh - mean(dxh) - xh mean(dxh xh)), dxh = dy w, dy = dout (* swish(g)),
// written (half) over the row's own staging; the gate's gradient is stored; per-column
// sums of dy xh and dy gather in LDS and are added to dgn_w, dgn_b once per tile.
constexpr int kOLd = kMaxDv + 4;   // staging row pitch (floats); a dO row (half) fits in its first half
__device__ __forceinline__ float lane_sum64(float x) {   // over the wave; every lane receives it
  x = row16_sum(x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
}
template <int OUTD, bool AFF>
__device__ __forceinline__ void gn_backward_rows(float* ost, const float (&o)[4][32],
                                                 const CallArgs& a, int h, int bh, int r0, int r1,
                                                 const void* gate, const void* dout, void* dgate,
                                                 float* dgn_w, float* dgn_b) {
  const int dv = a.dv, N = a.N;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const bool gt = a.flags & RN_EPI_GATE;
  const bool sums = AFF && (dgn_w || dgn_b);
  constexpr int esz = OUTD == RN_F32 ? 4 : 2;
  const int64_t hoff = int64_t(bh) * N * dv;
  const __amdgpu_buffer_rsrc_t rdo = head_rsrc(static_cast<const char*>(dout) + hoff * esz, int64_t(N) * dv * esz);
  const __amdgpu_buffer_rsrc_t rga =
      head_rsrc(gt ? static_cast<const char*>(gate) + hoff * 2 : nullptr, gt ? int64_t(N) * dv * 2 : 0);
  const __amdgpu_buffer_rsrc_t rdg =
      head_rsrc(gt && dgate ? static_cast<char*>(dgate) + hoff * 2 : nullptr, gt && dgate ? int64_t(N) * dv * 2 : 0);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 32; ++j) ost[(16 * w + 4 * g + r) * kOLd + l16 + 16 * j] = o[r][j];
  __syncthreads();
  const int c0 = 8 * l;
  const bool cl = c0 < dv;   // this lane has columns
  float wv[8], bv[8], swa[8], sba[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    wv[c] = (AFF && a.gn_w && cl) ? a.gn_w[h * dv + c0 + c] : 1.f;
    bv[c] = (AFF && a.gn_b && cl) ? a.gn_b[h * dv + c0 + c] : 0.f;
    swa[c] = sba[c] = 0.f;
  }
  const float inv_dv = 1.0f / float(dv);
  // dout / gate of row rr (16-byte pieces). Byte offsets within the head; rows past the
  // tile and lanes past d_v use an offset past the buffers' ranges (loads read zeros,
  // stores are dropped).
  auto boff = [&](int rr, int bytes) -> uint32_t {
    const int t = r0 + 16 * w + rr;
    return live_off(static_cast<uint32_t>((t * dv + c0) * bytes), t < r1 && cl);
  };
  // all rows of a batch are loaded before the first is used (16 rows for bf16 dout, 8 for
  // float32), so their latencies overlap
  constexpr int RB = OUTD == RN_F32 ? 8 : 16;
  constexpr int DW = OUTD == RN_F32 ? 2 : 1;   // 16-byte pieces of dout per row and lane
#pragma unroll
  for (int rb = 0; rb < 16; rb += RB) {
    u32x4 dl[RB][DW], gl[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t od = boff(rb + i, esz), og = boff(rb + i, 2);
#pragma unroll
      for (int p = 0; p < DW; ++p)
        dl[i][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, od + 16 * p, 0, 0));
      gl[i] = gt ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rga, og, 0, 0))
                 : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rr = rb + i;
      float d0[8], gv[8];
      if constexpr (OUTD == RN_F32) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          d0[c] = __uint_as_float(dl[i][0][c]);
          d0[4 + c] = __uint_as_float(dl[i][DW - 1][c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          d0[2 * c] = __uint_as_float(dl[i][0][c] << 16);
          d0[2 * c + 1] = __uint_as_float(dl[i][0][c] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gv[2 * c] = __uint_as_float(gl[i][c] << 16);
        gv[2 * c + 1] = __uint_as_float(gl[i][c] & 0xffff0000u);
      }
      const uint32_t og = boff(rr, 2);
      const int row = 16 * w + rr;
      float x[8];
      {
        const float4 x0 = *reinterpret_cast<const float4*>(&ost[row * kOLd + c0]);
        const float4 x1 = *reinterpret_cast<const float4*>(&ost[row * kOLd + c0 + 4]);
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
      }
      float s1 = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) s1 += cl ? x[c] : 0.f;
      const float mean = lane_sum64(s1) * inv_dv;
      float s2 = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float dd = x[c] - mean;
        s2 += cl ? dd * dd : 0.f;
      }
      const float rstd = __builtin_amdgcn_rsqf(lane_sum64(s2) * inv_dv + a.eps);
      float xh[8], dxh[8], dg[8];
      float m1 = 0.f, m2 = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        xh[c] = (x[c] - mean) * rstd;
        float dy = d0[c];
        if (gt) {
          const float gg = gv[c];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gg));
          dy = d0[c] * gg * sg;
          dg[c] = d0[c] * (xh[c] * wv[c] + bv[c]) * sg * (1.0f + gg * (1.0f - sg));
        }
        dxh[c] = dy * wv[c];
        m1 += dxh[c];
        m2 += dxh[c] * xh[c];
        if constexpr (AFF) {
          swa[c] += dy * xh[c];
          sba[c] += dy;
        }
      }
      if (gt) {
        const u32x4 pk{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]), pack_bf16x2(dg[4], dg[5]),
                       pack_bf16x2(dg[6], dg[7])};
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, pk), rdg, og, 0, 0);
      }
      m1 = lane_sum64(m1) * inv_dv;
      m2 = lane_sum64(m2) * inv_dv;
      float od[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) od[c] = rstd * (dxh[c] - m1 - xh[c] * m2);
      // the row's values were read above (this wave's LDS operations run in order)
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(&ost[row * kOLd]) + c0) =
          u32x4{pack_h2(od[0], od[1]), pack_h2(od[2], od[3]), pack_h2(od[4], od[5]), pack_h2(od[6], od[7])};
    }
  }
  // per-wave column sums go to the second halves of the wave's staging rows (the dO rows
  // take the first halves): row 16w + 2c + s holds, from float kOLd / 2 on, sum s
  // (0: dy xh, 1: dy) of column 8l + c at index l
  auto part = [&](int ww, int c, int sidx) { return ost + (16 * ww + 2 * c + sidx) * kOLd + kOLd / 2; };
  if (sums) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      part(w, c, 0)[l] = swa[c];
      part(w, c, 1)[l] = sba[c];
    }
  }
  __syncthreads();
  if (sums)
    for (int col = tid; col < dv; col += 256) {
      const int lc = col >> 3, c = col & 7;
      float xw = 0.f, xb = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        xw += part(ww, c, 0)[lc];
        xb += part(ww, c, 1)[lc];
      }
      if (dgn_w) atomicAdd(&dgn_w[h * dv + col], xw);
      if (dgn_b) atomicAdd(&dgn_b[h * dv + col], xb);
    }
}

// o recomputed: alpha (Qh Kh^T (.) D) V + alpha xi Qh S_c, then the GroupNorm / gate backward.
template <int OUTD, bool AFF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bm_dout(CallArgs a, Heads Hd, const void* gate, const void* dout, uint16_t* DR, uint16_t* DT,
        void* dgate, float* dgn_w, float* dgn_b) {
  __shared__ TileSharedD<3, kMaxDv * 4> sm;
  static_assert(sizeof(sm) >= kR * kOLd * sizeof(float), "staging fits");
  // dO of the tile in half (rows past the tile's end hold zeros), copied out at the end in
  // 16-byte runs, row-major to DR and transposed to DT; row r at dt + r * kDtLd
  float* ost = reinterpret_cast<float*>(&sm);
  uint16_t* dt = reinterpret_cast<uint16_t*>(ost);
  constexpr int kDtLd = 2 * kOLd;
  const int dk = a.dk, dv = a.dv, N = a.N, Np = Hd.Np;
  const TileAt at = tile_at(N, a.B * a.H, Hd.nch);
  const TileRows T = at.T;
  if (!at.valid || T.r0 >= T.r1) return;
  const int bh = at.bh, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const Src Q{Hd.QR + int64_t(bh) * N * dk, dk, N, false};
  const Src K{Hd.KR + int64_t(bh) * N * dk, dk, N, false};
  const Src VT{Hd.VT + int64_t(bh) * dv * Np, Np, dv, false};
  const Src ST{Hd.ST + (int64_t(bh) * Hd.nch + T.c) * dk * dv, dk, dv, false};
  float m[4][16];
  zero_acc(m);
  tmm16d<16, false, 3>(m, dk, sm, Q, T.r0, 1.f, 0.f, 0, 0, K, T.c0, 0);
  store_scores<true>(sm, m, T.r0, T.r1, T.c0, T.r1, lg, a.alpha);
  float o[4][32];
  zero_acc(o);
  tmm16d<32, true, 3>(o, T.r1 - T.c0, sm, Q, 0, 1.f, 0.f, 0, 0, VT, 0, T.c0);
  tmm16d<32, false, 3>(o, dk, sm, Q, T.r0, a.alpha, lg, T.r0 - T.c0 + 1, 1, ST, 0, 0);
  __syncthreads();   // the products' reads of the ring are done (the staging shares its space)
  if (a.flags & RN_EPI_GN) {
    gn_backward_rows<OUTD, AFF>(ost, o, a, h, bh, T.r0, T.r1, gate, dout, dgate,
                                dgn_w, dgn_b);
  } else {
    gn_backward_tile<RN_BF16, OUTD, AFF>(sm, o, a, h, bh, T.r0, T.r1, gate, dout, dgate, dgn_w, dgn_b,
        [&](int64_t, int, bool ok, float x, int rloc, int col) __attribute__((always_inline)) {
          dt[rloc * kDtLd + col] = ok ? h_bits(x) : uint16_t(0);
        });
  }
  __syncthreads();
  // row-major: the tile's rows below its end
  const int rows = T.r1 - T.r0, runs = dv / 8;
  uint16_t* DRh = DR + (int64_t(bh) * N + T.r0) * dv;
  for (int e = threadIdx.x; e < rows * runs; e += 256) {
    const int rr = e / runs, c8 = e - rr * runs;
    *reinterpret_cast<u32x4*>(DRh + int64_t(rr) * dv + 8 * c8) =
        *reinterpret_cast<const u32x4*>(&dt[rr * kDtLd + 8 * c8]);
  }
  // transposed: 8 tokens of one column per run, all 64 columns of the tile (the rows past
  // the sequence's end are zeros, as the padded layout wants)
  uint16_t* DTh = DT + int64_t(bh) * dv * Np + T.r0;
  for (int e = threadIdx.x; e < dv * 8; e += 256) {
    const int col = e >> 3, tg = e & 7;
    uint32_t wds[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wds[k] = uint32_t(dt[(8 * tg + 2 * k) * kDtLd + col]) | (uint32_t(dt[(8 * tg + 2 * k + 1) * kDtLd + col]) << 16);
    *reinterpret_cast<u32x4*>(DTh + int64_t(col) * Np + 8 * tg) = u32x4{wds[0], wds[1], wds[2], wds[3]};
  }
}

// dQh = [alpha (dO V^T) (.) D] Kh + alpha xi dO S_c^T, rotated back.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bm_dq(CallArgs a, Heads Hd, const uint16_t* v, void* dq) {
  __shared__ TileSharedD<2, kMaxDv * 2> sm;
  const int dk = a.dk, dv = a.dv, N = a.N, Np = Hd.Np;
  const TileAt at = tile_at(N, a.B * a.H, Hd.nch);
  const TileRows T = at.T;
  if (!at.valid || T.r0 >= T.r1) return;
  const int bh = at.bh, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const Src D{Hd.DR + int64_t(bh) * N * dv, dv, N, false};
  const Src V{v + int64_t(bh) * N * dv, dv, N, true};
  const Src KT{Hd.KT + int64_t(bh) * dk * Np, Np, dk, false};
  const Src S{Hd.S + (int64_t(bh) * Hd.nch + T.c) * dk * dv, dv, dk, false};
  float m[4][16];
  zero_acc(m);
  tmm16<16, false, 2>(m, dv, sm, D, T.r0, 1.f, 0.f, 0, 0, V, T.c0, 0);
  store_scores<true>(sm, m, T.r0, T.r1, T.c0, T.r1, lg, a.alpha);
  float gq[4][16];
  zero_acc(gq);
  tmm16d<16, true, 2>(gq, T.r1 - T.c0, sm, D, 0, 1.f, 0.f, 0, 0, KT, 0, T.c0);
  tmm16d<16, false, 2>(gq, dv, sm, D, T.r0, a.alpha, lg, T.r0 - T.c0 + 1, 1, S, 0, 0);
  store_rotated<RN_BF16>(sm, gq, a, seq_pos0(a, bh / a.H), bh, T.r0, T.r1, dq);
}

// Tile rows are keys s; later rows t in [s, c1): dKh = [alpha (V dO^T) (.) D'] Qh + zeta V G^T.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bm_dk(CallArgs a, Heads Hd, const uint16_t* v, void* dk_) {
  __shared__ TileSharedD<2, kMaxDv * 2> sm;
  const int dk = a.dk, dv = a.dv, N = a.N, Np = Hd.Np;
  const TileAt at = tile_at(N, a.B * a.H, Hd.nch);
  const TileRows T = at.T;
  if (!at.valid || T.r0 >= T.r1) return;
  const int bh = at.bh, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const Src V{v + int64_t(bh) * N * dv, dv, N, true};
  const Src D{Hd.DR + int64_t(bh) * N * dv, dv, N, false};
  const Src QT{Hd.QT + int64_t(bh) * dk * Np, Np, dk, false};
  const Src G{Hd.G + (int64_t(bh) * Hd.nch + T.c) * dk * dv, dv, dk, false};
  float m[4][16];
  zero_acc(m);
  tmm16<16, false, 2>(m, dv, sm, V, T.r0, 1.f, 0.f, 0, 0, D, T.r0, 0);
  store_scores<false>(sm, m, T.r0, T.r1, T.r0, T.c1, lg, a.alpha);
  float gk[4][16];
  zero_acc(gk);
  tmm16d<16, true, 2>(gk, T.c1 - T.r0, sm, V, 0, 1.f, 0.f, 0, 0, QT, 0, T.r0);
  tmm16<16, false, 2>(gk, dv, sm, V, T.r0, 1.f, lg, T.c1 - 1 - T.r0, -1, G, 0, 0);
  store_rotated<RN_BF16>(sm, gk, a, seq_pos0(a, bh / a.H), bh, T.r0, T.r1, dk_);
}

// dV = [alpha (Kh Qh^T) (.) D'] dO + zeta Kh G.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bm_dv(CallArgs a, Heads Hd, void* dv_) {
  __shared__ TileSharedD<3, kMaxDv * 4> sm;
  const int dk = a.dk, dv = a.dv, N = a.N, Np = Hd.Np;
  const TileAt at = tile_at(N, a.B * a.H, Hd.nch);
  const TileRows T = at.T;
  if (!at.valid || T.r0 >= T.r1) return;
  const int bh = at.bh, h = bh % a.H;
  const float lg = a.hp.log2g[h];
  const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
  const Src K{Hd.KR + int64_t(bh) * N * dk, dk, N, false};
  const Src Q{Hd.QR + int64_t(bh) * N * dk, dk, N, false};
  const Src DT{Hd.DT + int64_t(bh) * dv * Np, Np, dv, false};
  const Src GT{Hd.GT + (int64_t(bh) * Hd.nch + T.c) * dk * dv, dk, dv, false};
  float m[4][16];
  zero_acc(m);
  tmm16d<16, false, 3>(m, dk, sm, K, T.r0, 1.f, 0.f, 0, 0, Q, T.r0, 0);
  store_scores<false>(sm, m, T.r0, T.r1, T.r0, T.c1, lg, a.alpha);
  float o[4][32];
  zero_acc(o);
  tmm16d<32, true, 3>(o, T.c1 - T.r0, sm, K, 0, 1.f, 0.f, 0, 0, DT, 0, T.r0);
  tmm16d<32, false, 3>(o, dk, sm, K, T.r0, 1.f, lg, T.c1 - 1 - T.r0, -1, GT, 0, 0);
  // the tile (bf16) through LDS, then out in 16-byte runs of the rows below its end
  constexpr int kStLd = kMaxDv + 8;
  static_assert(sizeof(sm) >= kR * kStLd * sizeof(uint16_t), "tile staging fits");
  uint16_t* stg = reinterpret_cast<uint16_t*>(&sm);
  __syncthreads();   // the products' reads of shared memory are done
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < 32; ++j) stg[(4 * ty + r) * kStLd + tx + 16 * j] = f32_to_bf16(o[r][j]);
  __syncthreads();
  const int rows = T.r1 - T.r0, runs = dv / 8;
  uint16_t* dst = static_cast<uint16_t*>(dv_) + (int64_t(bh) * N + T.r0) * dv;
  for (int e = threadIdx.x; e < rows * runs; e += 256) {
    const int rr = e / runs, c8 = e - rr * runs;
    *reinterpret_cast<u32x4*>(dst + int64_t(rr) * dv + 8 * c8) = *reinterpret_cast<const u32x4*>(&stg[rr * kStLd + 8 * c8]);
  }
}

__global__ void fill_zero_m(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

template <int OUTD>
hipError_t launch_t(const CallArgs& a, const BwArgs& x, void* ws, hipStream_t st) {
  const MLayout L = m_layout(a);
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return reinterpret_cast<uint16_t*>(w + off); };
  const int BH = a.B * a.H;
  Heads Hd{at(L.QR), at(L.KR), at(L.QT), at(L.KT), at(L.VT), at(L.DR), at(L.DT),
           at(L.S), at(L.ST), at(L.G), at(L.GT), L.Np, L.nch};
  const dim3 gblk(L.Np / 64, BH);
  const dim3 gscan(static_cast<unsigned>(((a.dk + 63) / 64) * ((a.dv + 127) / 128) * 8 * ((BH + 7) / 8)));
  const dim3 gtiles(static_cast<unsigned>((BH * L.nch + 7) / 8) * 8 * (kBC / kR));
  hipLaunchKernelGGL(bm_prep, gblk, dim3(256), 0, st, a, static_cast<const uint16_t*>(x.q),
                     static_cast<const uint16_t*>(x.k), static_cast<const uint16_t*>(x.v), at(L.QR),
                     at(L.KR), at(L.QT), at(L.KT), at(L.VT), L.Np);
  hipLaunchKernelGGL(bm_scan<0>, gscan, dim3(256), 0, st, a, static_cast<const uint16_t*>(at(L.KT)),
                     static_cast<const uint16_t*>(at(L.VT)), x.state_in, at(L.S), at(L.ST),
                     static_cast<float*>(nullptr), L.Np);
  if (a.flags & RN_EPI_GN) {
    if (x.dgn_w) hipLaunchKernelGGL(fill_zero_m, dim3(8), dim3(256), 0, st, x.dgn_w, int64_t(a.H) * a.dv);
    if (x.dgn_b) hipLaunchKernelGGL(fill_zero_m, dim3(8), dim3(256), 0, st, x.dgn_b, int64_t(a.H) * a.dv);
  }
  if (a.gn_w || a.gn_b || x.dgn_w || x.dgn_b)
    hipLaunchKernelGGL((bm_dout<OUTD, true>), gtiles, dim3(256), 0, st, a, Hd, x.gate, x.dout, at(L.DR),
                       at(L.DT), x.dgate, x.dgn_w, x.dgn_b);
  else
    hipLaunchKernelGGL((bm_dout<OUTD, false>), gtiles, dim3(256), 0, st, a, Hd, x.gate, x.dout, at(L.DR),
                       at(L.DT), x.dgate, x.dgn_w, x.dgn_b);
  hipLaunchKernelGGL(bm_scan<1>, gscan, dim3(256), 0, st, a, static_cast<const uint16_t*>(at(L.QT)),
                     static_cast<const uint16_t*>(at(L.DT)), x.dstate_out, at(L.G), at(L.GT),
                     x.dstate_in, L.Np);
  hipLaunchKernelGGL(bm_dq, gtiles, dim3(256), 0, st, a, Hd, static_cast<const uint16_t*>(x.v), x.dq);
  hipLaunchKernelGGL(bm_dk, gtiles, dim3(256), 0, st, a, Hd, static_cast<const uint16_t*>(x.v), x.dk);
  hipLaunchKernelGGL(bm_dv, gtiles, dim3(256), 0, st, a, Hd, x.dv);
  return hipGetLastError();
}

}  // namespace

bool backward_mfma_supported(const CallArgs& a, int in_dt) {
  // (every per-head operand array is read through a buffer resource with 32-bit offsets:
  // under 2 GB, float32 dout included)
  return in_dt == RN_BF16 && a.dk % 8 == 0 && a.dv % 8 == 0 &&
         (int64_t(a.N) + 64) * max(a.dk, a.dv) * 4 < (int64_t(1) << 31);
}

size_t backward_mfma_ws_bytes(const CallArgs& a) { return m_layout(a).total; }

hipError_t launch_backward_mfma(const CallArgs& a, int out_dt, const BwArgs& x, void* ws,
                                hipStream_t st) {
  return out_dt == RN_F32 ? launch_t<RN_F32>(a, x, ws, st) : launch_t<RN_BF16>(a, x, ws, st);
}

}  // namespace rn
