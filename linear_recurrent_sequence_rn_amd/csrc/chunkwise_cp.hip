// Chunk-parallel schedule of the chunkwise form for bf16 q/k/v, d_k = 256, d_v = 512
// (hwhale notes: chunkwise equation and ChunkwiseRetention listing; m0nads notes,
// "Chunkwise representation"; GroupNorm + swish gate of the multi-scale layer).
//
// The chunkwise equation splits the output of chunk c (tokens [256c, 256c + 256)) into
//     O_t = alpha [ sum_{256c <= s <= t} gamma^(t-s) (Qh_t . Kh_s) V_s  +  gamma^(t-256c+1) Qh_t S_c ]
// where only the state S_c at the chunk's start links chunks. Two kernels, no
// communication between workgroups:
//   cp_states  walks each head's sequence once, carrying the float32 state, and writes
//              S_c (rounded to half) for every chunk of a window of 32 chunks:
//              S_{c+1} = gamma^L S_c + sum_j gamma^(L-1-j) Kh_j^T V_j.
//   cp_outputs computes 32 output rows per workgroup, independently: the cross term
//              against the chunk's snapshot, the causal intra-chunk part over the keys
//              from the chunk's start to its rows, then GroupNorm + gate and the store.
// Windows of 32 chunks bound the snapshot workspace independently of N; the float32
// state is carried between windows through the workspace.
//
// Both kernels compute with 16x16x32 f16 MFMA and float32 accumulation. Operands are
// rounded to IEEE half after the float32 rotation and decay (half keeps 3 more bits
// than bf16); they must stay within half's range, as must the state.
//
// One decay per coordinate pair (the form before the pages reduce the decay to a
// scalar: hwhale notes, A diagonalised as Λ(γe^{iθ})Λ^{-1}; m0nads notes, "Retention",
// γ and θ as two vectors). The decay of coordinate d can no longer be applied to a
// score after the product over d_k, so it is folded into the operands per coordinate,
// with every factor at most 1 wherever the fold allows it:
//   carry   Kh_j scaled by gamma_d^(L-1-j), state row d by gamma_d^L;
//   cross   Qh_t scaled by alpha gamma_d^(t-256c+1) before the product with S_c;
//   keys before the workgroup's rows (s < t0):
//           (alpha Qh_t gamma_d^(t-t0)) . (Kh_s gamma_d^(t0-s));
//   keys among its rows, per 16x16 score tile with anchor A (the middle of a diagonal
//   tile, the boundary between the two 16-row halves otherwise):
//           (alpha Qh_t gamma_d^(t-A)) . (Kh_s gamma_d^(A-s)),
//   formed in float32 from the unscaled half operands and multiplied as bf16 high and
//   low parts (three bf16 MFMA, about 16 significant bits), so that factors up to
//   gamma_d^-8 keep float32's exponent range; entries above the diagonal are dropped
//   by selection. Inside a diagonal tile a decay below 2^-13 is taken as 2^-13, which
//   changes a score term with t > s by less than 2^-13 of its undecayed size.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDK = 256;
constexpr int kDV = 512;
constexpr int kC = 256;                       // tokens per chunk (state snapshot spacing)
constexpr int kWin = 32;                      // chunks per window
constexpr int kHeadsPerGroup = 64;            // heads per pair of launches
constexpr size_t kSnapHalves = size_t(kDK) * kDV;   // one snapshot: 256 KB of half
constexpr uint32_t kSink = 0x80000000u;       // store offset past every range: dropped

// cp_states
constexpr int kT1 = 64;                       // tokens per block
constexpr int kBlkPerChunk = kC / kT1;
constexpr int kBlkPerWin = kWin * kBlkPerChunk;
constexpr int kLd1 = 72;                      // LDS pitch (half) of the transposed operands

// cp_outputs
constexpr int kQ = 32;                        // query rows per workgroup
constexpr int kKs = 32;                       // keys per intra-chunk step
constexpr int kPiece = 32;                    // d_k rows of a snapshot per cross step
constexpr int kLdQ = 264;                     // LDS pitch (half) of the Q / K row buffers
static_assert(kC / kQ == 8, "eight output workgroups per chunk (the grid mapping)");

template <int C> struct Ic { static constexpr int value = C; };

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 as_f16x8(u32x4 u) { return __builtin_bit_cast(f16x8, u); }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v;
  v[0] = static_cast<_Float16>(lo);
  v[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Buffer resource over [base, base + bytes): loads past the end return 0, stores past
// the end are dropped (ragged tails, rows past a sequence's length, sink offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes > 0 ? bytes : 0), 0x00020000);
}
__device__ __forceinline__ uint32_t ld_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void st_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, 0);
}
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8), through the builtin so that the compiler's own wait insertion sees them.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 15));
  __asm__ volatile("" ::: "memory");
}
// Barrier for LDS traffic only (global memory operations may stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ==================================== cp_states =========================================
// Workgroup (head, d_k quarter kq, d_v half vh): a 64 x 256 tile of the float32 state in
// MFMA accumulators (wave w: columns 64w..64w+63 of the half), walking the sequence in
// blocks of 64 tokens. Per block, each thread loads one rotation pair of K for 8
// consecutive tokens and two V columns for 4 x 8 tokens, rotates and decays K in
// float32, and writes both transposed into LDS (token-contiguous rows), where the
// carry's MFMA operands are read. Loads run two blocks ahead in registers; every
// iteration issues the same memory operations (snapshot stores outside chunk starts go
// to a dropped offset), so the waits have fixed counts.
//
// Decay within a chunk of L tokens: K row j (0-based in the chunk) is scaled by
// gamma^(L-1-j) before rounding, and the state by gamma^L at the chunk's start.
//
// Snapshot layout, per head and window slot: S^T in 8 pieces of 32 d_k rows,
// [piece][col 512][32] half, so that a piece is the A operand block of cp_outputs.
struct StateParams {
  CallArgs a;
  int head0, heads, win;
  const uint16_t* k;
  const uint16_t* v;
  const float* src;   // window's initial state, or null (zeros)
  int src_group;      // src indexed by group head (1) or by b*H + h (0)
  float* dst;         // window's final state, or null
  int dst_group;
  uint16_t* snap;     // [heads][kWin][kSnapHalves]
  uint32_t* status;   // the call's status word (bit 1: a non-finite final state)
};

constexpr int kLoads1 = 8 + 32;   // vector loads per thread and block
constexpr int kStores1 = 16;      // snapshot stores per thread and block

template <bool VEC>
__global__ void __launch_bounds__(256) cp_states(StateParams P) {
  const CallArgs& a = P.a;
  const int xcd = blockIdx.x & 7, L8 = blockIdx.x >> 3;
  const int hg = (L8 >> 3) * 8 + xcd;   // the 8 workgroups of a head share an XCD
  if (hg >= P.heads) return;
  const int sub = L8 & 7, kq = sub >> 1, vh = sub & 1;
  const int bh = P.head0 + hg, h = bh % a.H, seq = bh / a.H;
  const int N = a.N;
  const int len = seq_len(a, seq);
  const int64_t p0 = seq_pos0(a, seq);
  const int nb = (len + kT1 - 1) / kT1;
  const int b0 = P.win * kBlkPerWin;
  const int b1 = min(nb, b0 + kBlkPerWin);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const float lg = a.hp.log2g[h];

  __shared__ __attribute__((aligned(16))) uint16_t kt[2][64][kLd1];    // K^T: [d_k][token]
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][256][kLd1];   // V^T: [col][token]

  // state tile: acc[rt][ct] row d_k = 64kq + 16rt + 4g + r, column 256vh + 64w + 16ct + l16
  f32x4 acc[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (P.src) {
    const float* src = P.src + size_t(P.src_group ? hg : bh) * kDK * kDV;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 64 * kq + 16 * rt + 4 * g + r, c = 256 * vh + 64 * w + 16 * ct + l16;
          acc[rt][ct][r] = src[size_t(d) * kDV + c];
        }
  }

  const __amdgpu_buffer_rsrc_t rk = range_rsrc(P.k + size_t(bh) * N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(P.v + size_t(bh) * N * kDV, int64_t(len) * kDV * 2);
  const __amdgpu_buffer_rsrc_t rs =
      range_rsrc(P.snap + size_t(hg) * kWin * kSnapHalves, int64_t(kWin) * kSnapHalves * 2);

  // K: pair 32kq + pi of tokens 8tg .. 8tg+7 of a block
  const int pi = tid & 31, tg = tid >> 5;
  const float th = a.ap.theta[32 * kq + pi];
  // decays: of this thread's K pair, and of its accumulator rows (rt, r): pair
  // 32kq + 8rt + 2g + (r >> 1)
  const float lgk = VEC ? pair_log2g(a, h, 32 * kq + pi) : lg;
  float lgr[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) lgr[rt][hr] = VEC ? pair_log2g(a, h, 32 * kq + 8 * rt + 2 * g + hr) : lg;
  float c1, s1, c64, s64;
  angle_cs(1, th, &c1, &s1);
  angle_cs(kT1, th, &c64, &s64);
  float ca = 1.f, sa = 0.f;   // angle of token 8tg of the block being staged

  auto load = [&](int b, uint32_t* kr, uint32_t* vr) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      kr[j] = ld_b32(rk, static_cast<uint32_t>(((b * kT1 + 8 * tg + j) * kDK + 64 * kq + 2 * pi) * 2));
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = tid + 256 * it, cp = item & 127, vtg = item >> 7;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vr[8 * it + j] = ld_b32(rv, static_cast<uint32_t>(((b * kT1 + 8 * vtg + j) * kDV + 256 * vh + 2 * cp) * 2));
    }
  };
  // rotate, decay and transpose block b into LDS buffer bf
  auto stage = [&](int b, int bf, const uint32_t* kr, const uint32_t* vr) {
    if (((b - b0) & 15) == 0) angle_cs_fast(p0 + int64_t(b) * kT1 + 8 * tg, th, &ca, &sa);
    const int cidx = b / kBlkPerChunk;
    const int Lc = min(kC, len - kC * cidx);
    const int jc0 = kT1 * (b % kBlkPerChunk) + 8 * tg;
    float c = ca, s = sa;
    uint32_t ev[4], od[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      float y[2][2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint32_t x = kr[j + jj];
        const float x0 = bf_lo(x), x1 = bf_hi(x);
        const int jc = jc0 + j + jj;
        const float z = jc < Lc ? exp2f(lgk * float(Lc - 1 - jc)) : 0.f;
        y[jj][0] = (x0 * c - x1 * s) * z;
        y[jj][1] = (x0 * s + x1 * c) * z;
        const float cn = c * c1 - s * s1;
        s = c * s1 + s * c1;
        c = cn;
      }
      ev[j >> 1] = pack_f16x2(y[0][0], y[1][0]);
      od[j >> 1] = pack_f16x2(y[0][1], y[1][1]);
    }
    *reinterpret_cast<u32x4*>(&kt[bf][2 * pi][8 * tg]) = u32x4{ev[0], ev[1], ev[2], ev[3]};
    *reinterpret_cast<u32x4*>(&kt[bf][2 * pi + 1][8 * tg]) = u32x4{od[0], od[1], od[2], od[3]};
    {
      const float cn = ca * c64 - sa * s64;
      sa = ca * s64 + sa * c64;
      ca = cn;
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int item = tid + 256 * it, cp = item & 127, vtg = item >> 7;
      uint32_t e2[4], o2[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t x0 = vr[8 * it + j], x1 = vr[8 * it + j + 1];
        e2[j >> 1] = pack_f16x2(bf_lo(x0), bf_lo(x1));
        o2[j >> 1] = pack_f16x2(bf_hi(x0), bf_hi(x1));
      }
      *reinterpret_cast<u32x4*>(&vt[bf][2 * cp][8 * vtg]) = u32x4{e2[0], e2[1], e2[2], e2[3]};
      *reinterpret_cast<u32x4*>(&vt[bf][2 * cp + 1][8 * vtg]) = u32x4{o2[0], o2[1], o2[2], o2[3]};
    }
  };
  auto carry = [&](int bf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 A[4], Bv[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        A[rt] = as_f16x8(*reinterpret_cast<const u32x4*>(&kt[bf][16 * rt + l16][32 * ks + 8 * g]));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        Bv[ct] = as_f16x8(*reinterpret_cast<const u32x4*>(&vt[bf][64 * w + 16 * ct + l16][32 * ks + 8 * g]));
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma(A[rt], Bv[ct], acc[rt][ct]);
    }
  };

  uint32_t kr0[8], vr0[32], kr1[8], vr1[32];
  // one block: snapshot (at a chunk's start) and decay, carry, stage the next block,
  // issue the loads two blocks ahead
  auto iter = [&](int b, uint32_t* krn, uint32_t* vrn, int bf) {
    const bool live = b < b1;
    u32x2 snapv[4][4];
    const bool chunk_start = live && (b % kBlkPerChunk) == 0;
    if (chunk_start) {
      const float Lf = float(min(kC, len - kC * (b / kBlkPerChunk)));
      float gL[4][2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) gL[rt][hr] = exp2f(lgr[rt][hr] * Lf);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          snapv[rt][ct] = u32x2{pack_f16x2(acc[rt][ct][0], acc[rt][ct][1]),
                                pack_f16x2(acc[rt][ct][2], acc[rt][ct][3])};
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[rt][ct][r] *= gL[rt][r >> 1];
        }
    } else {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) snapv[rt][ct] = u32x2{0u, 0u};
    }
    if (live) carry(bf);
    wait_vm<kLoads1 + kStores1>();   // loads of block b+1 are complete
    stage(b + 1, bf ^ 1, krn, vrn);
    // outside chunk starts the offset is moved past the range (no branch, so that every
    // path issues the same stores)
    const int cl = max(b / kBlkPerChunk - P.win * kWin, 0);
    const uint32_t sink = chunk_start ? 0u : kSink;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col = 256 * vh + 64 * w + 16 * ct + l16;
        const uint32_t off = static_cast<uint32_t>(
            ((size_t(cl * 8 + 2 * kq + (rt >> 1)) * kDV + col) * kPiece + 16 * (rt & 1) + 4 * g) * 2);
        st_b64(rs, off + sink, snapv[rt][ct]);
      }
    load(b + 3, krn, vrn);
    lds_barrier();
  };

  if (b0 < b1) {
    load(b0, kr0, vr0);
    wait_vm<0>();
    stage(b0, 0, kr0, vr0);
    load(b0 + 1, kr1, vr1);
    load(b0 + 2, kr0, vr0);
    // nothing in flight on entry to the loop: the first iteration waits for what it
    // consumes, as the later ones do
    wait_vm<0>();
    lds_barrier();
    for (int b = b0; b < b1; b += 2) {
      iter(b, kr1, vr1, 0);
      iter(b + 1, kr0, vr0, 1);
    }
    wait_vm<0>();
  }

  if (P.dst) {
    float* dst = P.dst + size_t(P.dst_group ? hg : bh) * kDK * kDV;
    uint32_t bad = 0u;   // set by a non-finite value of the caller's final state
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = 64 * kq + 16 * rt + 4 * g + r, c = 256 * vh + 64 * w + 16 * ct + l16;
          dst[size_t(d) * kDV + c] = acc[rt][ct][r];
          bad |= __builtin_isfinite(acc[rt][ct][r]) ? 0u : 1u;
        }
    if (!P.dst_group && __builtin_amdgcn_ballot_w64(bad != 0u) != 0 && l == 0)
      __hip_atomic_fetch_or(P.status, kChunkwiseStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// =================================== cp_outputs =========================================
// Workgroup (head, 32 query rows t0 .. t0+31 of chunk c); four waves, wave w owning
// output columns 128w .. 128w+127. The output is computed transposed, O^T = A B with
// A = S^T or V^T (rows: output columns) and B = Qh or P (columns: query rows), so that
// each lane ends with 32 consecutive columns of one query row: column
// 128w + 32g + 4tb + r sits in accumulator tile tb, row 4g + r.
// Phases, each staged in LDS by the whole workgroup with the next phase's loads in
// flight behind it:
//   8 cross steps: a 32-row piece of S_c^T times alpha Qh (then each row scaled by
//     xi_t = gamma^(t - 256c + 1));
//   one step per 32 keys from the chunk's start to the workgroup's last row: scores
//     P^T = Kh (alpha Qh)^T with the decay gamma^(t-s) and the causal mask applied in
//     float32, rounded to half, then V^T P^T.
// GroupNorm statistics are reduced over the four waves through LDS.
struct OutParams {
  CallArgs a;
  int head0, heads, win;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  const uint16_t* snap;
  void* out;
  uint32_t* status;   // the call's status word (bit 1: a non-finite output)
};

// Rows of the transposed-operand buffer hold 32 half values (4 chunks of 16 bytes);
// chunk c of row r sits at position c ^ ((r >> 5) & 3), so the 16 rows one A-operand
// read touches (4 groups of 4 consecutive rows, 32 rows apart) hit distinct banks.
__device__ __forceinline__ int vt_chunk(int r, int c) { return c ^ ((r >> 5) & 3); }
// P rows (one per query) swizzle by (r >> 2) & 3: 16 consecutive rows, one chunk each.
__device__ __forceinline__ int ps_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }

struct alignas(16) SharedO {
  uint16_t qs[kQ][kLdQ];     // alpha Qh of the workgroup's rows
  uint16_t ks[kKs][kLdQ];    // Kh of the current key step
  uint16_t vt[kDV][32];      // V^T of the key step, or a snapshot piece (swizzled rows)
  uint16_t ps[kQ][32];       // P[q][key] (swizzled rows); GroupNorm partial sums at the end
  float gwb[2][kDV];         // GroupNorm weight and bias of the head
  float lgp[kDK / 2];        // log2 of each pair's decay (one decay per pair only)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x -> (hi, lo) with hi = bf16(x), lo = bf16(x - hi): hi + lo keeps about 16 bits of x
// over float32's exponent range. Element i of the two vectors.
__device__ __forceinline__ void split_bf16(float x, bf16x8& hi, bf16x8& lo, int i) {
  const __bf16 h = static_cast<__bf16>(x);
  hi[i] = h;
  lo[i] = static_cast<__bf16>(x - static_cast<float>(h));
}

template <int OUT, bool VEC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
cp_outputs(OutParams P) {
  const CallArgs& a = P.a;
  const int x = blockIdx.x;
  const int ci = 8 * (x >> 6) + (x & 7);   // (head, chunk) instance: its 8 workgroups share an XCD
  const int m = (x >> 3) & 7;              // 32-row block within the chunk
  const int hg = ci / kWin, cl = ci % kWin;
  if (hg >= P.heads) return;
  const int bh = P.head0 + hg, h = bh % a.H, seq = bh / a.H;
  const int N = a.N;
  const int len = seq_len(a, seq);
  const int64_t p0 = seq_pos0(a, seq);
  const int c0 = (P.win * kWin + cl) * kC;
  const int t0 = c0 + kQ * m;
  if (t0 >= len) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;
  const float lg = a.hp.log2g[h];
  const bool use_gn = a.flags & RN_EPI_GN;
  const bool has_gate = P.gate != nullptr;

  __shared__ SharedO sm;

  const __amdgpu_buffer_rsrc_t rq = range_rsrc(P.q + size_t(bh) * N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rk = range_rsrc(P.k + size_t(bh) * N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(P.v + size_t(bh) * N * kDV, int64_t(len) * kDV * 2);
  const __amdgpu_buffer_rsrc_t rg =
      range_rsrc((has_gate ? P.gate : P.v) + size_t(bh) * N * kDV, int64_t(len) * kDV * 2);
  const __amdgpu_buffer_rsrc_t rsn = range_rsrc(
      P.snap + (size_t(hg) * kWin + cl) * kSnapHalves, int64_t(kSnapHalves) * 2);
  const int osz = OUT == RN_BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t ro = range_rsrc(
      static_cast<uint8_t*>(P.out) + size_t(bh) * N * kDV * osz, int64_t(len) * kDV * osz);

  // GroupNorm affine parameters of the head (loaded with the prologue's rows)
  float gwv[2] = {1.f, 1.f}, gbv[2] = {0.f, 0.f};
  if (a.gn_w) {
    gwv[0] = a.gn_w[size_t(h) * kDV + tid];
    gwv[1] = a.gn_w[size_t(h) * kDV + tid + 256];
  }
  if (a.gn_b) {
    gbv[0] = a.gn_b[size_t(h) * kDV + tid];
    gbv[1] = a.gn_b[size_t(h) * kDV + tid + 256];
  }

  // Row loader/rotator for Q and K: pair pj of rows rg2 + 2i (i < 16) of a 32-row step.
  const int pj = tid & 127, rg2 = tid >> 7;
  const float th = a.ap.theta[pj];
  const float lgq = VEC ? pair_log2g(a, h, pj) : 0.f;   // decay of the staged pair
  float c2, s2;
  angle_cs(2, th, &c2, &s2);
  auto load_rows = [&](__amdgpu_buffer_rsrc_t r, int row0, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dst[i >> 2][i & 3] = ld_b32(r, static_cast<uint32_t>(((row0 + rg2 + 2 * i) * kDK + 2 * pj) * 2));
  };
  // Rows scaled by `scale`, and with one decay per pair by gamma^(row - anchor) as well
  // (lgs = log2 gamma of the staged pair, or its negative for gamma^(anchor - row)).
  auto stage_rows = [&](int row0, const u32x4* src, uint16_t (*buf)[kLdQ], float scale,
                        float lgs = 0.f, int anchor = 0) {
    float c, s;
    angle_cs_fast(p0 + row0 + rg2, th, &c, &s);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t word = src[i >> 2][i & 3];
      const float x0 = bf_lo(word), x1 = bf_hi(word);
      float f = scale;
      if constexpr (VEC) f *= exp2f(lgs * float(row0 + rg2 + 2 * i - anchor));
      *reinterpret_cast<uint32_t*>(&buf[rg2 + 2 * i][2 * pj]) =
          pack_f16x2((x0 * c - x1 * s) * f, (x0 * s + x1 * c) * f);
      const float cn = c * c2 - s * s2;
      s = c * s2 + s * c2;
      c = cn;
    }
  };
  // V^T of keys key0 .. key0+31: thread tiles of 4 keys x 4 columns
  auto load_v = [&](int key0, u32x4* dst) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u, cq = e & 127, kq4 = e >> 7;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 x = ld_b64(rv, static_cast<uint32_t>(((key0 + 4 * kq4 + i) * kDV + 4 * cq) * 2));
        const int te = 4 * u + i;
        dst[te >> 1][2 * (te & 1)] = x[0];
        dst[te >> 1][2 * (te & 1) + 1] = x[1];
      }
    }
  };
  auto stage_v = [&](const u32x4* src) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 256 * u, cq = e & 127, kq4 = e >> 7;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int te = 4 * u + i;
          const uint32_t word = src[te >> 1][2 * (te & 1) + (cc >> 1)];
          f[i] = (cc & 1) ? bf_hi(word) : bf_lo(word);
        }
        const int row = 4 * cq + cc;
        const int pos = 8 * vt_chunk(row, kq4 >> 1) + 4 * (kq4 & 1);
        *reinterpret_cast<u32x2*>(&sm.vt[row][pos]) = u32x2{pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3])};
      }
    }
  };
  // snapshot piece p: 32 KB contiguous, 16 bytes per thread and step
  auto load_piece = [&](int p, u32x4* dst) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      dst[u] = ld_b128(rsn, static_cast<uint32_t>((size_t(p) * kDV * kPiece) * 2 + 16 * (tid + 256 * u)));
  };
  auto stage_piece = [&](const u32x4* src) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = tid + 256 * u, row = e >> 2, c = e & 3;
      *reinterpret_cast<u32x4*>(&sm.vt[row][8 * vt_chunk(row, c)]) = src[u];
    }
  };
  // gate rows of the workgroup: lane's 32 columns of rows 16mq + l16
  auto load_gate = [&](u32x4* dst) {
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
      for (int pc = 0; pc < 4; ++pc)
        dst[4 * mq + pc] = ld_b128(rg, static_cast<uint32_t>(((t0 + 16 * mq + l16) * kDV + 128 * w + 32 * g + 8 * pc) * 2));
  };

  // A operand rows of tile tb: output column of A-row i = l16
  const int arow0 = 128 * w + 32 * (l16 >> 2) + (l16 & 3);
  f32x4 acc[8][2];
#pragma unroll
  for (int tb = 0; tb < 8; ++tb)
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) acc[tb][mq] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma_vt = [&](int bcol0, const uint16_t (*bsrc)[kLdQ], bool bq) {
    // acc += A (vt rows) x B; B rows from qs (cross: d_k offset bcol0) or ps (intra)
    f16x8 A[8], Bq[2];
#pragma unroll
    for (int tb = 0; tb < 8; ++tb) {
      const int row = arow0 + 4 * tb;
      A[tb] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.vt[row][8 * vt_chunk(row, g)]));
    }
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const int qr = 16 * mq + l16;
      if (bq)
        Bq[mq] = as_f16x8(*reinterpret_cast<const u32x4*>(&bsrc[qr][bcol0 + 8 * g]));
      else
        Bq[mq] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.ps[qr][8 * ps_chunk(qr, g)]));
    }
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) acc[tb][mq] = mfma(A[tb], Bq[mq], acc[tb][mq]);
  };

  // ---- prologue: Q rows and the first snapshot piece ------------------------------------
  // Each phase's data is loaded into `pre` while the phase before it computes: a
  // snapshot piece (pre[0..7]), or K rows (pre[0..3]) and V tiles (pre[4..11]). The
  // cross phases are unrolled and the key steps share one body, so that every phase
  // loads into the same registers unconditionally (no copies between them that would
  // wait for loads in flight).
  const int nsteps = m + 1;                 // key steps of 32 from the chunk's start
  u32x4 qx[4];
  u32x4 pre[12];
  u32x4 gt[8];                              // gate rows, loaded with the first key step
  load_rows(rq, t0, qx);
  load_piece(0, pre);
  wait_vm<0>();
  // cross operand: alpha Qh_t, with one decay per pair scaled by gamma^(t - c0 + 1) (xi)
  stage_rows(t0, qx, sm.qs, a.alpha, lgq, c0 - 1);
  if constexpr (VEC)
    if (tid < kDK / 2) sm.lgp[tid] = lgq;
  sm.gwb[0][tid] = gwv[0];
  sm.gwb[0][tid + 256] = gwv[1];
  sm.gwb[1][tid] = gbv[0];
  sm.gwb[1][tid + 256] = gbv[1];

  auto cross_phase = [&](auto pc) {
    constexpr int ph = decltype(pc)::value;
    lds_barrier();                          // the previous phase's LDS reads are done
    stage_piece(pre);
    if constexpr (ph + 1 < 8) {
      load_piece(ph + 1, pre);
    } else {
      load_rows(rk, c0, pre);
      load_v(c0, pre + 4);
      if constexpr (!VEC) load_gate(gt);   // with pair decays: after the key steps
    }
    lds_barrier();
    mma_vt(kPiece * ph, sm.qs, true);
    wait_vm<0>();                           // next phase's loads are complete
  };
  cross_phase(Ic<0>{});
  cross_phase(Ic<1>{});
  cross_phase(Ic<2>{});
  cross_phase(Ic<3>{});
  cross_phase(Ic<4>{});
  cross_phase(Ic<5>{});
  cross_phase(Ic<6>{});
  cross_phase(Ic<7>{});
  // xi_t = gamma^(t - c0 + 1) per query row (column of the transposed tiles); with one
  // decay per pair it was folded into the operand
  if constexpr (!VEC) {
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const float xi = exp2f(lg * float(t0 + 16 * mq + l16 - c0 + 1));
#pragma unroll
      for (int tb = 0; tb < 8; ++tb) acc[tb][mq] *= xi;
    }
  }

  for (int st = 0; st < nsteps; ++st) {
    const int key0 = c0 + kKs * st;
    const bool diag = st == nsteps - 1;     // keys t0 .. t0+31: the workgroup's own rows
    lds_barrier();
    if constexpr (VEC) {
      // keys before t0: Q by gamma^(t - t0), K by gamma^(t0 - s); own rows: unscaled
      // (the score tiles scale them in registers)
      if (diag)
        stage_rows(t0, qx, sm.qs, a.alpha);
      else if (st == 0)
        stage_rows(t0, qx, sm.qs, a.alpha, lgq, t0);
      stage_rows(key0, pre, sm.ks, 1.f, diag ? 0.f : -lgq, t0);
    } else {
      stage_rows(key0, pre, sm.ks, 1.f);
    }
    stage_v(pre + 4);
    // the next step's rows (past the last step: rows the workgroup does not use)
    load_rows(rk, key0 + kKs, pre);
    load_v(key0 + kKs, pre + 4);
    lds_barrier();
    // scores P^T = Kh (alpha Qh)^T for key tile mk = w >> 1, query tile mq = w & 1
    {
      const int mk = w >> 1, mq = w & 1;
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!VEC || !diag) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const f16x8 A = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.ks[16 * mk + l16][32 * kk + 8 * g]));
          const f16x8 Bq = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.qs[16 * mq + l16][32 * kk + 8 * g]));
          sc = mfma(A, Bq, sc);
        }
      } else if (mk <= mq) {   // (the tile with mk > mq lies above the diagonal)
        // tile among the workgroup's rows: decays applied here per coordinate around the
        // anchor A = t0 + 8 + 8 (mk + mq); A-operand row = key 16mk + l16, B-operand row
        // = query 16mq + l16, k-elements 32kk + 8g .. +7 (pairs 16kk + 4g .. +3)
        const int anc = 8 + 8 * (mk + mq);
        const float ek = float(anc - 16 * mk - l16), eq = float(16 * mq + l16 - anc);
        const float lo_lim = mk == mq ? -13.f : -__builtin_inff();
#pragma clang loop unroll(disable)
        for (int kk = 0; kk < 8; ++kk) {
          const f16x8 kx = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.ks[16 * mk + l16][32 * kk + 8 * g]));
          const f16x8 qv = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.qs[16 * mq + l16][32 * kk + 8 * g]));
          bf16x8 kh, kl, qh, ql;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lgv = fmaxf(sm.lgp[16 * kk + 4 * g + i], lo_lim);
            const float fk = exp2f(lgv * ek), fq = exp2f(lgv * eq);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              split_bf16(static_cast<float>(kx[2 * i + e]) * fk, kh, kl, 2 * i + e);
              split_bf16(static_cast<float>(qv[2 * i + e]) * fq, qh, ql, 2 * i + e);
            }
          }
          sc = mfma_bf16(kh, qh, sc);
          sc = mfma_bf16(kh, ql, sc);
          sc = mfma_bf16(kl, qh, sc);
        }
      }
      const int tq = t0 + 16 * mq + l16;
      float pvv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = key0 + 16 * mk + 4 * g + r;
        const float e = VEC ? 1.f : exp2f(lg * float(max(tq - s, 0)));
        pvv[r] = s <= tq ? sc[r] * e : 0.f;
      }
      const int qrow = 16 * mq + l16;
      const int kc = 16 * mk + 4 * g;        // first key of the lane's four
      *reinterpret_cast<u32x2*>(&sm.ps[qrow][8 * ps_chunk(qrow, kc >> 3) + (kc & 7)]) =
          u32x2{pack_f16x2(pvv[0], pvv[1]), pack_f16x2(pvv[2], pvv[3])};
    }
    lds_barrier();
    mma_vt(0, sm.qs, false);
    wait_vm<0>();
  }
  // with pair decays the gate rows are loaded here, behind the GroupNorm statistics,
  // which keeps them out of the registers the key steps need
  if constexpr (VEC) load_gate(gt);

  // ---- epilogue: GroupNorm over the 512 columns of each row, gate, store ----------------
  float y[8][2][4];
#pragma unroll
  for (int tb = 0; tb < 8; ++tb)
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
      for (int r = 0; r < 4; ++r) y[tb][mq][r] = acc[tb][mq][r];
  if (use_gn) {
    float* red = reinterpret_cast<float*>(&sm.ps[0][0]);   // [4 waves][32 rows]
    float mean[2], rstd[2];
    float part[2];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      float s = 0.f;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += y[tb][mq][r];
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      part[mq] = s;
    }
    lds_barrier();
    if (g == 0) {
      red[32 * w + l16] = part[0];
      red[32 * w + 16 + l16] = part[1];
    }
    lds_barrier();
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const int qrow = 16 * mq + l16;
      mean[mq] = (red[qrow] + red[32 + qrow] + red[64 + qrow] + red[96 + qrow]) * (1.f / kDV);
      float s = 0.f;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = y[tb][mq][r] - mean[mq];
          s = fmaf(d, d, s);
        }
      s += __shfl_xor(s, 16, 64);
      s += __shfl_xor(s, 32, 64);
      part[mq] = s;
    }
    lds_barrier();
    if (g == 0) {
      red[32 * w + l16] = part[0];
      red[32 * w + 16 + l16] = part[1];
    }
    lds_barrier();
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const int qrow = 16 * mq + l16;
      const float m2 = red[qrow] + red[32 + qrow] + red[64 + qrow] + red[96 + qrow];
      rstd[mq] = __frsqrt_rn(fmaf(m2, 1.f / kDV, a.eps));
    }
#pragma unroll
    for (int tb = 0; tb < 8; ++tb)
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = 128 * w + 32 * g + 4 * tb + r;
          y[tb][mq][r] = fmaf((y[tb][mq][r] - mean[mq]) * rstd[mq], sm.gwb[0][col], sm.gwb[1][col]);
        }
    if (has_gate) {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int pc = 0; pc < 4; ++pc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t word = gt[4 * mq + pc][e >> 1];
            const float gv = (e & 1) ? bf_hi(word) : bf_lo(word);
            const int tb = 2 * pc + (e >> 2), r = e & 3;
            y[tb][mq][r] *= swishf(gv);
          }
    }
  }
  {
    // a class test per stored value of the sequence's rows
    uint32_t bad = 0u;
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      const bool vrow = t0 + 16 * mq + l16 < len;
#pragma unroll
      for (int tb = 0; tb < 8; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) bad |= (vrow && !__builtin_isfinite(y[tb][mq][r])) ? 1u : 0u;
    }
    if (__builtin_amdgcn_ballot_w64(bad != 0u) != 0 && l == 0)
      __hip_atomic_fetch_or(P.status, kChunkwiseStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int mq = 0; mq < 2; ++mq) {
    const int row = t0 + 16 * mq + l16;
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      const int col = 128 * w + 32 * g + 8 * pc;
      const int tb = 2 * pc;
      if constexpr (OUT == RN_BF16) {
        st_b128(ro, static_cast<uint32_t>((row * kDV + col) * 2),
                u32x4{pack_bf16x2(y[tb][mq][0], y[tb][mq][1]), pack_bf16x2(y[tb][mq][2], y[tb][mq][3]),
                      pack_bf16x2(y[tb + 1][mq][0], y[tb + 1][mq][1]),
                      pack_bf16x2(y[tb + 1][mq][2], y[tb + 1][mq][3])});
      } else {
        st_b128(ro, static_cast<uint32_t>((row * kDV + col) * 4),
                __builtin_bit_cast(u32x4, f32x4{y[tb][mq][0], y[tb][mq][1], y[tb][mq][2], y[tb][mq][3]}));
        st_b128(ro, static_cast<uint32_t>((row * kDV + col) * 4 + 16),
                __builtin_bit_cast(u32x4, f32x4{y[tb + 1][mq][0], y[tb + 1][mq][1], y[tb + 1][mq][2],
                                                y[tb + 1][mq][3]}));
      }
    }
  }
}

int chunks_of(int N) { return (N + kC - 1) / kC; }

__global__ void cp_status_clear(uint32_t* status) {
  if (threadIdx.x == 0) status[0] = 0u;
}

constexpr size_t kStatusBytes = 256;   // the call's status word leads the workspace

}  // namespace

bool chunkwise_cp_supported(const CallArgs& a, int in_dt) {
  if (in_dt != RN_BF16 || a.dk != kDK || a.dv != kDV) return false;
  // 32-bit buffer offsets within one head's rows, with loads up to 512 rows past the end
  return (int64_t(a.N) + 512) * kDV * 4 < (int64_t(1) << 31);
}

// A full window of snapshots and the carried state per head of a group, whatever N is.
size_t chunkwise_cp_ws_bytes(const CallArgs& a) {
  const int heads = min(a.B * a.H, kHeadsPerGroup);
  return kStatusBytes + size_t(heads) * (kWin * kSnapHalves * sizeof(uint16_t) + size_t(kDK) * kDV * sizeof(float));
}

hipError_t launch_chunkwise_cp(const CallArgs& a, int out_dt, const void* q, const void* k,
                               const void* v, const void* gate, const float* s_in, float* s_out,
                               void* out, void* ws, size_t ws_bytes, hipStream_t st) {
  const int total = a.B * a.H;
  const int nch = chunks_of(a.N);
  const int nwin = (nch + kWin - 1) / kWin;
  const size_t snap_bytes = size_t(min(total, kHeadsPerGroup)) * kWin * kSnapHalves * sizeof(uint16_t);
  if (chunkwise_cp_ws_bytes(a) > ws_bytes) return hipErrorInvalidValue;
  uint32_t* status = static_cast<uint32_t*>(ws);
  uint16_t* snap = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + kStatusBytes);
  float* carry = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kStatusBytes + snap_bytes);
  hipLaunchKernelGGL(cp_status_clear, dim3(1), dim3(64), 0, st, status);
  for (int h0 = 0; h0 < total; h0 += kHeadsPerGroup) {
    const int heads = min(kHeadsPerGroup, total - h0);
    for (int win = 0; win < nwin; ++win) {
      StateParams sp;
      sp.a = a;
      sp.head0 = h0;
      sp.heads = heads;
      sp.win = win;
      sp.k = static_cast<const uint16_t*>(k);
      sp.v = static_cast<const uint16_t*>(v);
      sp.src = win == 0 ? s_in : carry;
      sp.src_group = win == 0 ? 0 : 1;
      sp.dst = win + 1 == nwin ? s_out : carry;
      sp.dst_group = win + 1 == nwin ? 0 : 1;
      sp.snap = snap;
      sp.status = status;
      if (a.gpair)
        hipLaunchKernelGGL(cp_states<true>, dim3(64 * ((heads + 7) / 8)), dim3(256), 0, st, sp);
      else
        hipLaunchKernelGGL(cp_states<false>, dim3(64 * ((heads + 7) / 8)), dim3(256), 0, st, sp);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      OutParams op;
      op.a = a;
      op.head0 = h0;
      op.heads = heads;
      op.win = win;
      op.q = static_cast<const uint16_t*>(q);
      op.k = static_cast<const uint16_t*>(k);
      op.v = static_cast<const uint16_t*>(v);
      op.gate = static_cast<const uint16_t*>(gate);
      op.snap = snap;
      op.out = out;
      op.status = status;
      const int inst = heads * kWin;
      const dim3 grid(64 * ((inst + 7) / 8));
      if (a.gpair) {
        if (out_dt == RN_BF16)
          hipLaunchKernelGGL((cp_outputs<RN_BF16, true>), grid, dim3(256), 0, st, op);
        else
          hipLaunchKernelGGL((cp_outputs<RN_F32, true>), grid, dim3(256), 0, st, op);
      } else {
        if (out_dt == RN_BF16)
          hipLaunchKernelGGL((cp_outputs<RN_BF16, false>), grid, dim3(256), 0, st, op);
        else
          hipLaunchKernelGGL((cp_outputs<RN_F32, false>), grid, dim3(256), 0, st, op);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace rn
