// Parallel retention with MFMA for bf16 q/k/v, d_k = 256, d_v = 512
// (hwhale notes: parallel-form equation, ParallelRetention listing and the list of
// three rescalings).
//
// Two kernels.
//  1. prep: rotates q (scaled by alpha) and k once into half precision, row-major, and
//     writes v transposed per 64-row block (V^T[block][d_v][64]) in half, into the
//     caller's workspace. Rotating k here instead of in the main kernel avoids redoing
//     it for every query block that reads the key block (32 x on average at N = 2048).
//  2. main: one 512-thread workgroup (8 waves) per (head, 128-row query block), walking
//     the 64-row key blocks that have causal pairs with it. Each key block of Kh is
//     copied once into LDS (buffer loads with the lds modifier, two buffers, two blocks
//     ahead). Wave w computes the scores of query rows 16w..16w+15 against the 64 keys
//     (16x16x32 f16 MFMA over all of d_k, taken as K Q^T), applies gamma^(t-s) (a per-lane
//     factor times a per-block one) and, on the two diagonal key blocks, the causal mask,
//     accumulates the signed row sums for the R normalisation and writes the scores to
//     LDS in half (two buffers: the scores of block kb+1 are computed while block kb is
//     multiplied with V); every wave then multiplies all 128 score rows with its 64
//     columns of V, whose fragments it loads in two halves of 32 keys: the first half
//     of the next key block during the current product, so V's latency sits behind a
//     half or a whole block of work. At the end each row is scaled by
//     c_t = 1/sqrt(sum_{m<=t} gamma^m) (D normalisation) and 1/max(c_t |rowsum|, 1)
//     (R normalisation), then GroupNorm (+ gate) over the 512 columns, whose sums are
//     combined across the waves in LDS.
// Register budget: the accumulators (128 rows x 64 columns per wave) take half of each
// wave's 256 VGPRs and the rest is full; with fewer rows per workgroup (64) the loop's
// LDS reads batch well but every key/value block is read twice as often, which was
// measured slower (0.64 against 0.56 ms per call at the 1.3B shape).
// Query blocks are launched from the last (most key blocks) to the first, and each head's
// blocks all go to one XCD.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kT = 64;      // rows per block
constexpr int kDK = 256;
constexpr int kDV = 512;
constexpr int kPLd = 72;    // LDS row stride (half) of the score block

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8), issued through the builtin so that the compiler's own wait insertion sees it.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

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
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over each row of 16 lanes, every lane receiving the row's sum (DPP moves, VALU
// only): swap neighbours, swap pairs, mirror within 8 lanes, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);    // lane ^ 1
  x += dpp_mov<0x4E>(x);    // lane ^ 2
  x += dpp_mov<0x141>(x);   // lane i <-> 7 - i within 8
  x += dpp_mov<0x140>(x);   // lane i <-> 15 - i within 16
  return x;
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes > 0 ? bytes : 0), 0x00020000);
}
__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}

// Workspace per head: Kh [Np][256], Vt [Np/64][512][64], both half, with Np = N rounded
// up to 64 (rows past N are zero). (q is rotated by the main kernel itself: each query
// row is read by one workgroup only.)
struct Ws {
  size_t k, v, head;   // element offsets within a head, and elements per head
};
__host__ __device__ inline Ws ws_layout(int N) {
  const size_t np = size_t((N + kT - 1) / kT) * kT;
  Ws w;
  w.k = 0;
  w.v = np * kDK;
  w.head = np * kDK + np * kDV;
  return w;
}

// Order of the 64 keys of a block inside a row of V^T (and of the score block in LDS):
// key s = 32e + 16h + 4g + r (e, h in {0,1}, g, r in [0,4)) sits at position
// 32e + 8g + 4h + r. Lane group g of a 16x16x32 MFMA then finds its 8 k-values (keys
// 32e + 4g + {0..3} and 32e + 16 + 4g + {0..3}) in 16 contiguous bytes, which are also
// the 8 scores that a lane holds after the transposed score product K Q^T.
__host__ __device__ constexpr int vt_pos(int s) {
  return 32 * (s >> 5) + 8 * ((s >> 2) & 3) + 4 * ((s >> 4) & 1) + (s & 3);
}

// ---- prep: one 256-thread block per (64-row block, head) ------------------------------
// bf16 inputs only. k: thread = (group of 4 coordinate pairs = 16 bytes, group of 8 rows);
// 16-byte loads, angles by recurrence along the rows. v: thread = 8 rows x 8 columns,
// transposed in registers, assembled as V^T (keys in vt_pos order) in LDS and written
// out as one contiguous run.
__global__ void __launch_bounds__(256) parallel_prep(CallArgs a, const uint16_t* k,
                                                     const uint16_t* v, uint16_t* ws) {
  const int jb = blockIdx.x, bh = blockIdx.y;
  const int N = a.N, tid = threadIdx.x;
  const Ws L = ws_layout(N);
  uint16_t* base = ws + size_t(bh) * L.head;
  const int row0 = jb * kT;
  const int64_t bytes_qk = int64_t(N) * kDK * 2, bytes_v = int64_t(N) * kDV * 2;
  const __amdgpu_buffer_rsrc_t rk = range_rsrc(k + size_t(bh) * N * kDK, bytes_qk);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(v + size_t(bh) * N * kDV, bytes_v);
  // Every load of the thread is issued before any store (the compiler cannot reorder a
  // load past a store to memory it cannot prove distinct), so the 32 loads are in
  // flight together.
  const int pg = tid & 31, rg = tid >> 5;     // k: pairs 4pg..4pg+3, rows 8rg..8rg+7
  u32x4 xk[8], xv[2][8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t off = static_cast<uint32_t>(((row0 + 8 * rg + u) * kDK + 8 * pg) * 2);
    xk[u] = ld_b128(rk, off);   // zero past N
  }
  // v: 8x8 tiles; 64 x 512 block = 512 tiles, 2 per thread: columns 8cg..8cg+7, rows
  // 8sg..8sg+7 of tile tid + 256 rep
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int tile = tid + 256 * rep;
    const int cg = tile & 63, sg = tile >> 6;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xv[rep][i] = ld_b128(rv, static_cast<uint32_t>(((row0 + 8 * sg + i) * kDV + 8 * cg) * 2));
  }
  {
    float cs[4], sn[4], c1[4], s1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float th = a.ap.theta[4 * pg + i];
      angle_cs(1, th, &c1[i], &s1[i]);
      angle_cs(a.pos0 + row0 + 8 * rg, th, &cs[i], &sn[i]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = row0 + 8 * rg + u;
      u32x4 ok;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float k0 = __uint_as_float(xk[u][i] << 16), k1 = __uint_as_float(xk[u][i] & 0xffff0000u);
        ok[i] = pack_f16x2(k0 * cs[i] - k1 * sn[i], k0 * sn[i] + k1 * cs[i]);
        const float cn = cs[i] * c1[i] - sn[i] * s1[i];
        sn[i] = cs[i] * s1[i] + sn[i] * c1[i];
        cs[i] = cn;
      }
      *reinterpret_cast<u32x4*>(base + L.k + size_t(t) * kDK + 8 * pg) = ok;
    }
  }
  // V^T of the block (512 rows of 64 keys in vt_pos order, 64 KB) is assembled in LDS
  // and written out as one contiguous run of 16-byte pieces. LDS row c holds its eight
  // 16-byte pieces in the order piece ^ ((c >> 3) & 7), which spreads the 8-byte
  // writes of a wave (rows 8 apart) over the banks and keeps the read-out conflict free.
  __shared__ __attribute__((aligned(16))) uint16_t tv[kDV * kT];
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int tile = tid + 256 * rep;
    const int cg = tile & 63, sg = tile >> 6;
    float f[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[i][2 * j] = __uint_as_float(xv[rep][i][j] << 16);
        f[i][2 * j + 1] = __uint_as_float(xv[rep][i][j] & 0xffff0000u);
      }
    // rows 8sg..8sg+3 and 8sg+4..8sg+7 land at key positions p0 and p0 + 8
    const int p0 = vt_pos(8 * sg), sw = (cg & 7) << 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint16_t* row = tv + (8 * cg + j) * kT;
      *reinterpret_cast<u32x2*>(row + (p0 ^ sw)) = u32x2{pack_f16x2(f[0][j], f[1][j]), pack_f16x2(f[2][j], f[3][j])};
      *reinterpret_cast<u32x2*>(row + ((p0 + 8) ^ sw)) = u32x2{pack_f16x2(f[4][j], f[5][j]), pack_f16x2(f[6][j], f[7][j])};
    }
  }
  __syncthreads();
  uint16_t* vt = base + L.v + size_t(jb) * kDV * kT;
#pragma unroll
  for (int r = 0; r < kDV * kT / 8 / 256; ++r) {
    const int piece = tid + 256 * r;   // 16-byte piece of the block's V^T
    const int c = piece >> 3, pc = piece & 7;
    const u32x4 x = *reinterpret_cast<const u32x4*>(tv + c * kT + ((pc ^ ((c >> 3) & 7)) << 3));
    *reinterpret_cast<u32x4*>(vt + size_t(piece) * 8) = x;
  }
}

// ---- main -------------------------------------------------------------------------------
constexpr int kQ = 128;       // query rows per workgroup
constexpr int kStgLd = 68;    // LDS row stride (floats) of the epilogue's 16 x 64 tiles
constexpr int kWaves = 8;     // 512 threads

struct alignas(16) PShared {
  u32x4 kh[2][kT * kDK / 8];     // two key blocks, half, 16-byte units (swizzled)
  uint16_t p[2][kQ][kPLd];       // scores of two key blocks, half
  float red[kWaves][kQ];         // per-wave row partials for the GroupNorm statistics
  float rs[kQ];                  // signed row sums of the scores
  float mean[kQ], rstd[kQ];      // GroupNorm statistics per row
  float scale[kQ];               // D and R rescaling factor per row
};

// Unit u (16 bytes = 8 halves, u in [0, 32)) of key row s sits at LDS unit
// 32 s + (u ^ (s & 31)): the 16 rows a 16-lane group reads for one fragment then fall
// into 16 different 4-bank groups.
__device__ __forceinline__ int kh_unit(int s, int u) { return 32 * s + (u ^ (s & 31)); }

// FACT: every head of the call has gamma^-127 in float's normal range, so the decay is
// formed from per-lane, per-row and per-block factors; otherwise each score takes its own
// exp2 (decided on the host, so the score loop has no branch on it).
template <int OUT, bool FACT>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
parallel_main(CallArgs a, const uint16_t* q, const uint16_t* ws, const void* gate, void* out) {
  const int N = a.N, nb = (N + kT - 1) / kT, nq = (N + kQ - 1) / kQ;
  const int BH = a.B * a.H;
  // Workgroups are dispatched round-robin over the 8 XCDs (id mod 8). XCD x owns the
  // heads bh = x (mod 8), so their key/value blocks are only ever read through its L2,
  // and walks them heaviest query block first (longest-job-first over that XCD's CUs).
  const int hpx = (BH + 7) / 8;   // heads per XCD
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int bh = 8 * (j % hpx) + xcd;
  const int qb = nq - 1 - j / hpx;
  if (bh >= BH) return;
  const int h = bh % a.H;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Ws L = ws_layout(N);
  const uint16_t* base = ws + size_t(bh) * L.head;
  const int64_t np = int64_t(nb) * kT;
  const __amdgpu_buffer_rsrc_t rq = range_rsrc(q + size_t(bh) * N * kDK, int64_t(N) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rk = range_rsrc(base + L.k, np * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(base + L.v, np * kDV * 2);
  __shared__ PShared sm;

  const float lg = a.hp.log2g[h];
  const int kb_end = min(2 * qb + 1, nb - 1);   // last key block with a causal pair

  // key block kb -> LDS buffer `buf`: each wave copies 4 KB (4 x 64 lanes x 16 B)
  auto stage_k = [&](int kb, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = (w * 4 + j) * 64 + l;             // LDS unit this lane fills
      const int s = p >> 5, u = (p & 31) ^ (s & 31);  // key row and 16-byte unit
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(&sm.kh[buf][(w * 4 + j) * 64]), 16,
          static_cast<uint32_t>(((kb * kT + s) * kDK + 8 * u) * 2), 0, 0, 0);
    }
  };

  // this wave's 16 query rows (B operand of the transposed score product: column t,
  // k = dk), rotated here and scaled by alpha: lane (l16, g) holds row t_row, coordinate
  // pairs 16c + 4g .. +3 of fragment c (rows past N read as zeros)
  const int t_row = qb * kQ + 16 * w + l16;
  f16x8 qf[8];
  {
    u32x4 xq[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
      xq[c] = ld_b128(rq, static_cast<uint32_t>((t_row * kDK + 32 * c + 8 * g) * 2));
    const int64_t p = a.pos0 + t_row;
    const float al = a.alpha;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float cs, sn;
        angle_cs_fast(p, a.ap.theta[16 * c + 4 * g + i], &cs, &sn);
        const float q0 = __uint_as_float(xq[c][i] << 16), q1 = __uint_as_float(xq[c][i] & 0xffff0000u);
        o[i] = pack_f16x2(al * (q0 * cs - q1 * sn), al * (q0 * sn + q1 * cs));
      }
      qf[c] = as_f16x8(o);
    }
  }

  float rsum = 0.f;   // partial signed sum of the scores of row 16w + l16

  // Decay gamma^(t-s) with t = 128qb + 16w + l16 and s = 64kb + 16i + 4g + r, as
  // rl * gr[r] * bi[i]: rl = gamma^(16w + l16 - 4g) per lane (exponent in [-12, 127]),
  // gr[r] = gamma^-r (scalar registers), bi[i] = gamma^(128qb - 64kb - 16i) per wave and
  // key block. The factors stay in float's normal range when gamma^-127 does
  // (gamma > 0.5035, FACT); below that every element takes its own exp2.
  const float rl = exp2f(lg * float(16 * w + l16 - 4 * g));
  float gr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    gr[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(exp2f(-lg * float(r)))));

  // scores of key block kb (in LDS buffer kb % 2) -> sm.p[kb % 2], half. The product is
  // taken transposed (A = Kh rows, B = Qh^T), so lane (l16, g) ends with, for query row
  // 16w + l16, the keys 16i + 4g + r: four consecutive keys per tile i.
  auto scores = [&](int kb) {
    const int buf = kb & 1;
    const int dq = qb * kQ - kb * kT;                 // t - s without the in-block offsets
    const bool diag = kb >= 2 * qb;                   // only these blocks hold s > t
    // two key tiles at a time: two independent accumulation chains, each pair decayed
    // and written to LDS before the next pair starts (fewer live registers)
#pragma unroll
    for (int ip = 0; ip < 2; ++ip) {
      f32x4 z[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f16x8 k0 = as_f16x8(sm.kh[buf][kh_unit(32 * ip + l16, 4 * c + g)]);
        const f16x8 k1 = as_f16x8(sm.kh[buf][kh_unit(32 * ip + 16 + l16, 4 * c + g)]);
        z[0] = mfma(k0, qf[c], z[0]);
        z[1] = mfma(k1, qf[c], z[1]);
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * ip + ii;
        const float bl = rl * exp2f(lg * float(dq - 16 * i));
        float val[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = dq + 16 * w + l16 - 16 * i - 4 * g - r;
          const float f = FACT ? bl * gr[r] : exp2f(lg * float(d));
          val[r] = (diag && d < 0) ? 0.f : z[ii][r] * f;
          rsum += val[r];
        }
        *reinterpret_cast<u32x2*>(&sm.p[buf][16 * w + l16][vt_pos(16 * i + 4 * g)]) =
            u32x2{pack_f16x2(val[0], val[1]), pack_f16x2(val[2], val[3])};
      }
    }
  };

  // output accumulators: all 128 rows (8 t-tiles) x this wave's 64 columns (4 tiles)
  f32x4 acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // V^T fragments of a key block, in two halves of 32 keys (e = 0, 1): this wave's 64
  // columns, B operand (col dv, k = keys in vt_pos order).
  auto load_vh = [&](int kb, int e, f16x8* dst) {
    const uint32_t vblk = static_cast<uint32_t>(kb) * kDV * kT;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int dv = 64 * w + 16 * n + l16;
      dst[n] = as_f16x8(ld_b128(rv, (vblk + static_cast<uint32_t>(dv * kT + 32 * e + 8 * g)) * 2));
    }
  };
  // O[:, this wave's columns] += P(kb)[:, half e] V(kb)[half e]
  auto pv_half = [&](int buf, int e, const f16x8* vf) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f16x8 pf = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.p[buf][16 * m + l16][32 * e + 8 * g]));
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = mfma(pf, vf[n], acc[m][n]);
    }
  };

  // prologue: key block 0 -> scores 0; key block 1 staged; first half of V(0) loaded
  stage_k(0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();
  if (kb_end >= 1) stage_k(1, 1);
  scores(0);
  f16x8 vh0[4], vh1[4];
  load_vh(0, 0, vh0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();

  // Per key block: the first half of V(kb) was loaded during the previous block; the
  // second half is loaded at the top and used last, and the first half of V(kb+1) is
  // loaded between the two halves of the product, so each V load has a half or a whole
  // block of work in front of it. That load is issued on every pass, also after the last
  // key block (block nb lies just past the end of V's range: the lanes read zeros):
  // issued under a condition, the compiler's waits before the second half of the product
  // would have to cover it too, exposing its latency.
  for (int kb = 0; kb <= kb_end; ++kb) {
    // scores(kb) are in sm.p[kb%2]; key block kb+1 is in sm.kh[(kb+1)%2]
    if (kb + 2 <= kb_end) stage_k(kb + 2, kb & 1);
    load_vh(kb, 1, vh1);
    if (kb + 1 <= kb_end) scores(kb + 1);
    const int buf = kb & 1;
    pv_half(buf, 0, vh0);
    load_vh(kb + 1, 0, vh0);
    pv_half(buf, 1, vh1);
    // key block kb+2 staged (and V's second half, used above); V(kb+1)'s first half
    // stays in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0));
    __syncthreads();
  }

  // ---- row scalars ------------------------------------------------------------------
  {
    float x = rsum;
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    if (g == 0) sm.rs[16 * w + l16] = x;
  }
  __syncthreads();
  const bool any_norm = a.flags & (RN_NORM_D_ROW | RN_NORM_R_ROW);
  if (any_norm) {
    // One factor per row, computed once (in float64) by the first 128 threads:
    // c_t = 1/sqrt(sum_{m<=t} gamma^m) (D rescaling), then 1/max(c_t |rowsum|, 1) (R).
    if (tid < kQ) {
      const int t = qb * kQ + tid;
      double ct = 1.0;
      if (a.flags & RN_NORM_D_ROW) {
        const double gm = a.hp.gamma[h];
        const double G = (gm == 1.0) ? double(t + 1) : -expm1(double(t + 1) * log(gm)) / (1.0 - gm);
        ct = 1.0 / sqrt(G);
      }
      double sc = ct;
      if (a.flags & RN_NORM_R_ROW) sc = ct / fmax(fabs(ct * double(sm.rs[tid])), 1.0);
      sm.scale[tid] = static_cast<float>(sc);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = sm.scale[16 * m + 4 * g + r];
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n][r] *= f;
      }
  }

  // ---- GroupNorm over the 512 columns of each row (8 waves x 64) ---------------------
  const bool gn = a.flags & RN_EPI_GN;
  const bool gt = a.flags & RN_EPI_GATE;
  auto row_partial = [&](auto f) {   // sum over this wave's 64 columns of f(value, m, r)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) x += f(acc[m][n][r], m, r);
        x = row16_sum(x);
        if (l16 == 0) sm.red[w][16 * m + 4 * g + r] = x;
      }
  };
  if (gn) {
    row_partial([](float v, int, int) { return v; });
    __syncthreads();
    if (tid < kQ) {
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) x += sm.red[ww][tid];
      sm.mean[tid] = x * (1.0f / kDV);
    }
    __syncthreads();
    row_partial([&](float v, int m, int r) {
      const float d = v - sm.mean[16 * m + 4 * g + r];
      return d * d;
    });
    __syncthreads();
    if (tid < kQ) {
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) x += sm.red[ww][tid];
      sm.rstd[tid] = 1.0f / sqrtf(x * (1.0f / kDV) + a.eps);
    }
    __syncthreads();
  }

  // ---- epilogue: one 16-row tile at a time through this wave's LDS area, so that each
  // lane ends with 16 consecutive columns of one row: normalise, gate, and store them as
  // 16-byte runs. The key buffers are free by now (the loop's last barrier has passed).
  float* stg = reinterpret_cast<float*>(&sm.kh[0][0]) + w * (16 * kStgLd);
  const int er = l >> 2, ec = 16 * (l & 3);          // row in the tile, first column
  const int col0 = 64 * w + ec;                      // first column of the lane's run
  float gw[16], gb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    gw[j] = (gn && a.gn_w) ? a.gn_w[h * kDV + col0 + j] : 1.f;
    gb[j] = (gn && a.gn_b) ? a.gn_b[h * kDV + col0 + j] : 0.f;
  }
  constexpr int kEsz = OUT == RN_BF16 ? 2 : 4;      // output element bytes
  const __amdgpu_buffer_rsrc_t rg =
      range_rsrc(gt ? static_cast<const uint16_t*>(gate) + size_t(bh) * N * kDV : nullptr,
                 gt ? int64_t(N) * kDV * 2 : 0);
  const __amdgpu_buffer_rsrc_t ro =
      range_rsrc(static_cast<uint8_t*>(out) + size_t(bh) * N * kDV * kEsz, int64_t(N) * kDV * kEsz);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) stg[(4 * g + r) * kStgLd + 16 * n + l16] = acc[m][n][r];
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    float y[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(&stg[er * kStgLd + ec + 4 * i]);
#pragma unroll
      for (int c = 0; c < 4; ++c) y[4 * i + c] = x4[c];
    }
    const int tl = 16 * m + er, t = qb * kQ + tl;
    // byte offsets within the head; rows past N go to an offset past the buffer's range,
    // where loads return zero and stores are dropped
    const uint32_t ooff = t < N ? static_cast<uint32_t>((t * kDV + col0) * kEsz) : 0x80000000u;
    const uint32_t goff = t < N ? static_cast<uint32_t>((t * kDV + col0) * 2) : 0x80000000u;
    if (gn) {
      const float mu = sm.mean[tl], rs = sm.rstd[tl];
#pragma unroll
      for (int j = 0; j < 16; ++j) y[j] = (y[j] - mu) * rs * gw[j] + gb[j];
      if (gt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const u32x4 gv = ld_b128(rg, goff + 16 * i);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            y[8 * i + 2 * c] *= swishf(__uint_as_float(gv[c] << 16));
            y[8 * i + 2 * c + 1] *= swishf(__uint_as_float(gv[c] & 0xffff0000u));
          }
        }
      }
    }
    if (OUT == RN_BF16) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        u32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = pack_bf16x2(y[8 * i + 2 * c], y[8 * i + 2 * c + 1]);
        st_b128(ro, ooff + 16 * i, v);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = __float_as_uint(y[4 * i + c]);
        st_b128(ro, ooff + 16 * i, v);
      }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // tile read back before it is rewritten
  }
}

}  // namespace

// Buffer offsets within one head's rows are 32-bit: N d_v elements of up to 4 bytes (a
// float32 output) must stay below 2^31 bytes.
bool parallel_mfma_supported(const CallArgs& a, int in_dt) {
  return in_dt == RN_BF16 && a.dk == kDK && a.dv == kDV && int64_t(a.N) * kDV * 4 < (int64_t(1) << 31);
}

size_t parallel_mfma_ws_bytes(const CallArgs& a) {
  return size_t(a.B) * a.H * ws_layout(a.N).head * sizeof(uint16_t);
}

hipError_t launch_parallel_mfma(const CallArgs& a, int out_dt, const void* q, const void* k,
                                const void* v, const void* gate, void* out, void* ws,
                                hipStream_t st) {
  const int nb = (a.N + kT - 1) / kT;
  const int BH = a.B * a.H;
  uint16_t* w = static_cast<uint16_t*>(ws);
  hipLaunchKernelGGL(parallel_prep, dim3(nb, BH), dim3(256), 0, st, a,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), w);
  const uint16_t* qh = static_cast<const uint16_t*>(q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nq = (a.N + kQ - 1) / kQ;
  const dim3 grid(static_cast<unsigned>(nq) * 8 * ((BH + 7) / 8));
  bool fact = true;
  for (int h = 0; h < a.H; ++h) fact = fact && a.hp.log2g[h] * 127.f >= -126.f;
  const dim3 blk(kWaves * 64);
  if (out_dt == RN_BF16) {
    if (fact) hipLaunchKernelGGL((parallel_main<RN_BF16, true>), grid, blk, 0, st, a, qh, w, gate, out);
    else hipLaunchKernelGGL((parallel_main<RN_BF16, false>), grid, blk, 0, st, a, qh, w, gate, out);
  } else {
    if (fact) hipLaunchKernelGGL((parallel_main<RN_F32, true>), grid, blk, 0, st, a, qh, w, gate, out);
    else hipLaunchKernelGGL((parallel_main<RN_F32, false>), grid, blk, 0, st, a, qh, w, gate, out);
  }
  return hipGetLastError();
}

}  // namespace rn
