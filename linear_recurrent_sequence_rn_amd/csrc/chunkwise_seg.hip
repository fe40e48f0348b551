// Segmented chunk-parallel schedule of the chunkwise form for bf16 q/k/v, d_k = 256,
// d_v = 512, one decay per head (hwhale notes: chunkwise equation and ChunkwiseRetention
// listing; m0nads notes, "Chunkwise representation"; GroupNorm + swish gate of the
// multi-scale layer).
//
// Unrolling the recurrent update S_t = gamma S_{t-1} + Kh_t^T V_t from a point s gives
// S_t = gamma^(t-s) S_s + (the same update started from zero at s). So the state at a
// chunk start c0 inside a segment that starts at s_g is
//     S_{c0} = L_{c0} + gamma^(c0 - s_g) T_g,
// with L the segment-local state (zero at s_g) and T_g the true state at s_g, and the
// segment-start states chain as T_{g+1} = gamma^(len_g) T_g + E_g, E_g being the local
// state at segment g's end. Three kernels per window of 32 chunks (8192 tokens) and group
// of up to 64 heads:
//   seg_states   one 8-wave workgroup per (head, 2048-token segment, 128 state rows) walks
//                its segment in 32-token steps from a zero state, each wave holding a
//                128 x 64 float32 tile in MFMA accumulators; K is rotated once per step for
//                all waves into LDS, V is transposed in registers. It writes L at every
//                chunk start inside the segment (half) and E at the segment's end (float32).
//   seg_scan     per state element: T_g for every segment (half) and the float32 state
//                leaving the window.
//   seg_outputs  one 512-thread workgroup per (head, chunk, 64 query rows):
//                O_t = alpha gamma^(t-c0+1) Qh_t (gamma^(c0-s_g) T_g + L_{c0})
//                      + sum_{c0 <= s <= t} alpha gamma^(t-s) (Qh_t . Kh_s) V_s,
//                then GroupNorm + gate and the store.
// Products are 16x16x32 f16 MFMA with float32 accumulation; operands are rounded to
// IEEE half after the float32 rotation and decay (half keeps 3 more bits than bf16), and
// must stay within half's range, as must the states. The decay enters only as factors
// at most 1 (operands) or in float32 (scores, row scales), so any gamma in (0, 1] works.
//
// MFMA lane layouts (16x16x32, lane = 16 g + l): A holds row l, k 8g..8g+7; B holds
// column l, k 8g..8g+7; D holds column l, rows 4g..4g+3. Where a lane loads 8 tokens of
// 4 consecutive features and transposes them in registers, the tile's row (or column)
// l stands for feature 4l + j of fragment j, which only permutes rows and columns of the
// results.
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
constexpr int kC = 256;                        // tokens per chunk (snapshot spacing)
constexpr int kWin = 32;                       // chunks per window
constexpr int kSegChunks = 8;                  // chunks per segment
constexpr int kSeg = kSegChunks * kC;          // 2048 tokens
constexpr int kSegMax = kWin / kSegChunks;     // segments per window
constexpr int kHeadsPerGroup = 64;             // heads per launch triple
constexpr size_t kSnap = size_t(kDK) * kDV;    // elements of one state
constexpr int kLdQ = 264;                      // LDS pitch (half) of the row buffers
constexpr uint32_t kSink = 0x80000000u;        // store offset past every range: dropped

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
// the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes > 0 ? bytes : 0), 0x00020000);
}
__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Buffer accesses at a per-lane offset plus a uniform one (the uniform part goes to the
// instruction's scalar offset, so a loop needs no per-access address registers).
__device__ __forceinline__ uint32_t ld_b32s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ u32x2 ld_b64s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ u32x4 ld_b128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ void st_b128s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, voff, soff, 0);
}
// An opaque copy: the compiler cannot precompute what depends on the result outside the
// loop iteration that produces it (which would keep one register per unrolled step).
__device__ __forceinline__ int opaque(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void st_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, 0);
}
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}

// cos and sin of the angle p * theta: the angle in revolutions is formed and reduced to
// [0, 1) in float64, then the hardware sine and cosine (which take revolutions) apply.
__device__ __forceinline__ void angle_rev(int64_t p, float theta, float* c, float* s) {
  const double r = static_cast<double>(p) * (static_cast<double>(theta) * 0.15915494309189535);
  const float f = static_cast<float>(r - floor(r));
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

// Blocks are dispatched round-robin over the 8 XCDs; this gives each XCD a contiguous
// range of work items (grid size a multiple of 8), so that items sharing data (the
// column blocks of one segment, the row tiles of one chunk) share an L2.
__device__ __forceinline__ int xcd_item(int bid, int nblocks) {
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

struct SegArgs {
  CallArgs a;
  int head0, heads;        // heads [head0, head0 + heads) of the B*H
  int win, nseg;           // window index; segments in this window
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  uint16_t* snap;          // [heads][kWin][kDV][kDK] half: L at chunk starts (S^T)
  float* ends;             // [heads][kSegMax][kDV][kDK] float: E per segment (S^T)
  uint16_t* starts;        // [heads][kSegMax][kDV][kDK] half: T per segment (S^T)
  const float* src;        // state entering the window, [kDK][kDV] per head, or null
  int src_group;           // 1: indexed by head within the group, 0: by global head
  float* dst;              // state leaving the window, or null
  int dst_group;
  void* out;
  uint32_t* status;        // the call's status word (bit 1: a non-finite output or final state)
};

// =================================== seg_states =========================================
// Workgroup (head, segment, feature half qd): rows [128 qd, 128 qd + 128) of the state,
// eight waves, wave cb owning columns [64 cb, 64 cb + 64). The segment is walked in
// 32-token steps, one chunk (eight steps) per loop iteration:
//   K: thread (pair p, tokens 4 tg .. 4 tg + 3 of the step) loads one rotation pair of
//      four tokens, rotates it, multiplies by gamma^(Lc-1-tau) (tau = token within its
//      chunk of Lc tokens) and writes it, in half, transposed into LDS (feature rows,
//      token columns), so every pair is rotated once for all eight waves;
//   V: lane (l, g) of wave cb loads tokens 8g .. 8g+7 of the step at columns
//      64 cb + 4l .. +3 and transposes them in registers into the B fragments.
// LDS row of feature f is 16 (f & 7) + (f >> 3), so A fragment j holds features 8l + j,
// and acc[j][jj] holds S[128 qd + 32 g + 8 r + j][64 cb + 4 l + jj] in its element r.
// The state is scaled by gamma^Lc at each chunk start. K is loaded two steps ahead of its
// use (one before it is staged) and V one, through register pairs; scheduling barriers
// keep the loads where they are issued.
constexpr int kRingK = 2;
constexpr int kRingV = 2;
constexpr int kLdT = 40;   // LDS pitch (half) of the transposed K step

__global__ void __launch_bounds__(512) seg_states(SegArgs P) {
  const CallArgs& a = P.a;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int qd = item & 1;
  const int sg = (item >> 1) % P.nseg;
  const int hl = (item >> 1) / P.nseg;
  if (hl >= P.heads) return;
  const int gh = P.head0 + hl, h = gh % a.H, seq = gh / a.H;
  const int len = seq_len(a, seq);
  const int64_t p0 = seq_pos0(a, seq);
  const int w0 = P.win * kWin * kC;
  const int s0 = w0 + sg * kSeg;
  const int s1 = static_cast<int>(uniform(static_cast<uint32_t>(min(min(s0 + kSeg, w0 + kWin * kC), len))));
  const int nch = s1 > s0 ? (s1 - s0 + kC - 1) / kC : 0;   // chunks of the segment
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int cb = static_cast<int>(uniform(static_cast<uint32_t>(tid >> 6)));   // the wave
  const float lg = a.hp.log2g[h];
  const int vc0 = 64 * cb + 4 * l16;    // the lane's four state columns
  // K staging role
  const int kp = tid & 63, ktg = cb;
  const float th = a.ap.theta[64 * qd + kp];
  float cs1, sn1;
  angle_rev(1, th, &cs1, &sn1);
  const int f0 = 2 * kp;                                  // features f0, f0 + 1 of the half
  const int row0 = 16 * (f0 & 7) + (f0 >> 3), row1 = 16 * ((f0 + 1) & 7) + (f0 >> 3);

  __shared__ uint16_t kt[2][128][kLdT];

  const __amdgpu_buffer_rsrc_t rk = range_rsrc(P.k + size_t(gh) * a.N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(P.v + size_t(gh) * a.N * kDV, int64_t(len) * kDV * 2);
  const __amdgpu_buffer_rsrc_t rs =
      range_rsrc(P.snap + size_t(hl) * kWin * kSnap, int64_t(kWin) * kSnap * 2);

  f32x4 acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[j][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t kx[kRingK][4];
  u32x2 vx[kRingV][8];
  // K: row s0 + 32u + 4 ktg + i (ktg is the wave index: uniform), pair column per lane
  const uint32_t kvoff = (128 * qd + f0) * 2;
  const uint32_t ksoff0 = uniform(static_cast<uint32_t>((s0 + 4 * ktg) * kDK * 2));
  auto load_k = [&](int u, uint32_t (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ld_b32s(rk, kvoff, ksoff0 + (32 * u + i) * kDK * 2);
  };
  // V: row s0 + 32u + 8g + e, columns vc0 .. +3
  const uint32_t vvoff = static_cast<uint32_t>((8 * g4 * kDV + vc0) * 2);
  const uint32_t vsoff0 = static_cast<uint32_t>(s0 * kDV * 2);
  auto load_v = [&](int u, u32x2 (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = ld_b64s(rv, vvoff, vsoff0 + (32 * u + e) * kDV * 2);
  };
  // rotated, decayed K of step u into LDS buffer u & 1 (chunk of Lc tokens from cstart).
  // The angle of the thread's first token, in revolutions, is carried from step to step:
  // reduced to [0, 1) in float64 once, then advanced by 32 positions (also reduced in
  // float64) and wrapped to [0, 1) at each step, so its error stays near 1e-6 revolutions.
  float ang;
  float rstep;
  {
    const double rt = static_cast<double>(th) * 0.15915494309189535;
    const double r0 = static_cast<double>(p0 + s0 + 4 * ktg) * rt;
    const double r32 = 32.0 * rt;
    ang = static_cast<float>(r0 - floor(r0));
    rstep = static_cast<float>(r32 - floor(r32));
  }
  auto stage_k = [&](int u, const uint32_t (&x)[4]) {
    const int cstart = s0 + kC * (u >> 3);
    const int Lc = max(min(kC, s1 - cstart), 0);
    const int tau0 = opaque(4 * ktg) + 32 * (u & 7);   // token of i = 0 within its chunk
    float sv = __builtin_amdgcn_sinf(ang), c = __builtin_amdgcn_cosf(ang);
    ang += rstep;
    ang -= floorf(ang);
    const float ez0 = float(Lc - 1 - tau0);
    uint32_t o0[2], o1[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float z = tau0 + i < Lc ? exp2f(lg * (ez0 - float(i))) : 0.f;
      const float x0 = bf_lo(x[i]), x1 = bf_hi(x[i]);
      const float y0 = (x0 * c - x1 * sv) * z, y1 = (x0 * sv + x1 * c) * z;
      const uint32_t h0 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(y0));
      const uint32_t h1 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(y1));
      if (i & 1) {
        o0[i >> 1] |= h0 << 16;
        o1[i >> 1] |= h1 << 16;
      } else {
        o0[i >> 1] = h0;
        o1[i >> 1] = h1;
      }
      const float cn = c * cs1 - sv * sn1;
      sv = c * sn1 + sv * cs1;
      c = cn;
    }
    *reinterpret_cast<u32x2*>(&kt[u & 1][row0][4 * ktg]) = u32x2{o0[0], o0[1]};
    *reinterpret_cast<u32x2*>(&kt[u & 1][row1][4 * ktg]) = u32x2{o1[0], o1[1]};
  };
  auto mma_step = [&](int u, const u32x2 (&x)[8]) {
    if ((u & 7) == 0) {
      const int Lc = max(min(kC, s1 - (s0 + kC * (u >> 3))), 0);
      const float gl = exp2f(lg * float(Lc));
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[j][jj] *= gl;
    }
    uint32_t bp[4][4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const u32x2 va = x[2 * e2], vb = x[2 * e2 + 1];
      bp[0][e2] = pack_f16x2(bf_lo(va[0]), bf_lo(vb[0]));
      bp[1][e2] = pack_f16x2(bf_hi(va[0]), bf_hi(vb[0]));
      bp[2][e2] = pack_f16x2(bf_lo(va[1]), bf_lo(vb[1]));
      bp[3][e2] = pack_f16x2(bf_hi(va[1]), bf_hi(vb[1]));
    }
    f16x8 B[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) B[jj] = as_f16x8(u32x4{bp[jj][0], bp[jj][1], bp[jj][2], bp[jj][3]});
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f16x8 A = as_f16x8(*reinterpret_cast<const u32x4*>(&kt[u & 1][16 * j + l16][8 * g4]));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[j][jj] = mfma(A, B[jj], acc[j][jj]);
    }
  };
  // L at the start of chunk ci + 1 when that chunk starts inside the segment
  auto store_snap = [&](int ci) {
    const int next = s0 + kC * (ci + 1);
    // the lane's offset is recomputed here rather than held across the loop
    const int ln = opaque(lane);
    const uint32_t svoff = static_cast<uint32_t>(((64 * cb + 4 * (ln & 15)) * kDK + 128 * qd + 32 * (ln >> 4)) * 2);
    const uint32_t voff = next < s1 ? svoff : kSink;
    const uint32_t soff = uniform(static_cast<uint32_t>((next - w0) / kC) * kDV * kDK * 2);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st_b128s(rs, voff + (jj * kDK + 8 * r) * 2, soff,
                 u32x4{pack_f16x2(acc[0][jj][r], acc[1][jj][r]), pack_f16x2(acc[2][jj][r], acc[3][jj][r]),
                       pack_f16x2(acc[4][jj][r], acc[5][jj][r]), pack_f16x2(acc[6][jj][r], acc[7][jj][r])});
  };

  // prologue: K of steps 0, 1 and V of step 0 in flight; step 0's K staged
  load_k(0, kx[0]);
  load_k(1, kx[1]);
  load_v(0, vx[0]);
  stage_k(0, kx[0]);
  __syncthreads();
  for (int ci = 0; ci < nch; ++ci) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = 8 * ci + i;
      __builtin_amdgcn_sched_barrier(0);
      load_v(u + 1, vx[(i + 1) % kRingV]);
      __builtin_amdgcn_sched_barrier(0);
      stage_k(u + 1, kx[(i + 1) % kRingK]);
      __builtin_amdgcn_sched_barrier(0);
      load_k(u + 2, kx[i % kRingK]);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(u, vx[i % kRingV]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    }
    store_snap(ci);
  }
  // E: the local state at the segment's end
  float* e = P.ends + (size_t(hl) * kSegMax + sg) * kSnap;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t off = size_t(vc0 + jj) * kDK + 128 * qd + 32 * g4 + 8 * r;
      *reinterpret_cast<f32x4*>(e + off) = f32x4{acc[0][jj][r], acc[1][jj][r], acc[2][jj][r], acc[3][jj][r]};
      *reinterpret_cast<f32x4*>(e + off + 4) = f32x4{acc[4][jj][r], acc[5][jj][r], acc[6][jj][r], acc[7][jj][r]};
    }
}

// ==================================== seg_scan ==========================================
// Thread (head, column n, features 8 cb .. 8 cb + 7): T_0 = state entering the window,
// T_{g+1} = gamma^(len_g) T_g + E_g, each T_g stored in half for the outputs, the last
// one in float32 as the state leaving the window.
__global__ void __launch_bounds__(256) seg_scan(SegArgs P) {
  const CallArgs& a = P.a;
  const int gt = blockIdx.x * 256 + threadIdx.x;
  const int cb = gt & 31, n = (gt >> 5) & (kDV - 1), hl = gt >> 14;
  if (hl >= P.heads) return;
  const int gh = P.head0 + hl, h = gh % a.H, seq = gh / a.H;
  const int len = seq_len(a, seq);
  const float lg = a.hp.log2g[h];
  const int w0 = P.win * kWin * kC;
  const size_t col = size_t(n) * kDK + 8 * cb;

  float S[8];
  if (P.src) {
    const float* src = P.src + size_t(P.src_group ? hl : gh) * kSnap;
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = src[size_t(8 * cb + i) * kDV + n];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = 0.f;
  }
  for (int g = 0; g < P.nseg; ++g) {
    const size_t slot = (size_t(hl) * kSegMax + g) * kSnap + col;
    const f32x4 e0 = *reinterpret_cast<const f32x4*>(P.ends + slot);
    const f32x4 e1 = *reinterpret_cast<const f32x4*>(P.ends + slot + 4);
    *reinterpret_cast<u32x4*>(P.starts + slot) =
        u32x4{pack_f16x2(S[0], S[1]), pack_f16x2(S[2], S[3]), pack_f16x2(S[4], S[5]), pack_f16x2(S[6], S[7])};
    const int s0 = w0 + g * kSeg;
    const int s1 = min(min(s0 + kSeg, w0 + kWin * kC), len);
    const float f = exp2f(lg * float(max(s1 - s0, 0)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S[i] = fmaf(f, S[i], e0[i]);
      S[4 + i] = fmaf(f, S[4 + i], e1[i]);
    }
  }
  if (P.dst) {
    float* dst = P.dst + size_t(P.dst_group ? hl : gh) * kSnap;
    uint32_t bad = 0u;   // set by a non-finite value of the caller's final state
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dst[size_t(8 * cb + i) * kDV + n] = S[i];
      bad |= __builtin_isfinite(S[i]) ? 0u : 1u;
    }
    if (!P.dst_group && __builtin_amdgcn_ballot_w64(bad != 0u) != 0 && (threadIdx.x & 63) == 0)
      __hip_atomic_fetch_or(P.status, kChunkwiseStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// =================================== seg_outputs ========================================
// Workgroup (head, chunk, row tile rt): rows t0 = c0 + 64 rt .. +63. Wave w owns output
// columns 64 w .. 64 w + 63; lane (l, g) holds acc[i][j][r] = O[16 i + 4 g + r][64 w + 4 l + j].
//   cross: acc = Qh T_g (A = Qh rows from LDS, B = T^T rows from the workspace),
//          acc *= gamma^(c0 - s_g), acc += Qh L_{c0}, then each row times
//          alpha gamma^(t - c0 + 1).
//   intra, key tiles kt = 0 .. rt of the chunk: scores P^T = Kh Qh^T in four 16 x 16
//          tiles per wave (rows 16 (w >> 1) .., keys 32 (w & 1) ..), scaled by
//          alpha gamma^(t - s) and masked to s <= t, into LDS as the A fragments of P V;
//          V comes straight from memory (8 tokens x 4 columns per lane, transposed in
//          registers) as the B fragments.
// Key slot order inside a 32-key half: lane group g holds keys 4g .. 4g+3 and
// 16 + 4g .. 16 + 4g + 3 (the rows of its score tiles), for P and V alike.
struct alignas(16) SharedS {
  uint16_t qs[64][kLdQ];       // Qh of the workgroup's rows (unscaled)
  uint16_t ks[2][64][kLdQ];    // Kh of a key tile (double buffer)
  u32x4 ps[2][4][2][64];       // P fragments: [buffer][row strip][key half][lane]
  float red[2][64][8];         // GroupNorm partial sums: [pass][row][wave]
};

template <int OUT>
__global__ void __launch_bounds__(512) seg_outputs(SegArgs P) {
  const CallArgs& a = P.a;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int rt = item & 3;
  const int cw = (item >> 2) % kWin;
  const int hl = (item >> 2) / kWin;
  if (hl >= P.heads) return;
  const int gh = P.head0 + hl, h = gh % a.H, seq = gh / a.H;
  const int N = a.N;
  const int len = static_cast<int>(uniform(static_cast<uint32_t>(seq_len(a, seq))));
  const int64_t p0 = seq_pos0(a, seq);
  const int w0 = P.win * kWin * kC;
  const int c0 = w0 + cw * kC;
  const int t0 = c0 + 64 * rt;
  if (t0 >= len) return;
  const int sg = cw / kSegChunks;
  const int sgs = w0 + sg * kSeg;                  // segment start
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int w = static_cast<int>(uniform(static_cast<uint32_t>(tid >> 6)));   // the wave
  const float lg = a.hp.log2g[h];
  const bool use_gn = a.flags & RN_EPI_GN;
  const bool has_gate = P.gate != nullptr;

  __shared__ SharedS sm;

  const __amdgpu_buffer_rsrc_t rq = range_rsrc(P.q + size_t(gh) * N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rk = range_rsrc(P.k + size_t(gh) * N * kDK, int64_t(len) * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = range_rsrc(P.v + size_t(gh) * N * kDV, int64_t(len) * kDV * 2);
  const __amdgpu_buffer_rsrc_t rgt =
      range_rsrc((has_gate ? P.gate : P.v) + size_t(gh) * N * kDV, int64_t(len) * kDV * 2);
  // T_g is zero for the first segment of the first window without an entering state, L
  // is zero at a segment's first chunk: empty ranges read as zeros
  const bool t_zero = sg == 0 && P.src == nullptr;
  const bool l_zero = c0 == sgs;
  const __amdgpu_buffer_rsrc_t rT = range_rsrc(
      P.starts + (size_t(hl) * kSegMax + sg) * kSnap, t_zero ? 0 : int64_t(kSnap) * 2);
  const __amdgpu_buffer_rsrc_t rL = range_rsrc(
      P.snap + (size_t(hl) * kWin + cw) * kSnap, l_zero ? 0 : int64_t(kSnap) * 2);
  const int osz = OUT == RN_BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t ro = range_rsrc(
      static_cast<uint8_t*>(P.out) + size_t(gh) * N * kDV * osz, int64_t(len) * kDV * osz);

  // ---- row staging: thread (rows 4 rg .. 4 rg + 3, features 8 cq .. 8 cq + 7) ----------
  const int cq = tid & 31, rg = tid >> 5;
  const uint32_t rvoff = static_cast<uint32_t>((4 * rg * kDK + 8 * cq) * 2);
  auto load_rows = [&](__amdgpu_buffer_rsrc_t r, int row0, u32x4 (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ld_b128s(r, rvoff, static_cast<uint32_t>((row0 + i) * kDK * 2));
  };
  auto stage_rows = [&](int row0, const u32x4 (&x)[4], uint16_t (*buf)[kLdQ]) {
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const float th = a.ap.theta[4 * cq + pp];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float c, s;
        angle_rev(p0 + row0 + 4 * rg + i, th, &c, &s);
        const uint32_t word = x[i][pp];
        const float x0 = bf_lo(word), x1 = bf_hi(word);
        *reinterpret_cast<uint32_t*>(&buf[4 * rg + i][8 * cq + 2 * pp]) =
            pack_f16x2(x0 * c - x1 * s, x0 * s + x1 * c);
      }
    }
  };
  // V of key tile kt for this wave: [key half][slot e] (8 bytes: 4 columns)
  const int vcol = 64 * w + 4 * l16;
  // rows 4g + (uniform row) at the lane's four columns: V, gate and output rows
  const uint32_t gvoff = static_cast<uint32_t>((4 * g4 * kDV + vcol) * 2);
  auto load_v = [&](int kt, u32x2 (&vx)[2][8]) {
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = c0 + 64 * kt + 32 * hk + (e < 4 ? e : 12 + e);
        vx[hk][e] = ld_b64s(rv, gvoff, static_cast<uint32_t>(key * kDV * 2));
      }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue ---------------------------------------------------------------------------
  u32x4 xr[4];        // raw Q rows, then raw K rows of the next key tile
  u32x2 vb[2][2][8];   // V of a key tile: [ring][key half][slot]
  {
    u32x4 kr0[4];
    load_rows(rq, t0, xr);
    load_rows(rk, c0, kr0);
    stage_rows(t0, xr, sm.qs);
    stage_rows(c0, kr0, sm.ks[0]);
  }
  load_v(0, vb[0]);
  load_rows(rk, c0 + 64, xr);

  // ---- cross term: 16 steps (T pass, then L pass) of 32 features -------------------------
  // B fragments run four steps ahead through a ring of five register sets; scheduling
  // barriers keep each step's loads where they are issued (hoisting them all would spill).
  {
    constexpr int kAheadX = 4, kRingX = kAheadX + 1;
    u32x4 bq[kRingX][4];
    const uint32_t bvoff = static_cast<uint32_t>((vcol * kDK + 8 * g4) * 2);
    auto load_b = [&](int st, u32x4 (&b)[4]) {
      const __amdgpu_buffer_rsrc_t r = st < 8 ? rT : rL;
      const int kk = st & 7;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = ld_b128s(r, bvoff + (j * kDK + 32 * kk) * 2, 0);
    };
#pragma unroll
    for (int st = 0; st < kAheadX; ++st) load_b(st, bq[st]);
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + kAheadX < 16) load_b(st + kAheadX, bq[(st + kAheadX) % kRingX]);
      const int kk = st & 7;
      f16x8 A[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        A[i] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.qs[16 * i + l16][32 * kk + 8 * g4]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(A[i], as_f16x8(bq[st % kRingX][j]), acc[i][j]);
      if (st == 7) {
        const float f = exp2f(lg * float(c0 - sgs));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] *= f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float xi = a.alpha * exp2f(lg * float(t0 + 16 * i + 4 * g4 + r - c0 + 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j][r] *= xi;
      }
  }

  // ---- intra-chunk part -------------------------------------------------------------------
  // One barrier per key tile: Kh of tile kt + 1 is staged into the other buffer and P of
  // tile kt into its own buffer before it; both were last read before the previous one.
  // Tiles go in pairs with no branch inside (a branch between a load and its use makes
  // the compiler wait for every load in flight): row tiles 0 and 2 run one more tile,
  // whose keys all lie past the rows, so the causal mask zeroes it.
  const int si = w >> 1, hk = w & 1;          // score strip and key half of this wave
  auto key_tile = [&](int kt, const u32x2 (&vc)[2][8], u32x2 (&vn)[2][8]) {
    __builtin_amdgcn_sched_barrier(0);
    load_v(kt + 1, vn);
    __builtin_amdgcn_sched_barrier(0);
    // scores of key tile kt
    {
      const uint16_t (*kb)[kLdQ] = sm.ks[kt & 1];
      f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const f16x8 B = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.qs[16 * si + l16][32 * kk + 8 * g4]));
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f16x8 A = as_f16x8(*reinterpret_cast<const u32x4*>(&kb[32 * hk + 16 * u + l16][32 * kk + 8 * g4]));
          sc[u] = mfma(A, B, sc[u]);
        }
      }
      const int t = t0 + 16 * si + l16;
      float pv[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = c0 + 64 * kt + 32 * hk + 16 * u + 4 * g4 + r;
          pv[u][r] = s <= t ? a.alpha * exp2f(lg * float(t - s)) * sc[u][r] : 0.f;
        }
      sm.ps[kt & 1][si][hk][lane] =
          u32x4{pack_f16x2(pv[0][0], pv[0][1]), pack_f16x2(pv[0][2], pv[0][3]),
                pack_f16x2(pv[1][0], pv[1][1]), pack_f16x2(pv[1][2], pv[1][3])};
    }
    // Kh of the next key tile into the other buffer; raw rows of the one after
    stage_rows(c0 + 64 * (kt + 1), xr, sm.ks[(kt + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    load_rows(rk, c0 + 64 * (kt + 2), xr);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // P V of key tile kt
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f16x8 B[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t bw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t x0 = vc[h2][2 * e2][j >> 1], x1 = vc[h2][2 * e2 + 1][j >> 1];
          bw[e2] = (j & 1) ? pack_f16x2(bf_hi(x0), bf_hi(x1)) : pack_f16x2(bf_lo(x0), bf_lo(x1));
        }
        B[j] = as_f16x8(u32x4{bw[0], bw[1], bw[2], bw[3]});
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x8 A = as_f16x8(sm.ps[kt & 1][i][h2][lane]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(A, B[j], acc[i][j]);
      }
    }
  };
  for (int kt = 0; kt <= rt; kt += 2) {
    key_tile(kt, vb[0], vb[1]);
    key_tile(kt + 1, vb[1], vb[0]);
  }

  // ---- epilogue: GroupNorm over the 512 columns of each row, gate, store -----------------
  u32x2 gt[4][4];
  if (has_gate) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        gt[i][r] = ld_b64s(rgt, gvoff, static_cast<uint32_t>((t0 + 16 * i + r) * kDV * 2));
  }
  if (use_gn) {
    float mean[4][4], rstd[4][4];
    // row sums over the lane's 4 columns, then over the 16 lanes of its group
    auto row_reduce = [&](int pass, float (&part)[4][4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = part[i][r];
          s += __shfl_xor(s, 1, 64);
          s += __shfl_xor(s, 2, 64);
          s += __shfl_xor(s, 4, 64);
          s += __shfl_xor(s, 8, 64);
          part[i][r] = s;
        }
      // lane l of group g writes row 16 (l >> 2) + 4 g + (l & 3)
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (l16 == 4 * i + r) mine = part[i][r];
      sm.red[pass][16 * (l16 >> 2) + 4 * g4 + (l16 & 3)][w] = mine;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* p = sm.red[pass][16 * i + 4 * g4 + r];
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(p);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(p + 4);
          part[i][r] = ((u0[0] + u0[1]) + (u0[2] + u0[3])) + ((u1[0] + u1[1]) + (u1[2] + u1[3]));
        }
    };
    float part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[i][r] = (acc[i][0][r] + acc[i][1][r]) + (acc[i][2][r] + acc[i][3][r]);
    row_reduce(0, part);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mean[i][r] = part[i][r] * (1.f / kDV);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = acc[i][j][r] - mean[i][r];
          s = fmaf(d, d, s);
        }
        part[i][r] = s;
      }
    row_reduce(1, part);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) rstd[i][r] = __frsqrt_rn(fmaf(part[i][r], 1.f / kDV, a.eps));
    f32x4 gw = f32x4{1.f, 1.f, 1.f, 1.f}, gb = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.gn_w) gw = *reinterpret_cast<const f32x4*>(a.gn_w + size_t(h) * kDV + vcol);
    if (a.gn_b) gb = *reinterpret_cast<const f32x4*>(a.gn_b + size_t(h) * kDV + vcol);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float y = fmaf((acc[i][j][r] - mean[i][r]) * rstd[i][r], gw[j], gb[j]);
          if (has_gate) {
            const uint32_t word = gt[i][r][j >> 1];
            y *= swishf((j & 1) ? bf_hi(word) : bf_lo(word));
          }
          acc[i][j][r] = y;
        }
  }
  {
    // a class test per stored value of the sequence's rows
    uint32_t bad = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool vrow = t0 + 16 * i + r < len;
#pragma unroll
        for (int j = 0; j < 4; ++j) bad |= (vrow && !__builtin_isfinite(acc[i][j][r])) ? 1u : 0u;
      }
    if (__builtin_amdgcn_ballot_w64(bad != 0u) != 0 && (threadIdx.x & 63) == 0)
      __hip_atomic_fetch_or(P.status, kChunkwiseStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t srow = static_cast<uint32_t>((t0 + 16 * i + r) * kDV);
      if constexpr (OUT == RN_BF16) {
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int,
                               u32x2{pack_bf16x2(acc[i][0][r], acc[i][1][r]), pack_bf16x2(acc[i][2][r], acc[i][3][r])}),
            ro, gvoff, srow * 2, 0);
      } else {
        st_b128s(ro, 2 * gvoff, srow * 4,
                 __builtin_bit_cast(u32x4, f32x4{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]}));
      }
    }
}

int chunks_of(int N) { return (N + kC - 1) / kC; }

__global__ void seg_status_clear(uint32_t* status) {
  if (threadIdx.x == 0) status[0] = 0u;
}

constexpr size_t kStatusBytes = 256;   // the call's status word leads the workspace

}  // namespace

bool chunkwise_seg_supported(const CallArgs& a, int in_dt) {
  if (in_dt != RN_BF16 || a.dk != kDK || a.dv != kDV || a.gpair) return false;
  // 32-bit buffer offsets within one head's rows, with loads up to 256 rows past the end
  return (int64_t(a.N) + 512) * kDV * 4 < (int64_t(1) << 31);
}

// Per head of a group: L for a window's chunks, E and T per segment, the carried state.
size_t chunkwise_seg_ws_bytes(const CallArgs& a) {
  const int heads = min(a.B * a.H, kHeadsPerGroup);
  const size_t per_head = kWin * kSnap * 2 + kSegMax * kSnap * 4 + kSegMax * kSnap * 2 + kSnap * 4;
  return kStatusBytes + size_t(heads) * per_head;
}

hipError_t launch_chunkwise_seg(const CallArgs& a, int out_dt, const void* q, const void* k,
                                const void* v, const void* gate, const float* s_in, float* s_out,
                                void* out, void* ws, size_t ws_bytes, hipStream_t st) {
  if (chunkwise_seg_ws_bytes(a) > ws_bytes) return hipErrorInvalidValue;
  const int total = a.B * a.H;
  const int group = min(total, kHeadsPerGroup);
  const int nch = chunks_of(a.N);
  const int nwin = (nch + kWin - 1) / kWin;
  uint32_t* status = static_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(seg_status_clear, dim3(1), dim3(64), 0, st, status);
  uint8_t* p = static_cast<uint8_t*>(ws) + kStatusBytes;
  uint16_t* snap = reinterpret_cast<uint16_t*>(p);
  p += size_t(group) * kWin * kSnap * 2;
  float* ends = reinterpret_cast<float*>(p);
  p += size_t(group) * kSegMax * kSnap * 4;
  uint16_t* starts = reinterpret_cast<uint16_t*>(p);
  p += size_t(group) * kSegMax * kSnap * 2;
  float* carry = reinterpret_cast<float*>(p);
  for (int h0 = 0; h0 < total; h0 += kHeadsPerGroup) {
    const int heads = min(kHeadsPerGroup, total - h0);
    for (int win = 0; win < nwin; ++win) {
      const int wch = min(kWin, nch - win * kWin);
      SegArgs P;
      P.a = a;
      P.head0 = h0;
      P.heads = heads;
      P.win = win;
      P.nseg = (wch + kSegChunks - 1) / kSegChunks;
      P.q = static_cast<const uint16_t*>(q);
      P.k = static_cast<const uint16_t*>(k);
      P.v = static_cast<const uint16_t*>(v);
      P.gate = static_cast<const uint16_t*>(gate);
      P.snap = snap;
      P.ends = ends;
      P.starts = starts;
      P.src = win == 0 ? s_in : carry;
      P.src_group = win == 0 ? 0 : 1;
      P.dst = win + 1 == nwin ? s_out : carry;
      P.dst_group = win + 1 == nwin ? 0 : 1;
      P.out = out;
      P.status = status;
      const int g1 = (heads * P.nseg * 2 + 7) & ~7;
      hipLaunchKernelGGL(seg_states, dim3(g1), dim3(512), 0, st, P);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(seg_scan, dim3(heads * (kDV * kDK / 8) / 256), dim3(256), 0, st, P);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      const int g3 = (heads * kWin * 4 + 7) & ~7;
      if (out_dt == RN_BF16)
        hipLaunchKernelGGL(seg_outputs<RN_BF16>, dim3(g3), dim3(512), 0, st, P);
      else
        hipLaunchKernelGGL(seg_outputs<RN_F32>, dim3(g3), dim3(512), 0, st, P);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace rn
