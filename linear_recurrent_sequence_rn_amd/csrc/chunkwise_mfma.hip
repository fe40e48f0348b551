// Fused chunkwise retention for bf16 q/k/v, d_k = 256, d_v in {64, 128, 256, 512}
// (hwhale notes: chunkwise equation and ChunkwiseRetention listing; m0nads notes,
// "Chunkwise representation"; GroupNorm + swish gate of the multi-scale layer).
//
// Work split. A head's float32 state S (d_k x d_v) is cut into nS = d_v/64 column
// slices; one 256-thread workgroup owns one slice (64 KB of state, kept in MFMA
// accumulator registers for the whole sequence) and walks the sequence in blocks of
// 64 tokens. Inside the workgroup the four waves split d_k into quarters: wave w
// keeps S[64w:64w+64, slice] and computes the quarter's partial products, which are
// summed through LDS. Per block and wave (16x16x32 f16 MFMA, fp32 accumulate):
//   cross   acc  = xi ⊙ (Qh_w S_w)                 (Qh_w: 64 x 64 quarter of Qh)
//   scores  P_w  = alpha (Kh_w Qh_w^T ⊙ D)^T       (partial over the quarter)
//   intra   acc += P_w V
//   carry   S_w  = gamma^L S_w + (zeta ⊙ Kh_w)^T V
// The output is the sum of the four waves' acc; GroupNorm (+ gate) follows.
//
// Operand precision. q, k, v arrive in bf16; the rotation runs in float32 and every
// MFMA operand (Qh, Kh, V, the decayed scores, the state copy used by the cross term)
// is rounded to IEEE half. bf16 values are exact in half within its range, and half
// keeps 3 more significand bits than bf16, which is what holds the error after
// GroupNorm well inside 2e-2 (bf16 operands put it near 2.6e-2 on RetNet-shaped data).
// Precondition of this path: operands within half's range (|x| < 65504); values
// outside it need the plain float32 kernels (RN_FORCE_GENERIC).
//
// Sharing between the slices of one head. Every slice needs the whole rotated block
// of q and k. Each of the nS workgroups rotates 64/nS rows of the NEXT block and
// writes Qh, Kh and (zeta ⊙ Kh)^T in half to a ring of 4 block slots in the
// workspace; a per-head counter says how many row groups are published. GroupNorm
// statistics (per-row mean and centred sum of squares of each slice) go through a
// second counter, and the normalisation of block j waits for them while block j+1
// is computed. All slices of a head are placed on one XCD (blockIdx mod 8), so the
// exchange runs through that XCD's L2: a writer waits for its stores to complete
// before a relaxed agent-scope increment; readers poll with agent-scope atomic loads
// and read shared data with L1-bypassing (sc0) buffer loads. If the slices of a
// head turn out to sit on different XCDs, the kernel switches to release/acquire
// fences at agent scope. Every wait has a time limit that ends the kernel normally
// and raises an error word in the workspace.
//
// Ring safety: consuming block j needs every slice to have published block j, which
// they do at their iteration j-1; so no workgroup is more than one block ahead of
// another, and with 4 slots the slot a workgroup overwrites (block j+1) is never one
// that a slower workgroup can still read (blocks j-1 and j). Statistics of block j are
// read at iteration j+1 and their slot is rewritten at iteration j+4, by which time
// every slice has passed iteration j+2.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kT = 64;          // tokens per block
constexpr int kDK = 256;        // d_k of this kernel
constexpr int kSl = 64;         // d_v columns per workgroup
constexpr int kRing = 4;        // ring slots
constexpr int kRedLd = 68;      // LDS row stride (floats) of the reduction buffer
constexpr int kVtLd = 72;       // LDS row stride (bf16) of the transposed V slice
constexpr uint32_t kCntWords = 64;             // counter words per head
constexpr size_t kStatsPerHead = size_t(kRing) * 8 * kT * 2 * sizeof(float);   // 16 KB
constexpr size_t kSlotElems = size_t(kT) * kDK;                                  // 16384 bf16
constexpr size_t kRingPerHead = size_t(kRing) * 3 * kSlotElems * sizeof(uint16_t);
constexpr int kMaxWgPerLaunch = 4096;
constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz wall clock

// counter words
// Counter words per head. Publication counts are kept per ring slot: slot s counts the
// row groups published for blocks s, s+4, s+8, ...; block j is complete when word
// kReady + j%4 reaches nS*(j/4 + 1). (A single running count per head would not do: a
// workgroup that is one block ahead adds its next publication to the same count and
// can complete it while a slower slice has not yet published the block being waited
// for.) The same holds for the GroupNorm statistics (kStat + j%4). Words [8, 16)
// record the XCD of each slice (diagnostics).
enum { kArrive = 2, kXccMask = 3, kError = 4, kXccOfSlice = 8, kReady = 16, kStat = 20 };

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 u) { return __builtin_bit_cast(f16x8, u); }

// Round-to-nearest-even float32 pair -> packed f16 (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v;
  v[0] = static_cast<_Float16>(lo);
  v[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID (id 20), bits [3:0]
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xf;
}

struct alignas(16) Shared {
  float red[4][kT][kRedLd];          // partial outputs of the four waves
  uint16_t vt[kSl][kVtLd];           // V slice of the block, transposed: [dv][s]
  uint32_t mode;                     // 1 = agent-scope fences
};

// Buffer resource over the whole workspace; loads through it use sc0 (bypass L1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_sc0_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 1));
}
__device__ __forceinline__ u32x2 ld_sc0_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 1));
}

__device__ __forceinline__ void store_fence_release(bool agent) {
  if (agent) {
    __threadfence();
  } else {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Thread 0 waits until cnt[word] >= target, then the block synchronises. A wait that
// exceeds kWaitTicks raises cnt[kError]; once raised, every later wait of every
// workgroup of the head returns at once, so a broken exchange costs one time limit.
__device__ __forceinline__ void wait_count(uint32_t* cnt, int word, uint32_t target, bool agent) {
  if (threadIdx.x == 0) {
    uint32_t* p = cnt + word;
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      const uint64_t t0 = wall_clock64();
      while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        if (__hip_atomic_load(cnt + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWaitTicks) {
          __hip_atomic_fetch_or(cnt + kError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
  if (agent) __atomic_thread_fence(__ATOMIC_ACQUIRE);
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void signal_count(uint32_t* cnt, int word) {
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(cnt + word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Params {
  CallArgs a;
  int head0;       // first (b*H + h) of this launch group
  int heads;       // heads in this group
  int nS;          // slices per head
  int nb;          // blocks of 64 tokens
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  const float* s_in;
  float* s_out;
  void* out;
  uint8_t* ws;
};

template <int OUT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
chunkwise_fused(Params P) {
  const CallArgs& a = P.a;
  const int xcd = blockIdx.x & 7, L8 = blockIdx.x >> 3;
  const int hg = (L8 / P.nS) * 8 + xcd;  // head within the launch group
  if (hg >= P.heads) return;
  const int sl = L8 % P.nS;              // d_v slice
  const int nS = P.nS;
  const int bh = P.head0 + hg;
  const int h = bh % a.H;
  const int N = a.N, DV = a.dv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l16 = l & 15, g = l >> 4;

  __shared__ Shared sm;

  // workspace views
  uint32_t* cnt = reinterpret_cast<uint32_t*>(P.ws) + size_t(hg) * kCntWords;
  uint8_t* stats_base = P.ws + size_t(P.heads) * kCntWords * 4;
  float* stats = reinterpret_cast<float*>(stats_base + size_t(hg) * kStatsPerHead);
  uint8_t* ring_base = stats_base + size_t(P.heads) * kStatsPerHead;
  uint16_t* ring = reinterpret_cast<uint16_t*>(ring_base + size_t(hg) * kRingPerHead);
  const __amdgpu_buffer_rsrc_t wsr = ws_rsrc(P.ws);
  const uint32_t ring_off = static_cast<uint32_t>((ring_base - P.ws) + size_t(hg) * kRingPerHead);
  const uint32_t stats_off = static_cast<uint32_t>((stats_base - P.ws) + size_t(hg) * kStatsPerHead);

  // ---- placement check: are all slices of this head on one XCD? ----------------
  if (tid == 0) {
    const uint32_t x = xcc_id();
    __hip_atomic_store(cnt + kXccOfSlice + sl, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(cnt + kXccMask, 1u << x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    __hip_atomic_fetch_add(cnt + kArrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_count(cnt, kArrive, nS, true);
  if (tid == 0) {
    uint32_t m = __hip_atomic_load(cnt + kXccMask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.mode = (__builtin_popcount(m) == 1) ? 0u : 1u;
  }
  __syncthreads();
  const bool agent = sm.mode != 0;

  // ---- per-lane constants --------------------------------------------------------
  const float lg = a.hp.log2g[h];
  const float alpha = a.alpha;
  // xi for row t = 16m + 4g + r: gamma^(4g+r+1) * gamma^(16m)
  float xiF[4], G16[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) xiF[r] = exp2f(lg * float(4 * g + r + 1));
#pragma unroll
  for (int m = 0; m < 4; ++m) G16[m] = exp2f(lg * float(16 * m));
  // decay for P^T tile (s-tile 2e+hh, t-tile m), element r:
  //   t - s = (l16 - 8g - 4hh - r) + 16 (m - 2e)
  const bool factored = lg * 31.0f > -100.0f;  // gamma^-31 stays far below overflow
  float decF[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int r = 0; r < 4; ++r) decF[hh][r] = alpha * exp2f(lg * float(l16 - 8 * g - 4 * hh - r));

  // producer constants: this thread rotates coordinate pair pp of q (tid < 128) or k
  const int pp = tid & 127;
  const bool prod_k = tid >= 128;
  const float theta_p = a.ap.theta[pp];
  float c1, s1;
  angle_cs(1, theta_p, &c1, &s1);
  const int rows_per = kT / nS;
  const int r_lo = sl * rows_per;

  // ---- state: S_w tiles [a][b], a = dk tile (permuted rows), b = dv tile ------------
  // accumulator row 4g+r of tile a = 2c+hh holds dk = 64w + 32c + 8g + 4hh + r
  f32x4 Sacc[4][4];
#pragma unroll
  for (int ta = 0; ta < 4; ++ta)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int dk = 64 * w + 32 * (ta >> 1) + 8 * g + 4 * (ta & 1) + r;
        const int dv = sl * kSl + 16 * tb + l16;
        Sacc[ta][tb][r] = P.s_in ? P.s_in[(size_t(bh) * kDK + dk) * DV + dv] : 0.f;
      }

  const uint16_t* qg = P.q + size_t(bh) * N * kDK;
  const uint16_t* kg = P.k + size_t(bh) * N * kDK;
  const uint16_t* vg = P.v + size_t(bh) * N * DV + sl * kSl;
  const uint16_t* gg = P.gate ? P.gate + size_t(bh) * N * DV + sl * kSl : nullptr;
  const bool use_gn = a.flags & RN_EPI_GN;

  // ---- producer: rotate rows [r_lo, r_lo + rows_per) of block jb into its ring slot --
  auto produce = [&](int jb) {
    uint16_t* slot = ring + size_t(jb % kRing) * 3 * kSlotElems;
    const int row0 = jb * kT;
    const int Lb = min(kT, N - row0);
    const uint16_t* src = prod_k ? kg : qg;
    uint16_t* dst = slot + (prod_k ? kSlotElems : 0);
    uint16_t* dstT = slot + 2 * kSlotElems;
    float c, s;
    angle_cs(a.pos0 + row0 + r_lo, theta_p, &c, &s);
    for (int r8 = 0; r8 < rows_per; r8 += 8) {
      float z0[8], z1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int rr = r_lo + r8 + u;     // row in block
        float x0 = 0.f, x1 = 0.f;
        if (rr < Lb) {
          const uint32_t wv = *reinterpret_cast<const uint32_t*>(src + size_t(row0 + rr) * kDK + 2 * pp);
          x0 = __uint_as_float(wv << 16);
          x1 = __uint_as_float(wv & 0xffff0000u);
        }
        const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
        *reinterpret_cast<uint32_t*>(dst + size_t(rr) * kDK + 2 * pp) = pack_f16x2(y0, y1);
        const float zeta = (rr < Lb) ? exp2f(lg * float(Lb - 1 - rr)) : 0.f;
        z0[u] = y0 * zeta;
        z1[u] = y1 * zeta;
        const float cn = c * c1 - s * s1;
        s = c * s1 + s * c1;
        c = cn;
      }
      if (prod_k) {
        u32x4 t0, t1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          t0[u] = pack_f16x2(z0[2 * u], z0[2 * u + 1]);
          t1[u] = pack_f16x2(z1[2 * u], z1[2 * u + 1]);
        }
        *reinterpret_cast<u32x4*>(dstT + size_t(2 * pp) * kT + r_lo + r8) = t0;
        *reinterpret_cast<u32x4*>(dstT + size_t(2 * pp + 1) * kT + r_lo + r8) = t1;
      }
    }
    store_fence_release(agent);
    signal_count(cnt, kReady + jb % kRing);
  };

  float o_prev[16];
  int prev_row = -1;  // first row of the block held in o_prev

  // GroupNorm + gate + store of this wave's 16 rows of block `jb` (values `o`)
  auto finalize = [&](int jb, const float* o) {
    const int t_loc = 16 * w + (l >> 2);
    const int t = jb * kT + t_loc;
    const int c0 = (l & 3) * 16;           // first column (within the slice)
    float y[16];
    if (use_gn) {
      // combine the slices' (mean, M2) for row t_loc, pairwise (Chan et al.)
      const uint32_t so = stats_off + static_cast<uint32_t>(((jb % kRing) * 8 * kT + t_loc) * 2 * sizeof(float));
      float mu = 0.f, m2 = 0.f, n = 0.f;
      for (int j = 0; j < nS; ++j) {
        u32x2 st = ld_sc0_b64(wsr, so + static_cast<uint32_t>(j * kT * 2 * sizeof(float)));
        const float mj = __uint_as_float(st[0]), m2j = __uint_as_float(st[1]);
        const float nn = n + float(kSl);
        const float d = mj - mu;
        mu += d * (float(kSl) / nn);
        m2 += m2j + d * d * (n * float(kSl) / nn);
        n = nn;
      }
      const float rstd = 1.0f / sqrtf(m2 / float(DV) + a.eps);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = (o[i] - mu) * rstd;
      const int col = h * DV + sl * kSl + c0;
      if (a.gn_w) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] *= a.gn_w[col + i];
      }
      if (a.gn_b) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] += a.gn_b[col + i];
      }
      if (gg && t < N) {
        const u32x4* gp = reinterpret_cast<const u32x4*>(gg + size_t(t) * DV + c0);
        u32x4 g0 = gp[0], g1 = gp[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[2 * i] *= swishf(__uint_as_float(g0[i] << 16));
          y[2 * i + 1] *= swishf(__uint_as_float(g0[i] & 0xffff0000u));
          y[8 + 2 * i] *= swishf(__uint_as_float(g1[i] << 16));
          y[8 + 2 * i + 1] *= swishf(__uint_as_float(g1[i] & 0xffff0000u));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = o[i];
    }
    if (t < N) {
      if constexpr (OUT == RN_BF16) {
        u32x4 p0, p1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
          p1[i] = pack_bf16x2(y[8 + 2 * i], y[8 + 2 * i + 1]);
        }
        u32x4* op = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(P.out) + (size_t(bh) * N + t) * DV + sl * kSl + c0);
        op[0] = p0;
        op[1] = p1;
      } else {
        f32x4* op = reinterpret_cast<f32x4*>(static_cast<float*>(P.out) + (size_t(bh) * N + t) * DV + sl * kSl + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) op[i] = f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
      }
    }
  };

  produce(0);

  for (int jb = 0; jb < P.nb; ++jb) {
    const int row0 = jb * kT;
    const int Lb = min(kT, N - row0);
    if (jb + 1 < P.nb) produce(jb + 1);   // ends with a block barrier

    // ---- stage V slice of this block, transposed, into LDS (zero rows >= Lb) ----
    {
      const int s0 = 4 * (tid >> 4), d0 = 4 * (tid & 15);
      u32x2 rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (s0 + i < Lb)
          rv[i] = *reinterpret_cast<const u32x2*>(vg + size_t(row0 + s0 + i) * DV + d0);
        else
          rv[i] = u32x2{0u, 0u};
      }
      float fv[4][4];   // [row i][column j] as float32
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fv[i][0] = __uint_as_float(rv[i][0] << 16);
        fv[i][1] = __uint_as_float(rv[i][0] & 0xffff0000u);
        fv[i][2] = __uint_as_float(rv[i][1] << 16);
        fv[i][3] = __uint_as_float(rv[i][1] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 o;
        o[0] = pack_f16x2(fv[0][j], fv[1][j]);
        o[1] = pack_f16x2(fv[2][j], fv[3][j]);
        *reinterpret_cast<u32x2*>(&sm.vt[d0 + j][s0]) = o;
      }
    }
    wait_count(cnt, kReady + jb % kRing, uint32_t(nS) * uint32_t(jb / kRing + 1), agent);  // + barrier

    const uint32_t slot_off = ring_off + static_cast<uint32_t>((jb % kRing) * 3 * kSlotElems * sizeof(uint16_t));
    const uint32_t kh_off = slot_off + static_cast<uint32_t>(kSlotElems * sizeof(uint16_t));
    const uint32_t kt_off = slot_off + static_cast<uint32_t>(2 * kSlotElems * sizeof(uint16_t));

    // ---- cross term: acc[m][b] = Qh[16m.., dk quarter] · S_w -------------------------
    f16x8 qf[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        qf[m][c] = as_f16x8(ld_sc0_b128(wsr, slot_off + static_cast<uint32_t>(((16 * m + l16) * kDK + 64 * w + 32 * c + 8 * g) * 2)));
    f16x8 sf[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        u32x4 u;
        u[0] = pack_f16x2(Sacc[2 * c][tb][0], Sacc[2 * c][tb][1]);
        u[1] = pack_f16x2(Sacc[2 * c][tb][2], Sacc[2 * c][tb][3]);
        u[2] = pack_f16x2(Sacc[2 * c + 1][tb][0], Sacc[2 * c + 1][tb][1]);
        u[3] = pack_f16x2(Sacc[2 * c + 1][tb][2], Sacc[2 * c + 1][tb][3]);
        sf[c][tb] = as_f16x8(u);
      }
    f32x4 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mfma(qf[m][0], sf[0][tb], z);
        z = mfma(qf[m][1], sf[1][tb], z);
        // xi_t = gamma^(t_local + 1), t_local = 16m + 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] *= alpha * xiF[r] * G16[m];
        acc[m][tb] = z;
      }

    // ---- scores: P^T tiles (s-tile i, t-tile m), e = i/2 <= m/2 ----------------------
    // K rows for tile i: A-row l16 <-> s = 32e + 8(l16>>2) + 4(i&1) + (l16&3)
    f16x8 kf[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 32 * (i >> 1) + 8 * (l16 >> 2) + 4 * (i & 1) + (l16 & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        kf[i][c] = as_f16x8(ld_sc0_b128(wsr, kh_off + static_cast<uint32_t>((s * kDK + 64 * w + 32 * c + 8 * g) * 2)));
    }
    // P A-fragments for the PV product: pf[m][e]
    f16x8 pf[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (e > (m >> 1)) continue;
        f32x4 pt[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int i = 2 * e + hh;
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = mfma(kf[i][0], qf[m][0], z);
          z = mfma(kf[i][1], qf[m][1], z);
          // element r: s = 32e + 8g + 4hh + r, t = 16m + l16
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = (l16 - 8 * g - 4 * hh - r) + 16 * (m - 2 * e);
            float f;
            if (factored)
              f = decF[hh][r] * G16[m - 2 * e];
            else
              f = alpha * exp2f(lg * float(d));
            z[r] = (d >= 0) ? z[r] * f : 0.f;
          }
          pt[hh] = z;
        }
        u32x4 u;
        u[0] = pack_f16x2(pt[0][0], pt[0][1]);
        u[1] = pack_f16x2(pt[0][2], pt[0][3]);
        u[2] = pack_f16x2(pt[1][0], pt[1][1]);
        u[3] = pack_f16x2(pt[1][2], pt[1][3]);
        pf[m][e] = as_f16x8(u);
      }

    // ---- V fragments (B operand, k = s): vf[e][b] -------------------------------
    f16x8 vf[2][4];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        vf[e][tb] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.vt[16 * tb + l16][32 * e + 8 * g]));

    // ---- intra term -------------------------------------------------------------
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[m][tb] = mfma(pf[m][0], vf[0][tb], acc[m][tb]);
        if (m >= 2) acc[m][tb] = mfma(pf[m][1], vf[1][tb], acc[m][tb]);
      }

    // ---- sum the four waves' partial outputs through LDS -----------------------------
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.red[w][16 * m + 4 * g + r][16 * tb + l16] = acc[m][tb][r];
    __syncthreads();
    float o_cur[16];
    {
      const int t_loc = 16 * w + (l >> 2), c0 = (l & 3) * 16;
#pragma unroll
      for (int i = 0; i < 16; ++i) o_cur[i] = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          f32x4 x = *reinterpret_cast<const f32x4*>(&sm.red[ww][t_loc][c0 + 4 * i4]);
#pragma unroll
          for (int r = 0; r < 4; ++r) o_cur[4 * i4 + r] += x[r];
        }
    }

    // ---- GroupNorm statistics of this slice: (mean, centred sum of squares) ----------
    if (use_gn) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += o_cur[i];
      sum += __shfl_xor(sum, 1, 64);
      sum += __shfl_xor(sum, 2, 64);
      const float mu = sum * (1.0f / kSl);
      float m2 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) { const float d = o_cur[i] - mu; m2 += d * d; }
      m2 += __shfl_xor(m2, 1, 64);
      m2 += __shfl_xor(m2, 2, 64);
      if ((l & 3) == 0) {
        const int t_loc = 16 * w + (l >> 2);
        float* sp = stats + ((jb % kRing) * 8 * kT + sl * kT + t_loc) * 2;
        *reinterpret_cast<u32x2*>(sp) = u32x2{__float_as_uint(mu), __float_as_uint(m2)};
      }
      store_fence_release(agent);
      signal_count(cnt, kStat + jb % kRing);
    }

    // ---- state carry: S_w = gamma^Lb S_w + (zeta ⊙ Kh)^T V ---------------------------
    {
      const float gL = exp2f(lg * float(Lb));
      f16x8 ktf[4][2];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const int dk = 64 * w + 32 * (ta >> 1) + 8 * (l16 >> 2) + 4 * (ta & 1) + (l16 & 3);
#pragma unroll
        for (int e = 0; e < 2; ++e)
          ktf[ta][e] = as_f16x8(ld_sc0_b128(wsr, kt_off + static_cast<uint32_t>((dk * kT + 32 * e + 8 * g) * 2)));
      }
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          f32x4 z = Sacc[ta][tb] * gL;
          z = mfma(ktf[ta][0], vf[0][tb], z);
          z = mfma(ktf[ta][1], vf[1][tb], z);
          Sacc[ta][tb] = z;
        }
    }

    // ---- normalise and store the previous block (its statistics are complete) --------
    if (use_gn) {
      if (prev_row >= 0) {
        wait_count(cnt, kStat + (jb - 1) % kRing, uint32_t(nS) * uint32_t((jb - 1) / kRing + 1), agent);
        finalize(jb - 1, o_prev);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) o_prev[i] = o_cur[i];
      prev_row = row0;
    } else {
      finalize(jb, o_cur);
    }
    __syncthreads();  // LDS buffers are reused by the next block
  }
  if (use_gn && prev_row >= 0) {
    wait_count(cnt, kStat + (P.nb - 1) % kRing, uint32_t(nS) * uint32_t((P.nb - 1) / kRing + 1), agent);
    finalize(P.nb - 1, o_prev);
  }

  if (P.s_out) {
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int dk = 64 * w + 32 * (ta >> 1) + 8 * g + 4 * (ta & 1) + r;
          const int dv = sl * kSl + 16 * tb + l16;
          P.s_out[(size_t(bh) * kDK + dk) * DV + dv] = Sacc[ta][tb][r];
        }
  }
}

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Heads per cooperative launch: every workgroup must be resident at once (one per CU).
int heads_per_group(int nS) {
  const int cus = cu_count();
  if (cus <= 0) return 0;
  return 8 * (cus / (8 * nS));
}

}  // namespace

bool chunkwise_mfma_supported(const CallArgs& a, int in_dt) {
  return in_dt == RN_BF16 && a.dk == kDK &&
         (a.dv == 64 || a.dv == 128 || a.dv == 256 || a.dv == 512);
}

size_t chunkwise_mfma_ws_bytes(const CallArgs& a) {
  const int nS = a.dv / kSl;
  int G = heads_per_group(nS);
  if (G <= 0) G = 8 * (256 / (8 * nS));  // no device visible: size for a 256-CU part
  G = min(G, a.B * a.H);
  return size_t(G) * (kCntWords * 4 + kStatsPerHead + kRingPerHead);
}

hipError_t launch_chunkwise_mfma(const CallArgs& a, int out_dt, const void* q, const void* k,
                                 const void* v, const void* gate, const float* s_in,
                                 float* s_out, void* out, void* ws, size_t ws_bytes,
                                 hipStream_t st) {
  const int nS = a.dv / kSl;
  const int G = heads_per_group(nS);
  if (G <= 0) return hipErrorNoDevice;
  const int total = a.B * a.H;
  Params p;
  p.a = a;
  p.nS = nS;
  p.nb = (a.N + kT - 1) / kT;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.gate = static_cast<const uint16_t*>(gate);
  p.s_in = s_in;
  p.s_out = s_out;
  p.out = out;
  p.ws = static_cast<uint8_t*>(ws);
  for (int h0 = 0; h0 < total; h0 += G) {
    const int heads = min(G, total - h0);
    if (size_t(heads) * (kCntWords * 4 + kStatsPerHead + kRingPerHead) > ws_bytes)
      return hipErrorInvalidValue;
    p.head0 = h0;
    p.heads = heads;
    const int nwords = heads * int(kCntWords);
    hipLaunchKernelGGL(zero_words, dim3((nwords + 255) / 256), dim3(256), 0, st,
                       static_cast<uint32_t*>(ws), nwords);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = 8 * nS * ((heads + 7) / 8);
    void* args[] = {&p};
    if (out_dt == RN_BF16)
      e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&chunkwise_fused<RN_BF16>),
                                     dim3(grid), dim3(256), args, 0, st);
    else
      e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&chunkwise_fused<RN_F32>),
                                     dim3(grid), dim3(256), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rn
