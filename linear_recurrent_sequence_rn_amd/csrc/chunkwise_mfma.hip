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
// they do at their iteration j-2; so no workgroup is more than one block ahead of
// another. Blocks are produced two ahead, so with 8 slots the slot a workgroup
// overwrites (block j+2) is never one a slower workgroup can still read (j-1, j). Statistics of block j are
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
constexpr int kRing = 8;        // ring slots (blocks of Qh/Kh/Kh^T)
constexpr int kStatRing = 4;    // statistics slots
constexpr int kRedLd = 68;      // LDS row stride (floats) of the reduction buffer
constexpr int kVtLd = 72;       // LDS row stride (bf16) of the transposed V slice
constexpr uint32_t kCntWords = 64;             // counter words per head
constexpr size_t kStatsPerHead = size_t(kStatRing) * 8 * kT * 2 * sizeof(float);   // 16 KB
constexpr size_t kSlotElems = size_t(kT) * kDK;                                  // 16384 bf16
constexpr size_t kRingPerHead = size_t(kRing) * 3 * kSlotElems * sizeof(uint16_t);
constexpr int kMaxWgPerLaunch = 4096;
constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz wall clock

// counter words
// Counter words per head. Publication counts are kept per ring slot and in waves:
// slot s counts the waves that published blocks s, s+kRing, s+2kRing, ...; block j is
// complete when word kReady + j%kRing reaches 4*nS*(j/kRing + 1). (A single running
// count per head would not do: a wave that is ahead adds its next publication to the
// same count and can complete it while a slower slice has not yet published the block
// being waited for.) The GroupNorm statistics use kStat + j%kStatRing the same way.
// Words [8, 16) record the XCD of each slice (diagnostics).
enum { kArrive = 2, kXccMask = 3, kError = 4, kXccOfSlice = 8, kReady = 16, kStat = 24 };

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
  u32x4 qk[4][16][64];               // next block's Qh/Kh fragments, per wave and lane
  uint32_t mode;                     // 1 = agent-scope fences
};

// Buffer resource over the whole workspace; loads through it use sc0 (bypass L1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// Buffer resource over [base, base + bytes): loads past the end return 0 and stores
// past the end are dropped, which is how ragged tails and rows beyond N are handled.
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
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
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
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, g = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)

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
  const float gam = a.hp.gamma[h];
  const float alpha = a.alpha;
  float G16[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) G16[m] = exp2f(lg * float(16 * m));
  // alpha * xi_t, xi_t = gamma^(t+1), for the row t = 16m + l16 this lane feeds to the
  // cross-term MFMA, as a half splat: the cross term scales the rows of Qh.
  f16x8 xs[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const _Float16 x = static_cast<_Float16>(alpha * exp2f(lg * float(16 * m + l16 + 1)));
    xs[m] = f16x8{x, x, x, x, x, x, x, x};
  }
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
  const bool prod_k = w >= 2;        // waves 0-1 rotate q, waves 2-3 rotate k
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

  // this head's rows of q or k (producer), and its d_v slice of v, gate and out
  const bool use_gn = a.flags & RN_EPI_GN;
  const bool has_gate = P.gate != nullptr;
  const int64_t qk_bytes = int64_t(N) * kDK * 2;
  const __amdgpu_buffer_rsrc_t r_src = range_rsrc((prod_k ? P.k : P.q) + size_t(bh) * N * kDK, qk_bytes);
  const int64_t slice_bytes = (int64_t(N) * DV - sl * kSl) * 2;  // to the end of this head
  const size_t slice0 = size_t(bh) * N * DV + sl * kSl;
  const __amdgpu_buffer_rsrc_t r_v = range_rsrc(P.v + slice0, slice_bytes);
  const __amdgpu_buffer_rsrc_t r_g = range_rsrc(has_gate ? P.gate + slice0 : P.v + slice0, slice_bytes);
  const int osz = (OUT == RN_BF16) ? 2 : 4;
  const __amdgpu_buffer_rsrc_t r_o =
      range_rsrc(static_cast<uint8_t*>(P.out) + slice0 * osz, slice_bytes / 2 * osz);
  const int t_fin = 16 * w + (l >> 2);     // row (in block) this lane normalises and stores
  const int c_fin = (l & 3) * 16;          // first of its 16 columns (within the slice)
  const float inv_nS = 1.0f / float(nS);

  // ---- producer ------------------------------------------------------------------
  // Rows [rbase, rbase + 8) of block jb for this thread's coordinate pair, as packed
  // bf16 pairs; zero past the end of the sequence.
  auto load8 = [&](int jb, int rbase, uint32_t* xr) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      xr[u] = ld_b32(r_src, static_cast<uint32_t>(((jb * kT + rbase + u) * kDK + 2 * pp) * 2));
  };
  // Rotates this workgroup's rows [r_lo, r_lo + rows_per) of block jb into the block's
  // ring slot. `first8` holds the first 8 rows, loaded one iteration earlier.
  auto produce = [&](int jb, const uint32_t* first8) {
    uint16_t* slot = ring + size_t(jb % kRing) * 3 * kSlotElems;
    const int row0 = jb * kT;
    const int Lb = min(kT, N - row0);
    uint16_t* dst = slot + (prod_k ? kSlotElems : 0);
    uint16_t* dstT = slot + 2 * kSlotElems;
    float c, s;
    angle_cs(a.pos0 + row0 + r_lo, theta_p, &c, &s);
    for (int r8 = 0; r8 < rows_per; r8 += 8) {
      uint32_t xr[8];
      if (r8 == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) xr[u] = first8[u];
      } else {
        load8(jb, r_lo + r8, xr);
      }
      float z0[8], z1[8];
      // zeta_rr = gamma^(Lb-1-rr) for rr < Lb, else 0: computed at the last valid row of
      // these 8 and multiplied by gamma going back (no overflow for gamma in (0, 1])
      float zeta[8];
      if (prod_k) {
        const int rfirst = r_lo + r8;
        const int rlast = min(rfirst + 7, Lb - 1);
        float zcur = exp2f(lg * float(max(Lb - 1 - rlast, 0)));
#pragma unroll
        for (int u = 7; u >= 0; --u) {
          const bool ok = rfirst + u <= rlast;
          zeta[u] = ok ? zcur : 0.f;
          zcur = ok ? zcur * gam : zcur;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int rr = r_lo + r8 + u;     // row in block
        const float x0 = __uint_as_float(xr[u] << 16);
        const float x1 = __uint_as_float(xr[u] & 0xffff0000u);
        const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
        *reinterpret_cast<uint32_t*>(dst + size_t(rr) * kDK + 2 * pp) = pack_f16x2(y0, y1);
        if (prod_k) {
          z0[u] = y0 * zeta[u];
          z1[u] = y1 * zeta[u];
        }
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
  };
  // Flags are per wave: every wave publishes its own stores and every wave checks
  // readiness for itself, so no block barrier is needed around an exchange. Counts are
  // therefore kept in waves: block j is complete once 4*nS waves have published it.
  const uint32_t nW = 4u * uint32_t(nS);
  // Publishes this wave's stores: block `ready_block` of the ring and/or the statistics
  // of block `stat_block` (-1 = none).
  auto release = [&](int ready_block, int stat_block) {
    store_fence_release(agent);
    if (l == 0) {
      if (ready_block >= 0)
        __hip_atomic_fetch_add(cnt + kReady + ready_block % kRing, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (stat_block >= 0)
        __hip_atomic_fetch_add(cnt + kStat + stat_block % kStatRing, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // Issues a read of a count (lane 0); `settle` later waits until it reaches `target`.
  auto poll = [&](int word) -> uint32_t {
    uint32_t v = 0u;
    if (l == 0) v = __hip_atomic_load(cnt + word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return v;
  };
  auto settle = [&](uint32_t v, int word, uint32_t target) {
    v = __builtin_amdgcn_readfirstlane(v);
    if (v < target) {
      const uint64_t t0 = wall_clock64();
      while (true) {
        uint32_t x = 0u, err = 0u;
        if (l == 0) {
          x = __hip_atomic_load(cnt + word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          err = __hip_atomic_load(cnt + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        x = __builtin_amdgcn_readfirstlane(x);
        err = __builtin_amdgcn_readfirstlane(err);
        if (x >= target || err) break;
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWaitTicks) {
          if (l == 0) __hip_atomic_fetch_or(cnt + kError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    if (agent) __atomic_thread_fence(__ATOMIC_ACQUIRE);
    __asm__ volatile("" ::: "memory");
  };
  auto ready_target = [&](int jb) { return nW * uint32_t(jb / kRing + 1); };
  auto stat_target = [&](int jb) { return nW * uint32_t(jb / kStatRing + 1); };

  // ---- per-block operand loads ----------------------------------------------------
  auto load_v = [&](int jb, u32x2* rv) {   // V rows s0..s0+3, columns d0..d0+3 (bf16)
    const int s0 = 4 * (tid >> 4), d0 = 4 * (tid & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rv[i] = ld_b64(r_v, static_cast<uint32_t>(((jb * kT + s0 + i) * DV + d0) * 2));
  };
  auto load_gate = [&](int jb, u32x4* gt) {
    const uint32_t off = static_cast<uint32_t>(((jb * kT + t_fin) * DV + c_fin) * 2);
    if (has_gate && use_gn) {
      gt[0] = ld_b128(r_g, off);
      gt[1] = ld_b128(r_g, off + 16);
    } else {
      gt[0] = gt[1] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // The next block's Qh / Kh fragments of this wave are copied from the ring straight
  // into LDS (buffer loads with the lds modifier, sc0), one iteration ahead; each lane
  // later reads back the 16 bytes it loaded. Fragment f: Qh (m, c) -> 2m + c,
  // Kh (i, c) -> 8 + 2i + c.
  auto stage_qk = [&](int jb) {
    const uint32_t slot_off = ring_off + static_cast<uint32_t>((jb % kRing) * 3 * kSlotElems * sizeof(uint16_t));
    const uint32_t kh_off = slot_off + static_cast<uint32_t>(kSlotElems * sizeof(uint16_t));
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wsr, (__attribute__((address_space(3))) void*)(&sm.qk[w][2 * m + c][0]), 16,
            slot_off + static_cast<uint32_t>(((16 * m + l16) * kDK + 64 * w + 32 * c + 8 * g) * 2), 0, 0, 1);
    // K rows for tile i: A-row l16 <-> s = 32e + 8(l16>>2) + 4(i&1) + (l16&3)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 32 * (i >> 1) + 8 * (l16 >> 2) + 4 * (i & 1) + (l16 & 3);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wsr, (__attribute__((address_space(3))) void*)(&sm.qk[w][8 + 2 * i + c][0]), 16,
            kh_off + static_cast<uint32_t>((s * kDK + 64 * w + 32 * c + 8 * g) * 2), 0, 0, 1);
    }
  };
  auto read_qk = [&](f16x8 (*qf)[2], f16x8 (*kf)[2]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c) qf[m][c] = as_f16x8(sm.qk[w][2 * m + c][l]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) kf[i][c] = as_f16x8(sm.qk[w][8 + 2 * i + c][l]);
  };

  // GroupNorm + gate + store of this lane's row of block `jb` (values `o`), with the
  // slices' statistics `st` and the gate row `gt` loaded earlier.
  auto finalize = [&](int jb, const float* o, const u32x2* st, const u32x4* gt) {
    float y[16];
    if (use_gn) {
      // combine the slices' (mean, M2): equal counts, so the mean is the average of the
      // slice means and M2 = sum M2_j + 64 sum (mean_j - mean)^2 (Chan et al.)
      float mu = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nS) mu += __uint_as_float(st[j][0]);
      mu *= inv_nS;
      float m2 = 0.f, dd = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < nS) {
          const float d = __uint_as_float(st[j][0]) - mu;
          m2 += __uint_as_float(st[j][1]);
          dd = fmaf(d, d, dd);
        }
      m2 = fmaf(float(kSl), dd, m2);
      const float rstd = 1.0f / sqrtf(m2 / float(DV) + a.eps);
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = (o[i] - mu) * rstd;
      const int col = h * DV + sl * kSl + c_fin;
      if (a.gn_w) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] *= a.gn_w[col + i];
      }
      if (a.gn_b) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] += a.gn_b[col + i];
      }
      if (has_gate) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[2 * i] *= swishf(__uint_as_float(gt[0][i] << 16));
          y[2 * i + 1] *= swishf(__uint_as_float(gt[0][i] & 0xffff0000u));
          y[8 + 2 * i] *= swishf(__uint_as_float(gt[1][i] << 16));
          y[8 + 2 * i + 1] *= swishf(__uint_as_float(gt[1][i] & 0xffff0000u));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = o[i];
    }
    const uint32_t ooff = static_cast<uint32_t>(((jb * kT + t_fin) * DV + c_fin) * osz);
    if constexpr (OUT == RN_BF16) {
      u32x4 p0, p1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p0[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
        p1[i] = pack_bf16x2(y[8 + 2 * i], y[8 + 2 * i + 1]);
      }
      st_b128(r_o, ooff, p0);
      st_b128(r_o, ooff + 16, p1);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_b128(r_o, ooff + 16 * i, __builtin_bit_cast(u32x4, f32x4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]}));
    }
  };

  // ---- prologue: publish blocks 0 and 1, prefetch for iteration 0 -----------------
  uint32_t xq_a[8];               // producer rows of the block produced next
  load8(0, r_lo, xq_a);
  produce(0, xq_a);
  if (P.nb > 1) {
    load8(1, r_lo, xq_a);
    produce(1, xq_a);
  }
  store_fence_release(agent);
  if (l == 0) {
    __hip_atomic_fetch_add(cnt + kReady + 0, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (P.nb > 1) __hip_atomic_fetch_add(cnt + kReady + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  load8(2, r_lo, xq_a);
  u32x2 rv_a[4], rv_b[4];         // V rows of blocks jb and jb+1
  load_v(0, rv_a);
  load_v(1, rv_b);
  u32x4 gt_a[2], gt_b[2];         // gate rows of the block normalised next
  gt_a[0] = gt_a[1] = u32x4{0u, 0u, 0u, 0u};
  settle(poll(kReady + 0), kReady + 0, ready_target(0));
  stage_qk(0);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float o_prev[16];
  uint32_t ps = 0u;               // pre-read count of the previous block's statistics

  for (int jb = 0; jb < P.nb; ++jb) {
    const int Lb = min(kT, N - jb * kT);
    const bool produced = jb + 2 < P.nb;
    // readiness of the next block, read now and checked at the end of the iteration
    const uint32_t pr = (jb + 1 < P.nb) ? poll(kReady + (jb + 1) % kRing) : 0u;

    // (a) stage the V slice of this block, transposed, in LDS (rows >= Lb are zero)
    {
      const int s0 = 4 * (tid >> 4), d0 = 4 * (tid & 15);
      float fv[4][4];   // [row i][column j] as float32
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fv[i][0] = __uint_as_float(rv_a[i][0] << 16);
        fv[i][1] = __uint_as_float(rv_a[i][0] & 0xffff0000u);
        fv[i][2] = __uint_as_float(rv_a[i][1] << 16);
        fv[i][3] = __uint_as_float(rv_a[i][1] & 0xffff0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 o;
        o[0] = pack_f16x2(fv[0][j], fv[1][j]);
        o[1] = pack_f16x2(fv[2][j], fv[3][j]);
        *reinterpret_cast<u32x2*>(&sm.vt[d0 + j][s0]) = o;
      }
    }
    __syncthreads();   // (b) V visible; the previous block's LDS reads are done

    // this block's Qh / Kh fragments (staged during the previous iteration), then the
    // next block's into the same LDS region once the reads have returned
    f16x8 qf[4][2], kf[4][2];
    read_qk(qf, kf);
    if (jb + 1 < P.nb) {
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      settle(pr, kReady + (jb + 1) % kRing, ready_target(jb + 1));
      stage_qk(jb + 1);
    }

    // (c) statistics of the previous block, for the normalisation at the end
    u32x2 st[8];
    if (use_gn && jb > 0) {
      settle(ps, kStat + (jb - 1) % kStatRing, stat_target(jb - 1));
      const uint32_t so = stats_off + static_cast<uint32_t>((((jb - 1) % kStatRing) * 8 * kT + t_fin) * 2 * sizeof(float));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        st[j] = (j < nS) ? ld_sc0_b64(wsr, so + static_cast<uint32_t>(j * kT * 2 * sizeof(float))) : u32x2{0u, 0u};
    }

    // transposed, zeta-weighted K of this quarter for the state carry (A operand),
    // loaded early: it is used last
    f16x8 ktf[4][2];
    {
      const uint32_t kt_off = ring_off + static_cast<uint32_t>(((jb % kRing) * 3 + 2) * kSlotElems * sizeof(uint16_t));
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        const int dk = 64 * w + 32 * (ta >> 1) + 8 * (l16 >> 2) + 4 * (ta & 1) + (l16 & 3);
#pragma unroll
        for (int e = 0; e < 2; ++e)
          ktf[ta][e] = as_f16x8(ld_sc0_b128(wsr, kt_off + static_cast<uint32_t>((dk * kT + 32 * e + 8 * g) * 2)));
      }
    }

    // (d) rotate this workgroup's rows of block jb + 2 into the ring
    if (produced) produce(jb + 2, xq_a);

    // (5) scores first (they need Qh unscaled), then the cross term
    // scores: P^T tiles (s-tile i, t-tile m), e = i/2 <= m/2
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
            const float f = factored ? decF[hh][r] * G16[m - 2 * e] : alpha * exp2f(lg * float(d));
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
    // cross term: acc[m][b] = (alpha xi ⊙ Qh)[16m.., dk quarter] · S_w; the row factor
    // alpha * xi_t is applied to the Qh fragments (after the scores used them)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 2; ++c) qf[m][c] = qf[m][c] * xs[m];
    f32x4 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mfma(qf[m][0], sf[0][tb], z);
        z = mfma(qf[m][1], sf[1][tb], z);
        acc[m][tb] = z;
      }

    // V fragments (B operand, k = s): vf[e][b]
    f16x8 vf[2][4];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        vf[e][tb] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.vt[16 * tb + l16][32 * e + 8 * g]));

    // intra term
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[m][tb] = mfma(pf[m][0], vf[0][tb], acc[m][tb]);
        if (m >= 2) acc[m][tb] = mfma(pf[m][1], vf[1][tb], acc[m][tb]);
      }

    // sum the four waves' partial outputs through LDS
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.red[w][16 * m + 4 * g + r][16 * tb + l16] = acc[m][tb][r];
    __syncthreads();
    float o_cur[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o_cur[i] = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 x = *reinterpret_cast<const f32x4*>(&sm.red[ww][t_fin][c_fin + 4 * i4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) o_cur[4 * i4 + r] += x[r];
      }

    // GroupNorm statistics of this slice: (mean, centred sum of squares) per row
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
        float* sp = stats + ((jb % kStatRing) * 8 * kT + sl * kT + t_fin) * 2;
        *reinterpret_cast<u32x2*>(sp) = u32x2{__float_as_uint(mu), __float_as_uint(m2)};
      }
    }

    // state carry: S_w = gamma^Lb S_w + (zeta ⊙ Kh)^T V
    {
      const float gL = exp2f(lg * float(Lb));
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

    // (e) publish this wave's ring rows of block jb + 2 and statistics of block jb
    release(produced ? jb + 2 : -1, use_gn ? jb : -1);
    // (f) prefetch from HBM for later iterations
    load8(jb + 3, r_lo, xq_a);
#pragma unroll
    for (int i = 0; i < 4; ++i) rv_a[i] = rv_b[i];
    load_v(jb + 2, rv_b);
    load_gate(jb, gt_b);
    // (h) normalise and store the previous block (or this one without GroupNorm)
    if (use_gn) {
      if (jb > 0) finalize(jb - 1, o_prev, st, gt_a);
#pragma unroll
      for (int i = 0; i < 16; ++i) o_prev[i] = o_cur[i];
      gt_a[0] = gt_b[0];
      gt_a[1] = gt_b[1];
      ps = poll(kStat + jb % kStatRing);
    } else {
      finalize(jb, o_cur, st, gt_a);
    }
  }
  if (use_gn) {
    const int jl = P.nb - 1;
    settle(ps, kStat + jl % kStatRing, stat_target(jl));
    u32x2 st[8];
    const uint32_t so = stats_off + static_cast<uint32_t>(((jl % kStatRing) * 8 * kT + t_fin) * 2 * sizeof(float));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      st[j] = (j < nS) ? ld_sc0_b64(wsr, so + static_cast<uint32_t>(j * kT * 2 * sizeof(float))) : u32x2{0u, 0u};
    finalize(jl, o_prev, st, gt_a);
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
