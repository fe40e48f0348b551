// Fused chunkwise retention for bf16 q/k/v, d_k = 256, d_v in {64, 128, 256, 512}
// (hwhale notes: chunkwise equation and ChunkwiseRetention listing; m0nads notes,
// "Chunkwise representation"; GroupNorm + swish gate of the multi-scale layer).
//
// Work split. A head's float32 state S (d_k x d_v) is cut into nS = d_v/64 column
// slices; one 512-thread workgroup owns one slice and walks the sequence in blocks of
// 64 tokens. Its eight waves take two roles, one wave of each per SIMD, so that the
// matrix work of one role runs while the other role's vector work issues:
//   M waves (0-3): wave w keeps rows [64w, 64w+64) of the slice's state (64 KB in all,
//     in MFMA accumulator registers for the whole sequence) and does every MFMA of a
//     block over its quarter of d_k. Its partial outputs go to LDS. The M waves also do
//     every wait on other workgroups, because their only memory traffic is the L2 ->
//     LDS copies they issue themselves, so a wait there never drains an HBM prefetch.
//   E waves (4-7): everything else. They rotate this slice's share of a future block
//     into the shared ring, stage V^T for the next block, sum the four partial outputs
//     of the previous block, publish its GroupNorm statistics, normalise + gate + store
//     the block computed four iterations earlier, and keep the HBM streams (q, k, v,
//     gate) two iterations ahead in registers.
// Two LDS-only barriers per block separate the phases (B1 at the top of an iteration,
// B2 once the E waves have read the partial outputs).
//
// Decay folded into the operands. With j the row of a token inside its block, the
// rotated rows are stored in half as
//     Qt_j = alpha gamma^(j-31) Qh_j,      Kt_j = gamma^(31-j) Kh_j,
// and the state is carried as Sc = gamma^32 S. Then, for a block of L rows,
//     scores   Qt_t . Kt_s  = alpha gamma^(t-s) Qh_t . Kh_s       (causal mask only)
//     cross    Qt_t Sc      = alpha gamma^(t+1) Qh_t S            (xi_t applied)
//     carry    Sc <- gamma^L (Sc + Kt^T V)                        (zeta_s applied)
// which is the chunkwise recurrence with the state update weighted per row by
// gamma^(L-1-s), read off by unrolling the recurrent update over the block. The
// factors gamma^(+-32) bound the operand range; the path requires gamma^32 >= 2^-6.
// Per block and M wave (16x16x32 f16 MFMA, fp32 accumulate):
//   scores  P_w^T = Kt_w Qt_w^T                   (partial over the quarter, 20 MFMA)
//   Kt_w^T  by MFMA against 0/1 selection matrices  (16 MFMA, exact)
//   then per 16-column tile of the slice:
//     cross  acc  = Qt_w Sc_w                     (8 MFMA)
//     intra  acc += P_w V                         (6 MFMA)
//     carry  Sc_w = gamma^L (Sc_w + Kt_w^T V)     (8 MFMA)
// (a column tile's cross term reads its state columns before the carry updates them).
// The output is the sum of the four waves' acc; GroupNorm (+ gate) follows.
//
// Operand precision. q, k, v arrive in bf16; the rotation runs in float32 and every
// MFMA operand is rounded to IEEE half, which keeps 3 more significand bits than bf16
// (bf16 operands put the error after GroupNorm near 2.6e-2 on RetNet-shaped data,
// half keeps it near 4e-3). Operands must stay within half's range (|x| < 65504).
//
// Sharing between the slices of a head. Every slice needs the whole rotated block.
// Each of the nS workgroups rotates 64/nS rows of the block three ahead of the one
// its M waves compute and writes Qt, Kt to a ring of 8 block slots in the workspace;
// per-slot counters, incremented once per E wave after its stores have completed, say
// when a block is whole. GroupNorm statistics (per-row mean and centred sum of squares
// of each slice) go through an 8-slot ring the same way. All slices of a head are
// placed on one XCD (blockIdx mod 8), so the exchange stays in that XCD's L2: shared
// data is read with L1-bypassing (sc1) buffer loads. If the slices turn out to span
// XCDs, the kernel uses agent-scope release/acquire fences. Every wait has a time
// limit that ends the kernel normally and raises an error word in the workspace.
//
// Schedule of iteration i (both roles run iterations 0 .. nb+3, rounded up to a
// multiple of 4; iterations past the end do only what is left of the last blocks):
//   M: wait for its copies; read the fragments of block i; wait for block i+1 to be
//      whole; wait for the statistics of block i-3 and copy them to LDS | B2 | copy
//      block i+1 into its LDS region; poll the counts for the next iteration; compute
//      block i. (The 16 copies per wave are issued after B2: issued before it, their
//      issue, slowed by the HBM streams in the same memory pipeline, held up both
//      roles at the barrier.)
//   E: read the partial outputs of block i-1 | B2 | form its statistics; rotate this
//      slice's rows of block i+3; normalise and gate block i-4; stage V^T of block i+1;
//      then store the statistics, the ring rows and the outputs, issue the loads of
//      blocks i+5 (q, k), i+3 (v) and i-2 (gate), and raise the counts once the ring
//      and statistics stores have completed. (The stores follow the arithmetic: issued
//      right after B2 they wait behind the M waves' copies in the memory pipeline.)
// Ring safety. At iteration i an E wave writes slot (i+3) mod 8 after its M waves saw
// block i+1 whole, which means every slice has finished iteration i-2, so every copy
// of the block previously held in that slot (block i-5, copied at iteration i-6) is
// done. The statistics slot written at iteration i (block i-1) last held block i-9,
// copied at iteration i-6.
#include "rn_device.h"
#include "rn_kernels.h"

namespace rn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;   // 4 M waves + 4 E waves
constexpr int kT = 64;          // tokens per block
constexpr int kDK = 256;        // d_k of this kernel
constexpr int kSl = 64;         // d_v columns per workgroup
constexpr int kRing = 8;        // ring slots (blocks of Qt/Kt)
constexpr int kStatRing = 8;    // statistics slots
constexpr int kAhead = 3;       // blocks produced ahead of the block computed
constexpr int kLag = 4;         // iterations between computing a block and storing it
constexpr int kReanchor = 16;   // blocks between exact (float64-reduced) angle anchors
constexpr int kVtLd = 72;       // LDS row stride (half) of the transposed V slice
constexpr uint32_t kCntWords = 64;             // counter words per head
constexpr size_t kStatsPerHead = size_t(kStatRing) * 8 * kT * 2 * sizeof(float);   // 32 KB
constexpr size_t kSlotElems = size_t(kT) * kDK;                                  // 16384 half
constexpr size_t kRingPerHead = size_t(kRing) * 2 * kSlotElems * sizeof(uint16_t);  // 512 KB
constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz wall clock
// Buffer offset past the end of every range used for stores: the store is dropped
// (it still counts as an issued memory operation, which keeps the waits' counts fixed).
constexpr uint32_t kSink = 0x80000000u;

// Counter words per head. Publication counts are kept per ring slot and in waves:
// slot s counts the waves that published blocks s, s+kRing, s+2kRing, ...; block j is
// complete when word kReady + j%kRing reaches 4*nS*(j/kRing + 1). (A single running
// count per head would not do: a wave that is ahead adds its next publication to the
// same count and can complete it while a slower slice has not yet published the block
// being waited for.) The GroupNorm statistics use kStat + j%kStatRing the same way.
// Words 2-3 form one 64-bit arrival word: each slice adds 1 << (4 x) for its XCD x, so
// nibble x counts the slices on XCD x (at most 8 of a head: no carry between nibbles)
// and the nibbles sum to the slices that have arrived. Words [8, 16) record the XCD of
// each slice (diagnostics).
enum { kArrive = 2, kError = 4, kXccOfSlice = 8, kReady = 16, kStat = 24 };

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

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum over each group of 8 lanes, every lane receiving the group's sum, with DPP moves
// (VALU only): swap neighbours, swap pairs, mirror within 8 lanes.
__device__ __forceinline__ float row8_sum(float x) {
  x += dpp_mov<0xB1>(x);    // lane ^ 1
  x += dpp_mov<0x4E>(x);    // lane ^ 2
  x += dpp_mov<0x141>(x);   // lane i <-> 7 - i within 8
  return x;
}

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID (id 20), bits [3:0]
  return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xf;
}

// Order of the 64 keys of a block inside a row of V^T: key s = 32e + 16h + 4g + r
// (e, h in {0,1}; g, r in [0,4)) sits at position 32e + 8g + 4h + r. Lane group g of
// a 16x16x32 MFMA then finds its 8 k-values (keys 32e + 4g + {0..3} and
// 32e + 16 + 4g + {0..3}) in 16 contiguous bytes, which are also the 8 values a lane
// holds after a transposed product (two 16x16 tiles, four consecutive rows each).
__device__ __forceinline__ constexpr int vt_pos(int s) {
  return 32 * (s >> 5) + 8 * ((s >> 2) & 3) + 4 * ((s >> 4) & 1) + (s & 3);
}

// Swizzle of the reduction buffer: column c of a wave's partial output keeps its row
// group q (rows 4q..4q+3) at q ^ red_swz(c), so that both the 16-byte writes (16
// consecutive columns, one row group) and the 16-byte reads (columns 4b + cc for 16
// values of b, one row group) touch 16 distinct 4-bank groups.
__device__ __forceinline__ int red_swz(int c) { return ((c >> 2) & 15) ^ ((c & 3) << 2); }

struct alignas(16) Shared {
  float red[4][kSl][kT];             // partial outputs of the M waves: [wave][col][row]
  u32x4 fr[4][16][64];               // the current block's Qt/Kt fragments, per M wave and lane
  uint16_t vt[2][kSl][kVtLd];        // V slice of two blocks, transposed, vt_pos order
  float stat[2][8][kT][2];           // statistics of the block to normalise: [slice][row][mean, M2]
  uint32_t mode;                     // 1 = agent-scope fences
};

// Buffer resource over the whole workspace (the exchange copies read it with sc1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// Buffer resource over [base, base + bytes): loads past the end return 0 and stores
// past the end are dropped, which is how ragged tails, rows past a sequence's length
// and the blocks before the first and after the last one are handled.
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
__device__ __forceinline__ void st_b128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v), r, off, 0, 0);
}
__device__ __forceinline__ void st_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v), r, off, 0, 0);
}
// 16 bytes per lane from the workspace into LDS at dst + 16 * lane, with device scope
// (sc1): the CU's L1 is bypassed, so data another CU has just written to the XCD's L2 is
// seen. (A load with sc0 alone may be served from a stale L1 line on this chip.)
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 16);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8). Issued through the builtin rather than inline assembly so that the
// compiler's own wait insertion sees them and does not wait again for what they cover.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 15));
  __asm__ volatile("" ::: "memory");
}

// Barrier over the workgroup for LDS traffic only: this wave's LDS operations are
// complete, global memory operations may still be in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Bits of the call's status word (first word of the workspace, cleared at the start of
// every call): a wait hit its time limit; an output or the final state is not finite.
constexpr uint32_t kStatusTimeout = kChunkwiseStatusTimeout, kStatusNonFinite = kChunkwiseStatusNonFinite;
constexpr size_t kStatusBytes = 256;   // status region at the start of the workspace

// A wait that hit its time limit: raises the head's error word (every later wait of
// every workgroup of the head then returns at once, so a broken exchange costs one time
// limit, and every workgroup writes NaN outputs at its end) and the call's status word.
__device__ __forceinline__ void raise_timeout(uint32_t* cnt, uint32_t* status) {
  __hip_atomic_fetch_or(cnt + kError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the 16 nibbles of v.
__device__ __forceinline__ uint32_t nibble_sum(uint64_t v) {
  v = (v & 0x0F0F0F0F0F0F0F0Full) + ((v >> 4) & 0x0F0F0F0F0F0F0F0Full);   // byte sums
  return static_cast<uint32_t>((v * 0x0101010101010101ull) >> 56);
}

// Thread 0 waits until nS slices have added to the arrival word, then the block
// synchronises. With `force` (the RN_TEST_FORCE_TIMEOUT flag) the wait gives up at once,
// as if its limit had passed.
__device__ __forceinline__ void wait_arrivals(uint32_t* cnt, uint32_t nS, uint32_t* status, bool force) {
  if (threadIdx.x == 0) {
    uint64_t* p = reinterpret_cast<uint64_t*>(cnt + kArrive);
    if (force) {
      raise_timeout(cnt, status);
    } else if (nibble_sum(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < nS) {
      const uint64_t t0 = wall_clock64();
      while (nibble_sum(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < nS) {
        if (__hip_atomic_load(cnt + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWaitTicks) {
          raise_timeout(cnt, status);
          break;
        }
      }
    }
  }
  __syncthreads();
}

struct Params {
  CallArgs a;
  int head0;       // first (b*H + h) of this launch group
  int heads;       // heads in this group
  int nS;          // slices per head
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;
  const float* s_in;
  float* s_out;
  void* out;
  uint8_t* ws;          // this launch group's counters, statistics and ring
  uint32_t* status;     // the call's status word
};

template <int C> struct Ic { static constexpr int value = C; };

template <int OUT, int NS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
chunkwise_fused(Params P) {
  const CallArgs& a = P.a;
  const int xcd = blockIdx.x & 7, L8 = blockIdx.x >> 3;
  const int hg = (L8 / NS) * 8 + xcd;    // head within the launch group
  if (hg >= P.heads) return;
  const int sl = L8 % NS;                // d_v slice
  constexpr int nS = NS;
  const int bh = P.head0 + hg;
  const int h = bh % a.H;
  const int N = a.N, DV = a.dv;          // N: row stride of the padded layout
  const int len = seq_len(a, bh / a.H);  // tokens of this sequence
  const int nb = (len + kT - 1) / kT;    // blocks of 64 tokens
  // iterations: the E waves store block nb-1 at iteration nb-1+kLag; the count is
  // rounded up to a multiple of 4 (the E waves' loop body holds four iterations)
  const int n_iter = (nb + kLag + 3) & ~3;
  const int tid = threadIdx.x, l = tid & 63, l16 = l & 15, g = l >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)

  __shared__ Shared sm;

  // workspace views
  uint32_t* cnt = reinterpret_cast<uint32_t*>(P.ws) + size_t(hg) * kCntWords;
  uint8_t* stats_base = P.ws + size_t(P.heads) * kCntWords * 4;
  uint8_t* ring_base = stats_base + size_t(P.heads) * kStatsPerHead;
  const __amdgpu_buffer_rsrc_t wsr = ws_rsrc(P.ws);
  const uint32_t ring_off = static_cast<uint32_t>((ring_base - P.ws) + size_t(hg) * kRingPerHead);
  const uint32_t stats_off = static_cast<uint32_t>((stats_base - P.ws) + size_t(hg) * kStatsPerHead);

  // ---- placement check: are all slices of this head on one XCD? ----------------
  // One atomic per slice carries both its arrival and its XCD, so no fence is needed
  // between the two (a device-scope fence here writes back the XCD's L2, which the
  // previous call has filled with dirty lines: about 18 us per call).
  if (tid == 0) {
    const uint32_t x = xcc_id();
    __hip_atomic_store(cnt + kXccOfSlice + sl, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(cnt + kArrive), uint64_t(1) << (4 * x),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_arrivals(cnt, nS, P.status, (a.flags & RN_TEST_FORCE_TIMEOUT) != 0);
  if (tid == 0) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(cnt + kArrive), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    bool one = false;   // every slice on one XCD: one nibble holds them all
#pragma unroll
    for (int x = 0; x < 16; ++x) one |= ((v >> (4 * x)) & 15u) == uint64_t(nS);
    sm.mode = one ? 0u : 1u;
  }
  __syncthreads();
  const bool agent = sm.mode != 0;

  const float lg = a.hp.log2g[h];
  const bool use_gn = a.flags & RN_EPI_GN;
  const uint32_t nW = 4u * uint32_t(nS);   // publishing (E) waves per head
  auto ready_target = [&](int b) { return nW * uint32_t(b / kRing + 1); };
  auto stat_target = [&](int b) { return nW * uint32_t(b / kStatRing + 1); };

  if (wv < 4) {
    // =============================== M waves ===========================================
    const int w = wv;
    // Issues a read of a count (every lane reads the same word, so the load is
    // unconditional); `settle` later waits until it reaches `target`.
    auto poll = [&](int word) -> uint32_t {
      return __hip_atomic_load(cnt + word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
            if (l == 0) raise_timeout(cnt, P.status);
            break;
          }
        }
      }
      if (agent) __atomic_thread_fence(__ATOMIC_ACQUIRE);
      __asm__ volatile("" ::: "memory");
    };
    // The fragments of block b are copied from the ring straight into this wave's LDS
    // region: fragment f of lane l lands at fr[w][f][l], Qt (m, c) -> f = 2m + c,
    // Kt (i, c) -> f = 8 + 2i + c; lane l holds row 16m + l16 (16i + l16), d_k
    // 64w + 32c + 8g .. +8.
    auto stage_frags = [&](int b) {
      const uint32_t so = ring_off + static_cast<uint32_t>((b & (kRing - 1)) * 2 * kSlotElems * sizeof(uint16_t));
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t o = static_cast<uint32_t>(((16 * m + l16) * kDK + 64 * w + 32 * c + 8 * g) * 2);
          copy_to_lds(wsr, &sm.fr[w][2 * m + c][0], so + o);
          copy_to_lds(wsr, &sm.fr[w][8 + 2 * m + c][0], so + static_cast<uint32_t>(kSlotElems * 2) + o);
        }
    };
    // Statistics slot of block b (every slice's 64 rows) -> sm.stat[buf]: 4 KB, one
    // 16-byte piece per lane of the four M waves.
    auto stage_stats = [&](int b, int buf) {
      const uint32_t so = stats_off + static_cast<uint32_t>(((b & (kStatRing - 1)) * 8 * kT * 2) * sizeof(float));
      copy_to_lds(wsr, reinterpret_cast<uint8_t*>(&sm.stat[buf][0][0][0]) + 1024 * w,
                  so + static_cast<uint32_t>(1024 * w + 16 * l));
    };

    // 0/1 selection matrices (B operand) for the MFMA transpose of Kt: column n of
    // E_hh picks d_k row 8(n>>2) + 4hh + (n&3) of a 32-wide chunk.
    f16x8 E[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        E[hh][jj] = (g == (l16 >> 2) && jj == 4 * hh + (l16 & 3)) ? _Float16(1.0f) : _Float16(0.0f);

    // state: Sc_w tiles [ta][tb], ta = d_k tile (permuted rows), tb = d_v tile;
    // accumulator row 4g+r of tile ta = 2c+hh holds d_k = 64w + 32c + 8g + 4hh + r
    const float g32 = exp2f(lg * 32.f);
    f32x4 Sacc[4][4];
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int dk = 64 * w + 32 * (ta >> 1) + 8 * g + 4 * (ta & 1) + r;
          const int dv = sl * kSl + 16 * tb + l16;
          Sacc[ta][tb][r] = P.s_in ? g32 * P.s_in[(size_t(bh) * kDK + dk) * DV + dv] : 0.f;
        }

    // prologue: block 0 (published by the E waves' prologue) copied in
    uint32_t poll_r = 0u, poll_s = 0u;
    if (nb > 0) settle(poll(kReady + 0), kReady + 0, ready_target(0));
    stage_frags(0);
    poll_r = poll(kReady + 1);

    for (int i = 0; i < n_iter; ++i) {
      lds_barrier();   // B1
      // copies of the previous iteration (fragments of block i, statistics of block
      // i-4) and the polled counts are complete
      wait_vm<0>();
      u32x4 q[4][2], k[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          q[m][c] = sm.fr[w][2 * m + c][l];
          k[m][c] = sm.fr[w][8 + 2 * m + c][l];
        }
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
      __asm__ volatile("" ::: "memory");
      // block i+1 into the fragment region just read; statistics of block i-3
      if (i + 1 < nb) settle(poll_r, kReady + (i + 1) % kRing, ready_target(i + 1));
      if (use_gn && i >= 3 && i - 3 < nb) settle(poll_s, kStat + (i - 3) % kStatRing, stat_target(i - 3));
      stage_stats(i - 3, i & 1);
      lds_barrier();   // B2: the E waves have read the partial outputs of block i-1
      // block i+1 into the fragment region read at the top (its copies then have this
      // iteration's matrix work to complete in, and do not hold up the barrier)
      stage_frags(i + 1);
      // counts for the next iteration: block i+2 whole, statistics of block i-2
      poll_r = poll(kReady + (i + 2) % kRing);
      poll_s = poll(kStat + ((i - 2) & (kStatRing - 1)));
      if (i >= nb) continue;

      const int vb = i & 1;
      // scores P^T tiles (i, m), i <= m, partial over this wave's quarter of d_k:
      // D row s = 16i + 4g + r, column t = 16m + l16
      f16x8 pf[4][2];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 pt[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          pt[ii] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (ii > m) continue;
          f32x4 z = mfma(as_f16x8(k[ii][0]), as_f16x8(q[m][0]), pt[ii]);
          z = mfma(as_f16x8(k[ii][1]), as_f16x8(q[m][1]), z);
          if (ii == m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) z[r] = (4 * g + r <= l16) ? z[r] : 0.f;
          }
          pt[ii] = z;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          u32x4 u;
          u[0] = pack_f16x2(pt[2 * e][0], pt[2 * e][1]);
          u[1] = pack_f16x2(pt[2 * e][2], pt[2 * e][3]);
          u[2] = pack_f16x2(pt[2 * e + 1][0], pt[2 * e + 1][1]);
          u[3] = pack_f16x2(pt[2 * e + 1][2], pt[2 * e + 1][3]);
          pf[m][e] = as_f16x8(u);
        }
      }
      // Kt^T of this quarter as the carry's A operand (row d_k, k = keys in vt_pos
      // order): tile ta = 2c + hh from Kt rows 16i.. times E_hh
      f16x8 ktf[4][2];
#pragma unroll
      for (int ta = 0; ta < 4; ++ta) {
        f32x4 T[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          T[ii] = mfma(as_f16x8(k[ii][ta >> 1]), E[ta & 1], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          u32x4 u;
          u[0] = pack_f16x2(T[2 * e][0], T[2 * e][1]);
          u[1] = pack_f16x2(T[2 * e][2], T[2 * e][3]);
          u[2] = pack_f16x2(T[2 * e + 1][0], T[2 * e + 1][1]);
          u[3] = pack_f16x2(T[2 * e + 1][2], T[2 * e + 1][3]);
          ktf[ta][e] = as_f16x8(u);
        }
      }
      const float gL = exp2f(lg * float(min(kT, len - i * kT)));
      // per 16-column tile: cross term from the old state, intra term, partial output
      // to LDS, then the carry of that tile's state columns
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f16x8 sf[2], vf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 u;
          u[0] = pack_f16x2(Sacc[2 * c][tb][0], Sacc[2 * c][tb][1]);
          u[1] = pack_f16x2(Sacc[2 * c][tb][2], Sacc[2 * c][tb][3]);
          u[2] = pack_f16x2(Sacc[2 * c + 1][tb][0], Sacc[2 * c + 1][tb][1]);
          u[3] = pack_f16x2(Sacc[2 * c + 1][tb][2], Sacc[2 * c + 1][tb][3]);
          sf[c] = as_f16x8(u);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
          vf[e] = as_f16x8(*reinterpret_cast<const u32x4*>(&sm.vt[vb][16 * tb + l16][32 * e + 8 * g]));
        const int col = 16 * tb + l16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 acc = mfma(as_f16x8(q[m][0]), sf[0], f32x4{0.f, 0.f, 0.f, 0.f});
          acc = mfma(as_f16x8(q[m][1]), sf[1], acc);
          acc = mfma(pf[m][0], vf[0], acc);
          if (m >= 2) acc = mfma(pf[m][1], vf[1], acc);
          *reinterpret_cast<f32x4*>(&sm.red[w][col][4 * ((4 * m + g) ^ red_swz(col))]) = acc;
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
          f32x4 z = mfma(ktf[ta][0], vf[0], Sacc[ta][tb]);
          z = mfma(ktf[ta][1], vf[1], z);
          Sacc[ta][tb] = z * gL;
        }
      }
    }

    // A wait of this head that hit its time limit leaves the exchange, hence the
    // state, invalid: the slice's final state is then written as NaN.
    const bool failed = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(cnt + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0u;
    if (P.s_out) {
      const float gi32 = exp2f(-lg * 32.f);
      uint32_t bad = 0u;   // set by a non-finite state value
#pragma unroll
      for (int ta = 0; ta < 4; ++ta)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int dk = 64 * w + 32 * (ta >> 1) + 8 * g + 4 * (ta & 1) + r;
            const int dv = sl * kSl + 16 * tb + l16;
            const float x = Sacc[ta][tb][r] * gi32;
            bad |= __builtin_isfinite(x) ? 0u : 1u;
            P.s_out[(size_t(bh) * kDK + dk) * DV + dv] = failed ? __builtin_nanf("") : x;
          }
      if (__builtin_amdgcn_ballot_w64(bad != 0u) != 0 && l == 0)
        __hip_atomic_fetch_or(P.status, kStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    // =============================== E waves ===========================================
    const int te = tid - 256;   // 0..255
    const float alpha = a.alpha;
    const bool has_gate = P.gate != nullptr;
    uint16_t* ring = reinterpret_cast<uint16_t*>(ring_base + size_t(hg) * kRingPerHead);
    float* stats = reinterpret_cast<float*>(stats_base + size_t(hg) * kStatsPerHead);

    // ---- producer: this thread rotates rows r_lo + pr + 8u (u < U) of each block,
    // pairs 4pq..4pq+3 (d_k 8pq..8pq+7), for q and k -------------------------------
    constexpr int rows_per = kT / nS, U = rows_per / 8;
    const int r_lo = sl * rows_per;
    const int pr = te >> 5, pq = te & 31;
    float th[4], c64[4], s64[4], cc[U][4], ss[U][4], fq[U], fk[U];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      th[i] = a.ap.theta[4 * pq + i];
      angle_cs(kT, th[i], &c64[i], &s64[i]);   // once per thread: exact
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r_lo + pr + 8 * u;
      fq[u] = alpha * exp2f(lg * float(row - 31));
      fk[u] = exp2f(lg * float(31 - row));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cc[u][i] = 1.f;
        ss[u][i] = 0.f;
      }
    }
    const int64_t p_row0 = seq_pos0(a, bh / a.H) + r_lo + pr;   // position of row u = 0 in block 0
    const size_t qk_head = size_t(bh) * N * kDK;
    const int64_t qk_bytes = int64_t(len) * kDK * 2;
    const __amdgpu_buffer_rsrc_t r_q = range_rsrc(P.q + qk_head, qk_bytes);
    const __amdgpu_buffer_rsrc_t r_k = range_rsrc(P.k + qk_head, qk_bytes);
    const __amdgpu_buffer_rsrc_t r_ring = range_rsrc(ring, int64_t(kRingPerHead));
    const __amdgpu_buffer_rsrc_t r_stats = range_rsrc(stats, int64_t(kStatsPerHead));
    // raw rows of blocks to produce, two blocks in flight (past the sequence: zeros)
    u32x4 xq[2][U], xk[2][U];
    auto load_raw = [&](int b, u32x4* dq, u32x4* dk) {
      const int bb = b < 0 ? 0 : b;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = static_cast<uint32_t>(((bb * kT + r_lo + pr + 8 * u) * kDK + 8 * pq) * 2);
        dq[u] = ld_b128(r_q, off);
        dk[u] = ld_b128(r_k, off);
      }
    };
    // Rotates and stores this workgroup's rows of block b. Blocks are produced in
    // order; the angles advance by 64 theta per block and are re-anchored from their
    // float64-reduced values every kReanchor blocks.
    auto produce_calc = [&](int b, const u32x4* sq, const u32x4* sk, u32x4* poq, u32x4* pok, uint32_t* pso) {
      const bool anchor = (b % kReanchor) == 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (anchor) {
            angle_cs_fast(p_row0 + int64_t(b) * kT + 8 * u, th[i], &cc[u][i], &ss[u][i]);
          } else {
            const float cn = cc[u][i] * c64[i] - ss[u][i] * s64[i];
            ss[u][i] = cc[u][i] * s64[i] + ss[u][i] * c64[i];
            cc[u][i] = cn;
          }
        }
        u32x4 oq, ok;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float q0 = __uint_as_float(sq[u][i] << 16), q1 = __uint_as_float(sq[u][i] & 0xffff0000u);
          const float k0 = __uint_as_float(sk[u][i] << 16), k1 = __uint_as_float(sk[u][i] & 0xffff0000u);
          const float cq = cc[u][i] * fq[u], sq_ = ss[u][i] * fq[u];
          const float ck = cc[u][i] * fk[u], sk_ = ss[u][i] * fk[u];
          oq[i] = pack_f16x2(q0 * cq - q1 * sq_, q0 * sq_ + q1 * cq);
          ok[i] = pack_f16x2(k0 * ck - k1 * sk_, k0 * sk_ + k1 * ck);
        }
        // (blocks past the last: an offset past the end of the ring, store dropped)
        pso[u] = b < nb ? static_cast<uint32_t>(
            ((size_t(b & (kRing - 1)) * 2 * kSlotElems + size_t(r_lo + pr + 8 * u) * kDK + 8 * pq) * 2))
                        : kSink;
        poq[u] = oq;
        pok[u] = ok;
      }
    };
    auto store_ring = [&](const u32x4* poq, const u32x4* pok, const uint32_t* pso) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        st_b128(r_ring, pso[u], poq[u]);
        st_b128(r_ring, pso[u] + static_cast<uint32_t>(kSlotElems * 2), pok[u]);
      }
    };
    auto produce = [&](int b, const u32x4* sq, const u32x4* sk) {
      u32x4 poq[U], pok[U];
      uint32_t pso[U];
      produce_calc(b, sq, sk, poq, pok, pso);
      store_ring(poq, pok, pso);
    };

    // V slice: thread loads rows vs0..vs0+3, columns vd0..vd0+3 (bf16) of the slice
    // to the end of the sequence's last row (rows past it read as zeros, stores dropped)
    const int64_t slice_bytes = max(int64_t(len) * DV - sl * kSl, int64_t(0)) * 2;
    const size_t slice0 = size_t(bh) * N * DV + sl * kSl;
    const __amdgpu_buffer_rsrc_t r_v = range_rsrc(P.v + slice0, slice_bytes);
    const __amdgpu_buffer_rsrc_t r_g = range_rsrc(has_gate ? P.gate + slice0 : P.v + slice0, slice_bytes);
    const int osz = (OUT == RN_BF16) ? 2 : 4;
    const __amdgpu_buffer_rsrc_t r_o =
        range_rsrc(static_cast<uint8_t*>(P.out) + slice0 * osz, slice_bytes / 2 * osz);
    const int vs0 = 4 * (te >> 4), vd0 = 4 * (te & 15);
    auto load_v = [&](int b, u32x2* rv) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rv[i] = ld_b64(r_v, static_cast<uint32_t>(((b * kT + vs0 + i) * DV + vd0) * 2));
    };
    auto stage_v = [&](int buf, const u32x2* rv) {
      float fv[4][4];   // [row i][column jj]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fv[i][0] = __uint_as_float(rv[i][0] << 16);
        fv[i][1] = __uint_as_float(rv[i][0] & 0xffff0000u);
        fv[i][2] = __uint_as_float(rv[i][1] << 16);
        fv[i][3] = __uint_as_float(rv[i][1] & 0xffff0000u);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<u32x2*>(&sm.vt[buf][vd0 + jj][vt_pos(vs0)]) =
            u32x2{pack_f16x2(fv[0][jj], fv[1][jj]), pack_f16x2(fv[2][jj], fv[3][jj])};
    };

    // ---- epilogue mapping: thread (ea, eb) owns rows 2ea, 2ea+1 and columns
    // 8eb..8eb+7, so that gate rows and bf16 output rows move in 16-byte pieces ----
    const int ea = te >> 3, eb = te & 7;
    float gw[8], gbias[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = h * DV + sl * kSl + 8 * eb + c;
      gw[c] = a.gn_w ? a.gn_w[col] : 1.f;
      gbias[c] = a.gn_b ? a.gn_b[col] : 0.f;
    }
    // gate rows of block b (reads v when there is no gate: unused; before the first
    // block: an offset past the end, so zeros)
    auto load_gate = [&](int b, u32x4* gt) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        gt[rr] = ld_b128(r_g, static_cast<uint32_t>(((b * kT + 2 * ea + rr) * DV + 8 * eb) * 2));
    };
    // Normalises block b with the statistics of all slices in sm.stat[sbuf] (lane
    // eb < nS reads slice eb's mean and M2 of rows 2ea, 2ea+1), gates and stores
    // (blocks outside the sequence: offsets past the end, stores dropped).
    const float inv_dv = 1.0f / float(DV);
    uint32_t nonfinite = 0u;   // set by a non-finite output of the sequence
    constexpr int kOutPieces = (OUT == RN_BF16) ? 2 : 4;   // 16-byte output pieces per thread
    auto finalize_calc = [&](int b, const float (*o)[8], const u32x4* gt, int sbuf, u32x4* fo, uint32_t* foff) {
      float y[2][8];
      if (use_gn) {
        const u32x4 st = *reinterpret_cast<const u32x4*>(&sm.stat[sbuf][eb][2 * ea][0]);
        const bool mine = eb < nS;
        // equal counts per slice: mean = average of the slice means,
        // M2 = sum M2_s + 64 sum (mean_s - mean)^2 (Chan et al.)
        const float inv_nS = 1.0f / float(nS);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const float mu_s = mine ? __uint_as_float(st[2 * rr]) : 0.f;
          const float m2_s = mine ? __uint_as_float(st[2 * rr + 1]) : 0.f;
          const float mu = row8_sum(mu_s) * inv_nS;
          const float d = mu_s - mu;
          const float m2 = row8_sum(mine ? fmaf(float(kSl) * d, d, m2_s) : 0.f);
          const float rstd = __frsqrt_rn(fmaf(m2, inv_dv, a.eps));
#pragma unroll
          for (int c = 0; c < 8; ++c) y[rr][c] = fmaf((o[rr][c] - mu) * rstd, gw[c], gbias[c]);
          if (has_gate) {
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) {
              y[rr][2 * c2] *= swishf(__uint_as_float(gt[rr][c2] << 16));
              y[rr][2 * c2 + 1] *= swishf(__uint_as_float(gt[rr][c2] & 0xffff0000u));
            }
          }
        }
      } else {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int c = 0; c < 8; ++c) y[rr][c] = o[rr][c];
      }
      {
        // (a class test per value: x - x would not do, since the compiler may contract
        // the product that forms x with the subtraction, leaving its rounding error)
        uint32_t bad = 0u;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int c = 0; c < 8; ++c) bad |= __builtin_isfinite(y[rr][c]) ? 0u : 1u;
        nonfinite |= (b >= 0 && b < nb) ? bad : 0u;
      }
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        foff[rr] = static_cast<uint32_t>(((b * kT + 2 * ea + rr) * DV + 8 * eb) * osz);
        if constexpr (OUT == RN_BF16) {
          fo[rr] = u32x4{pack_bf16x2(y[rr][0], y[rr][1]), pack_bf16x2(y[rr][2], y[rr][3]),
                         pack_bf16x2(y[rr][4], y[rr][5]), pack_bf16x2(y[rr][6], y[rr][7])};
        } else {
          fo[2 * rr] = __builtin_bit_cast(u32x4, f32x4{y[rr][0], y[rr][1], y[rr][2], y[rr][3]});
          fo[2 * rr + 1] = __builtin_bit_cast(u32x4, f32x4{y[rr][4], y[rr][5], y[rr][6], y[rr][7]});
        }
      }
    };
    auto store_out = [&](const u32x4* fo, const uint32_t* foff) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        if constexpr (OUT == RN_BF16) {
          st_b128(r_o, foff[rr], fo[rr]);
        } else {
          st_b128(r_o, foff[rr], fo[2 * rr]);
          st_b128(r_o, foff[rr] + 16, fo[2 * rr + 1]);
        }
      }
    };

    // Makes this wave's ring and statistics stores complete, then raises the counts.
    // Vector memory operations of a wave complete in issue order; the last kTail
    // operations issued (2 output stores, 4 for float32 output; 2U raw loads, 4 v loads,
    // 2 gate loads) need not be waited for. Every iteration issues the same operations (stores
    // that fall outside the sequence go to a dropped offset), so the count is fixed.
    constexpr int kTail = (OUT == RN_BF16 ? 2 : 4) + 2 * U + 4 + 2;
    auto release = [&](bool ring_pub, int rb, bool stat_pub, int sb) {
      if (agent) {
        __threadfence();
      } else {
        wait_vm<kTail>();
      }
      if (l == 0) {
        if (ring_pub)
          __hip_atomic_fetch_add(cnt + kReady + rb % kRing, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (stat_pub)
          __hip_atomic_fetch_add(cnt + kStat + sb % kStatRing, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };

    // deferred outputs and gate rows of the blocks awaiting normalisation, by block mod
    // 4; V rows two iterations ahead, by block mod 2
    float ob[4][2][8];
    u32x4 gb[4][2];
    u32x2 vb[2][4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        gb[s][rr] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 8; ++c) ob[s][rr][c] = 0.f;
      }

    // ---- prologue: blocks 0 .. kAhead-1 produced and published, V^T of block 0
    // staged; then the loads the first two iterations consume: q/k rows of blocks 3
    // and 4, V of blocks 1 and 2 (the gate rows they would use belong to blocks before
    // the first, whose outputs are dropped) ---------------------------------------------
    {
      // (all loads first: one memory latency rather than one per block)
      u32x4 tq[kAhead][U], tk[kAhead][U];
#pragma unroll
      for (int b = 0; b < kAhead; ++b) load_raw(b, tq[b], tk[b]);
      load_v(0, vb[0]);
#pragma unroll
      for (int b = 0; b < kAhead; ++b) produce(b, tq[b], tk[b]);
      stage_v(0, vb[0]);
    }
    if (agent) __threadfence();
    else wait_vm<0>();
    if (l == 0) {
      for (int b = 0; b < kAhead && b < nb; ++b)
        __hip_atomic_fetch_add(cnt + kReady + b % kRing, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    load_raw(kAhead, xq[kAhead & 1], xk[kAhead & 1]);
    load_raw(kAhead + 1, xq[(kAhead + 1) & 1], xk[(kAhead + 1) & 1]);
    load_v(1, vb[1]);
    load_v(2, vb[0]);
    // nothing in flight on entry to the loop: its first iteration then waits for
    // exactly what it consumes, as later ones do
    wait_vm<0>();

    // one iteration; C = i mod 4 (compile time)
    auto iter = [&](auto cst, int i) {
      constexpr int C = decltype(cst)::value;
      float o_cur[2][8];
      lds_barrier();   // B1
      // (1) partial outputs of block i-1 summed: rows 2ea, 2ea+1 sit in row group ea/2
      // of each column, at offset 2 (ea % 2)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int c = 0; c < 8; ++c) o_cur[rr][c] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = 8 * eb + c;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(
              &sm.red[ww][col][4 * ((ea >> 1) ^ red_swz(col)) + 2 * (ea & 1)]);
          o_cur[0][c] += __uint_as_float(x[0]);
          o_cur[1][c] += __uint_as_float(x[1]);
        }
      }
      lds_barrier();   // B2
      // (2) statistics of block i-1 (per row: mean, centred sum of squares) -> ring
      uint32_t st_so;
      u32x4 st_v;
      {
        float st[4];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          float sum = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) sum += o_cur[rr][c];
          const float mu = row8_sum(sum) * (1.0f / kSl);
          float m2 = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const float d = o_cur[rr][c] - mu;
            m2 = fmaf(d, d, m2);
          }
          st[2 * rr] = mu;
          st[2 * rr + 1] = row8_sum(m2);
        }
        st_so = (i >= 1 && i <= nb) ? static_cast<uint32_t>(
            (((((i - 1) & (kStatRing - 1)) * 8 + sl) * kT + 2 * ea) * 2) * sizeof(float)) : kSink;
        st_v = __builtin_bit_cast(u32x4, f32x4{st[0], st[1], st[2], st[3]});
      }
      // (3) this workgroup's rows of block i+3 for the ring (raw rows loaded at i-2)
      u32x4 poq[U], pok[U];
      uint32_t pso[U];
      produce_calc(i + kAhead, xq[(C + kAhead) & 1], xk[(C + kAhead) & 1], poq, pok, pso);
      // (4) block i-4: normalise, gate (statistics copied by the M waves at i-1)
      u32x4 fo[kOutPieces];
      uint32_t foff[2];
      finalize_calc(i - kLag, ob[C], gb[C], (i - 1) & 1, fo, foff);
      // (5) V^T of block i+1 (loaded at i-2)
      stage_v((C + 1) & 1, vb[(C + 1) & 1]);
      // (5b) the stores, after the arithmetic: issued right after B2 they would wait
      // behind the M waves' fragment copies in the memory pipeline
      st_b128(r_stats, st_so, st_v);
      store_ring(poq, pok, pso);
      store_out(fo, foff);
      __asm__ volatile("" ::: "memory");
      // (6) prefetches: q/k rows of block i+5, V of block i+3, gate of block i-2
      load_raw(i + kAhead + 2, xq[(C + kAhead) & 1], xk[(C + kAhead) & 1]);
      load_v(i + 3, vb[(C + 3) & 1]);
      load_gate(i - 2, gb[(C + 2) & 3]);
      // (7) keep block i-1's outputs for its normalisation at i+3
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int c = 0; c < 8; ++c) ob[(C + 3) & 3][rr][c] = o_cur[rr][c];
      // (8) publish the ring rows of block i+3 and the statistics of block i-1
      release(i + kAhead < nb, i + kAhead, use_gn && i >= 1 && i <= nb, i - 1);
    };
    for (int i0 = 0; i0 < n_iter; i0 += 4) {
      iter(Ic<0>{}, i0);
      iter(Ic<1>{}, i0 + 1);
      iter(Ic<2>{}, i0 + 2);
      iter(Ic<3>{}, i0 + 3);
    }
    if (__builtin_amdgcn_ballot_w64(nonfinite != 0u) != 0 && l == 0)
      __hip_atomic_fetch_or(P.status, kStatusNonFinite, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // A wait of this head that hit its time limit leaves the exchange invalid: every row
    // this thread stored is written again as NaN (same thread, same addresses, so the
    // NaN stores land after the earlier ones).
    if (__builtin_amdgcn_readfirstlane(
            __hip_atomic_load(cnt + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0u) {
      const float qn = __builtin_nanf("");
      for (int b = 0; b < nb; ++b)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const uint32_t ooff = static_cast<uint32_t>(((b * kT + 2 * ea + rr) * DV + 8 * eb) * osz);
          if constexpr (OUT == RN_BF16) {
            const uint32_t nn = pack_bf16x2(qn, qn);
            st_b128(r_o, ooff, u32x4{nn, nn, nn, nn});
          } else {
            const u32x4 nn = __builtin_bit_cast(u32x4, f32x4{qn, qn, qn, qn});
            st_b128(r_o, ooff, nn);
            st_b128(r_o, ooff + 16, nn);
          }
        }
    }
  }
}

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

const void* kernel_for(int out_dt, int nS) {
#define RN_CW_CASE(NS_)                                                                  \
  case NS_:                                                                              \
    return out_dt == RN_BF16 ? reinterpret_cast<const void*>(&chunkwise_fused<RN_BF16, NS_>) \
                             : reinterpret_cast<const void*>(&chunkwise_fused<RN_F32, NS_>);
  switch (nS) {
    RN_CW_CASE(1)
    RN_CW_CASE(2)
    RN_CW_CASE(4)
    RN_CW_CASE(8)
  }
#undef RN_CW_CASE
  return nullptr;
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

// The decay factors gamma^(+-32) folded into the half operands need gamma^32 >= 2^-6.
// Buffer offsets within one head's rows are 32-bit: N d_v (4-byte output) and N d_k
// (2-byte input) must stay below 2^31 bytes.
bool chunkwise_mfma_supported(const CallArgs& a, int in_dt) {
  if (in_dt != RN_BF16 || a.dk != kDK ||
      !(a.dv == 64 || a.dv == 128 || a.dv == 256 || a.dv == 512))
    return false;
  if (int64_t(a.N) * a.dv * 4 >= (int64_t(1) << 31) || int64_t(a.N) * kDK * 2 >= (int64_t(1) << 31))
    return false;
  for (int h = 0; h < a.H; ++h)
    if (!(a.hp.log2g[h] * 32.0f >= -6.0f)) return false;
  return true;
}

size_t chunkwise_mfma_ws_bytes(const CallArgs& a) {
  const int nS = a.dv / kSl;
  int G = heads_per_group(nS);
  if (G <= 0) G = 8 * (256 / (8 * nS));  // no device visible: size for a 256-CU part
  G = min(G, a.B * a.H);
  return kStatusBytes + size_t(G) * (kCntWords * 4 + kStatsPerHead + kRingPerHead);
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
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.gate = static_cast<const uint16_t*>(gate);
  p.s_in = s_in;
  p.s_out = s_out;
  p.out = out;
  // the call's status word first, then the launch group's counters, statistics and ring
  p.status = static_cast<uint32_t*>(ws);
  p.ws = static_cast<uint8_t*>(ws) + kStatusBytes;
  for (int h0 = 0; h0 < total; h0 += G) {
    const int heads = min(G, total - h0);
    if (kStatusBytes + size_t(heads) * (kCntWords * 4 + kStatsPerHead + kRingPerHead) > ws_bytes)
      return hipErrorInvalidValue;
    p.head0 = h0;
    p.heads = heads;
    // the first group also clears the status word (which later groups only raise)
    const int first = h0 == 0 ? int(kStatusBytes / 4) : 0;
    const int nwords = first + heads * int(kCntWords);
    hipLaunchKernelGGL(zero_words, dim3((nwords + 255) / 256), dim3(256), 0, st,
                       reinterpret_cast<uint32_t*>(p.ws) - first, nwords);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int grid = 8 * nS * ((heads + 7) / 8);
    void* args[] = {&p};
    e = hipLaunchCooperativeKernel(kernel_for(out_dt, nS), dim3(grid), dim3(kThreads), args, 0, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rn
