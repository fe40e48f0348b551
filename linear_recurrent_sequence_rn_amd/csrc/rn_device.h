// Device helpers shared by the retention kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rn_retention.h"

namespace rn {

constexpr int kMaxDk = 256;
constexpr int kMaxDv = 512;
constexpr int kMaxHeads = 128;   // per-head decay travels in the kernel argument block

// Per-call parameters that every kernel reads from its argument block. The decay
// and angle arrays are copied by value (they are host arrays in the ABI).
struct HeadParams {
  float gamma[kMaxHeads];     // per-head decay
  float log2g[kMaxHeads];     // log2(gamma), formed in float64 on the host
};
struct AngleParams {
  float theta[kMaxDk / 2];    // one angle per coordinate pair
};

// ---- bf16 / f32 element access --------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
// Round-to-nearest-even float32 -> bfloat16 (hardware v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

template <int DT> struct Elem;
template <> struct Elem<RN_F32> {
  __device__ static __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};
template <> struct Elem<RN_BF16> {
  __device__ static __forceinline__ float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
  }
};

// ---- rotation angle -------------------------------------------------------------------
// cos/sin of p*theta. The product is formed in float64 and reduced modulo 2*pi with a
// two-term Cody–Waite split of 2*pi, so the float32 sincos sees |r| <= pi with an
// absolute error near 1e-12 even at positions ~1e6 (a float32 product p*theta would
// already be off by ~4e-3 rad at p = 65536).
__device__ __forceinline__ void angle_cs(int64_t p, float theta, float* c, float* s) {
  const double kTwoPiHi = 6.283185307179586232;        // nearest double to 2*pi
  const double kTwoPiLo = 2.4492935982947064e-16;      // 2*pi - kTwoPiHi
  const double kInvTwoPi = 0.15915494309189535;
  double a = static_cast<double>(p) * static_cast<double>(theta);
  double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  sincosf(static_cast<float>(r), s, c);
}

// Same reduction, then the hardware sine/cosine (absolute error near 1e-6 on the
// reduced range [-pi, pi]): for paths whose operands are rounded to half anyway.
__device__ __forceinline__ void angle_cs_fast(int64_t p, float theta, float* c, float* s) {
  const double kTwoPiHi = 6.283185307179586232;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double kInvTwoPi = 0.15915494309189535;
  double a = static_cast<double>(p) * static_cast<double>(theta);
  double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  const float rf = static_cast<float>(r);
  *s = __sinf(rf);
  *c = __cosf(rf);
}

// gamma^n for a non-negative (possibly fractional) exponent, exact 1 at n = 0 and for
// gamma = 1 (log2g = 0).
__device__ __forceinline__ float gpow(float log2g, float n) {
  return exp2f(log2g * n);
}

// ---- reductions ------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// swish(g) = g * sigmoid(g), with the hardware exp2 and reciprocal (about 3e-7 relative)
__device__ __forceinline__ float swishf(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

}  // namespace rn

namespace rn {

// Scalars of one call, passed by value to every kernel.
struct CallArgs {
  int32_t B, H, N, dk, dv;
  int32_t chunk;
  int64_t pos0;
  float alpha;
  float eps;
  uint32_t flags;
  const float* gn_w;   // device [H*dv] or null
  const float* gn_b;   // device [H*dv] or null
  const int64_t* pos;  // device [B]: position of each sequence's token 0, or null (pos0)
  const int32_t* lens; // device [B]: tokens of each sequence, or null (N)
  const float* gpair;  // device [H * dk/2]: one decay per (head, coordinate pair), or null
  HeadParams hp;
  AngleParams ap;
};

// log2 of the decay of coordinate pair j of head h: the pair's own decay when the call
// gives one per pair (log2 formed in float64, as the host does for the per-head decay),
// else the head's.
__device__ __forceinline__ float pair_log2g(const CallArgs& a, int h, int j) {
  if (a.gpair) return static_cast<float>(log2(static_cast<double>(a.gpair[h * (a.dk / 2) + j])));
  return a.hp.log2g[h];
}
__device__ __forceinline__ float pair_gamma(const CallArgs& a, int h, int j) {
  return a.gpair ? a.gpair[h * (a.dk / 2) + j] : a.hp.gamma[h];
}

// Absolute position of token 0 of sequence b.
__device__ __forceinline__ int64_t seq_pos0(const CallArgs& a, int b) {
  return a.pos ? a.pos[b] : a.pos0;
}
// Tokens of sequence b, clamped to [0, N] (the rows of the padded layout), so that a
// length out of range can never move an access outside the caller's buffers.
__device__ __forceinline__ int seq_len(const CallArgs& a, int b) {
  return a.lens ? min(max(a.lens[b], 0), a.N) : a.N;
}

// Sum over a block of NT threads (NT/64 waves). `red` is NT/64 floats of LDS; every
// thread receives the total. Ends with the LDS slots free for reuse after a barrier.
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}
__device__ __forceinline__ float block_sum256(float x, float* red) { return block_sum<256>(x, red); }

// GroupNorm (+ swish gate) epilogue of one row of d_v values held in LDS `o`
// (float32), computed by a block of NT threads and stored at out[row_off + c].
// Statistics: mean, then the biased variance of (o - mean), eps inside the root.
template <int IN, int OUT, int NT = 256>
__device__ __forceinline__ void row_epilogue(const float* o, int dv, const CallArgs& a,
                                             int head, const void* gate, int64_t row_off,
                                             void* out, float* red) {
  const bool gn = a.flags & RN_EPI_GN;
  const bool gt = a.flags & RN_EPI_GATE;
  float mean = 0.f, rstd = 1.f;
  if (gn) {
    float s = 0.f;
    for (int c = threadIdx.x; c < dv; c += NT) s += o[c];
    mean = block_sum<NT>(s, red) / dv;
    float s2 = 0.f;
    for (int c = threadIdx.x; c < dv; c += NT) { float d = o[c] - mean; s2 += d * d; }
    float var = block_sum<NT>(s2, red) / dv;
    rstd = 1.0f / sqrtf(var + a.eps);
  }
  for (int c = threadIdx.x; c < dv; c += NT) {
    float y = o[c];
    if (gn) {
      y = (y - mean) * rstd;
      if (a.gn_w) y *= a.gn_w[head * dv + c];
      if (a.gn_b) y += a.gn_b[head * dv + c];
      if (gt) y *= swishf(Elem<IN>::load(gate, row_off + c));
    }
    Elem<OUT>::store(out, row_off + c, y);
  }
}
template <int IN, int OUT>
__device__ __forceinline__ void row_epilogue256(const float* o, int dv, const CallArgs& a,
                                                int head, const void* gate, int64_t row_off,
                                                void* out, float* red) {
  row_epilogue<IN, OUT, 256>(o, dv, a, head, gate, row_off, out, red);
}

}  // namespace rn
