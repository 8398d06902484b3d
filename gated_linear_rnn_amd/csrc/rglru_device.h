// Device helpers shared by the gfx950 kernels of the RG-LRU temporal branch.
//
// Definitions follow the Griffin model-architecture page: the "Recurrent block" section
// (causal Conv1D of temporal width 4 before the RG-LRU) and the "Real-Gated Linear
// Recurrent Unit (RG-LRU)" section, Eq. (1)-(4), with a = sigma(Lambda), c = 8 and
// a^{c r_t} evaluated in log space.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rglru {

// ------------------------------------------------------------------ element types
typedef uint16_t bf16_t;   // raw bf16 bits; arithmetic is always fp32

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// 16 bytes that this kernel reads exactly once, loaded with the non-temporal hint: a stream
// of such loads keeps more of HBM's read bandwidth than ordinary ones (measured on a plain
// 1 GiB read: ~6.1-6.6 TB/s against ~5.2-5.9 TB/s).  Not for data that is read again soon.
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_once4(const void* p) {
  const f32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// I/O element traits: load/store 4 consecutive channels as fp32.
template <typename IO> struct Io;

template <> struct Io<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float4 load4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ __forceinline__ static void store4(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
  // a store of output that nothing in the kernel reads back, with the non-temporal hint
  __device__ __forceinline__ static void store4_once(float* p, float4 v) {
    __builtin_nontemporal_store(f32x4v_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4v_t*>(p));
  }
  __device__ __forceinline__ static float round(float v) { return v; }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <> struct Io<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float4 load4(const bf16_t* p) {
    uint2 r = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
  __device__ __forceinline__ static void store4(bf16_t* p, float4 v) {
    uint2 r;
    r.x = uint32_t(f2bf(v.x)) | (uint32_t(f2bf(v.y)) << 16);
    r.y = uint32_t(f2bf(v.z)) | (uint32_t(f2bf(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = r;
  }
  __device__ __forceinline__ static void store4_once(bf16_t* p, float4 v) {
    typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
    const u32x2v_t r = {uint32_t(f2bf(v.x)) | (uint32_t(f2bf(v.y)) << 16),
                        uint32_t(f2bf(v.z)) | (uint32_t(f2bf(v.w)) << 16)};
    __builtin_nontemporal_store(r, reinterpret_cast<u32x2v_t*>(p));
  }
  // value after rounding to bf16 (nearest even), as fp32
  __device__ __forceinline__ static float round(float v) { return bf2f(f2bf(v)); }
  __device__ __forceinline__ static float load1(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store1(bf16_t* p, float v) { *p = f2bf(v); }
};

__device__ __forceinline__ float f4get(const float4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}
__device__ __forceinline__ void f4set(float4& v, int j, float s) {
  if (j == 0) v.x = s; else if (j == 1) v.y = s; else if (j == 2) v.z = s; else v.w = s;
}

// ------------------------------------------------------------------ wave halves
// The value of x in lanes 0-31 and in lanes 32-63, side by side in every lane:
// lo[i] = x[i mod 32], hi[i] = x[32 + (i mod 32)].  One gfx950 v_permlane32_swap_b32 with x
// as both operands (a VALU instruction, no LDS round trip as with ds_bpermute).
struct WaveHalves {
  float lo, hi;
};
__device__ __forceinline__ WaveHalves wave_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// ------------------------------------------------------------------ conv (R1)
// fp64 -> bf16, round to nearest even in one step (no intermediate fp32 rounding), returned
// as the fp32 value it represents.  Normal range: the 45 dropped significand bits are
// rounded away on the bit pattern (adding half an ulp minus one plus the lowest kept bit
// carries exactly when the dropped part exceeds half, or equals half with an odd kept part),
// and the result, 8 significant bits, converts to fp32 exactly.  Below 2^-126 bf16 is
// subnormal with a fixed ulp of 2^-133: rounded with rint at that scale.
__device__ __forceinline__ float f64_to_bf16_value(double v) {
  if (!(fabs(v) >= 0x1p-126)) {                     // subnormal range, zero, or NaN
    if (v != v) return __builtin_nanf("");
    return float(rint(v * 0x1p133) * 0x1p-133);
  }
  uint64_t bits = uint64_t(__double_as_longlong(v));
  bits += ((uint64_t(1) << 44) - 1) + ((bits >> 45) & 1);
  bits &= ~((uint64_t(1) << 45) - 1);
  return float(__longlong_as_double((long long)bits));
}

// u = RNE_io(b + w0 x_t + w1 x_{t-1} + w2 x_{t-2} + w3 x_{t-3}), rounded once: the exact sum
// (taken in fp64 in one fixed order, bias then taps 0..3; every product of two fp32 or bf16
// values is exact in fp64, so fma(w, x, acc) is the add of the exact product), rounded once
// to the I/O dtype.  Every kernel that evaluates u uses this, so all of them produce the
// same bits.
__device__ __forceinline__ double conv_sum_f64(float b, float w0, float w1, float w2, float w3,
                                               float x0, float x1, float x2, float x3) {
  double acc = double(b);
  acc = fma(double(w0), double(x0), acc);
  acc = fma(double(w1), double(x1), acc);
  acc = fma(double(w2), double(x2), acc);
  acc = fma(double(w3), double(x3), acc);
  return acc;
}

template <typename IO>
__device__ __forceinline__ float conv_u(float b, float w0, float w1, float w2, float w3,
                                        float x0, float x1, float x2, float x3);

template <>
__device__ __forceinline__ float conv_u<float>(float b, float w0, float w1, float w2, float w3,
                                               float x0, float x1, float x2, float x3) {
  return float(conv_sum_f64(b, w0, w1, w2, w3, x0, x1, x2, x3));
}

// bf16 I/O, mostly in fp32: the fp32 fma chain s (each bf16 product is exact in fp32, so the
// chain only rounds its 4 partial sums) is within 4.01 * 2^-24 * m of the exact sum S, where
// m = |b| + sum |w_k x_k|.  bf16 rounding changes value only at the halfway points between
// bf16 neighbours; the one inside s's bf16 interval has s's top 16 bits and 0x8000 below.
// When s is more than 8 * 2^-24 * m from it, S lies strictly on the same side of it (and no
// other halfway point is nearer than half a bf16 ulp), so RNE_bf16(s) = RNE_bf16(S).  The
// rare sums closer than that (about 2^-12 of them for sums without cancellation) take the
// fp64 sum and its one rounding instead.
template <>
__device__ __forceinline__ float conv_u<bf16_t>(float b, float w0, float w1, float w2, float w3,
                                                float x0, float x1, float x2, float x3) {
  float s = fmaf(w0, x0, b);
  s = fmaf(w1, x1, s);
  s = fmaf(w2, x2, s);
  s = fmaf(w3, x3, s);
  float m = fmaf(fabsf(w0), fabsf(x0), fabsf(b));
  m = fmaf(fabsf(w1), fabsf(x1), m);
  m = fmaf(fabsf(w2), fabsf(x2), m);
  m = fmaf(fabsf(w3), fabsf(x3), m);
  const float mid = __uint_as_float((__float_as_uint(s) & 0xffff0000u) | 0x8000u);
  if (__builtin_expect(fabsf(s - mid) > m * 0x1p-21f, 1))   // s - mid is exact (one binade)
    return Io<bf16_t>::round(s);
  return f64_to_bf16_value(conv_sum_f64(b, w0, w1, w2, w3, x0, x1, x2, x3));
}

// ------------------------------------------------------------------ GeLU
// GeLU(q) = q Phi(q) (the exact form).  fp64 (the fp32-I/O paths): through the
// complementary error function, Phi(q) = erfc(-q / sqrt 2) / 2, which keeps its relative
// accuracy in the lower tail where 1 + erf(q / sqrt 2) would cancel.
__device__ __forceinline__ double gelu_d(double q) { return 0.5 * q * erfc(-0.70710678118654752440 * q); }
// fp32 for the bf16 epilogues: Phi(-|q|) = erfc(x) / 2, x = |q| / sqrt 2, with erfc from the
// rational approximation of Abramowitz and Stegun (Handbook of Mathematical Functions,
// formula 7.1.26): erfc(x) ~ (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^{-x^2},
// t = 1 / (1 + p x), absolute error <= 1.5e-7 for x >= 0 (about 3e-7 on Phi in fp32 here,
// far below the bf16 rounding of the result); one reciprocal and one exp2 instead of the
// library erfc, which dominated the epilogues that apply it.
__device__ __forceinline__ float gelu_fast(float q) {
  const float x = fabsf(q) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float tail = 0.5f * poly * __builtin_amdgcn_exp2f(-(x * x) * 1.4426950408889634f);  // Phi(-|q|)
  return q * (q >= 0.f ? 1.f - tail : tail);
}

// ------------------------------------------------------------------ gate math
__device__ __forceinline__ float sigmoidf_stable(float z) {
  if (z >= 0.f) return 1.f / (1.f + expf(-z));
  float e = expf(z);
  return e / (1.f + e);
}

// log sigma(Lambda) = -log(1 + e^{-Lambda}), without overflow or cancellation.
__device__ __forceinline__ float log_sigmoidf(float lam) {
  float t = log1pf(expf(-fabsf(lam)));
  return lam >= 0.f ? -t : lam - t;
}

// sigma(-Lambda) = 1 - sigma(Lambda): derivative of log sigma(Lambda).
__device__ __forceinline__ float sigmoid_negf(float lam) { return sigmoidf_stable(-lam); }

// Eq. (3) in log space and the sqrt(1 - a^2) factor of Eq. (4):
//   log a = c r L,  a = exp(log a),  m = sqrt(-expm1(2 log a)).
struct Gate {
  float r, i, a, m;
};
__device__ __forceinline__ Gate gate_from_ri(float r, float i, float L, float c) {
  Gate g;
  g.r = r;
  g.i = i;
  float ell = (c * r) * L;
  g.a = expf(ell);
  g.m = sqrtf(-expm1f(2.f * ell));
  return g;
}

// a_t and m_t = sqrt(1 - a_t^2) of Eq. (3)-(4) from r_t in the precision of a scan state:
// fp32 as above, or fp64 for an fp64 state (fp32 I/O), where a_t's fp32 rounding would
// otherwise compound through the recurrence (about one rounding of a per step carried).
// L is log sigma(Lambda) in the same precision.
struct GateAmF { float a, m; };
struct GateAmD { double a, m; };
__device__ __forceinline__ GateAmF gate_am(float r, float L, float c) {
  const Gate g = gate_from_ri(r, 0.f, L, c);
  return {g.a, g.m};
}
__device__ __forceinline__ GateAmD gate_am(float r, double L, float c) {
  const double ell = (double(c) * double(r)) * L;
  return {exp(ell), sqrt(-expm1(2.0 * ell))};
}
__device__ __forceinline__ double log_sigmoid_d(float lam) {
  const double t = log1p(exp(-fabs(double(lam))));
  return lam >= 0.f ? -t : double(lam) - t;
}
template <typename Acc> __device__ __forceinline__ Acc log_sigmoid_acc(float lam);
template <> __device__ __forceinline__ float log_sigmoid_acc<float>(float lam) { return log_sigmoidf(lam); }
template <> __device__ __forceinline__ double log_sigmoid_acc<double>(float lam) { return log_sigmoid_d(lam); }

// Fast form of the same gate math for the bf16 MFMA epilogue, on the hardware
// transcendentals (v_exp_f32 = 2^x, v_rcp_f32, v_sqrt_f32; about 1 ulp each):
//   sigma(z) = 1 / (1 + 2^(-z log2 e)), with the bias folded into the exp2 argument;
//   log2 a = r * (c log2 sigma(Lambda)),  a = 2^(log2 a);
//   1 - a^2 = -expm1(x), x = 2 ln2 log2 a <= 0: a degree-6 Taylor series of -expm1 for
//   x > -1/4 (truncation below 6e-8 relative), 1 - a*a otherwise (a^2 < 0.78 there, so
//   the difference loses under 2 bits: below 5e-7 relative).
// r = 0 or c = 0 still gives a = 1 and sqrt(1 - a^2) = 0 exactly.
struct GateChan {
  float nba;   // -b_a log2 e
  float nbx;   // -b_x log2 e
  float cl2;   // c log2 sigma(Lambda)
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ GateChan gate_chan(float ba, float bx, float lam, float c) {
  GateChan k;
  k.nba = -ba * kLog2e;
  k.nbx = -bx * kLog2e;
  k.cl2 = c * (log_sigmoidf(lam) * kLog2e);
  return k;
}

// returns a and beta = sqrt(1 - a^2) * i from the accumulated W_a u and W_x u
__device__ __forceinline__ void gate_fast(float za, float zx, const GateChan& k, float& a,
                                          float& beta) {
  const float r = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(za, -kLog2e, k.nba)));
  const float i = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(zx, -kLog2e, k.nbx)));
  const float l2 = r * k.cl2;
  a = __builtin_amdgcn_exp2f(l2);
  const float x = l2 * (2.f * kLn2);
  float q = 1.3888888888888889e-03f;                  // 1/6!
  q = fmaf(q, x, 8.3333333333333333e-03f);            // 1/5!
  q = fmaf(q, x, 4.1666666666666667e-02f);            // 1/4!
  q = fmaf(q, x, 1.6666666666666667e-01f);            // 1/3!
  q = fmaf(q, x, 0.5f);                               // 1/2!
  q = fmaf(q, x, 1.f);
  const float m2 = x > -0.25f ? -x * q : fmaf(-a, a, 1.f);
  beta = __builtin_amdgcn_sqrtf(m2) * i;
}

// r and i only (the backward's recompute)
__device__ __forceinline__ void gate_fast_ri(float za, float zx, const GateChan& k, float& r,
                                             float& i) {
  r = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(za, -kLog2e, k.nba)));
  i = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(zx, -kLog2e, k.nbx)));
}

// ------------------------------------------------------------------ scan look-back
// Chunk summaries of the affine map h -> A h + H are published word by word with
// agent-scope atomics, one word per value: 32-bit words for an fp32 scan state, 64-bit
// words for an fp64 one.  A word holding all ones has not been written yet; a published
// value with those bits is replaced by the canonical quiet NaN.
template <typename Acc> struct Words;
template <> struct Words<float> {
  typedef uint32_t W;
  static constexpr W kEmpty = 0xffffffffu;
  static constexpr W kNaN = 0x7fc00000u;
  __device__ __forceinline__ static W bits(float v) { return __float_as_uint(v); }
  __device__ __forceinline__ static float val(W w) { return __uint_as_float(w); }
};
template <> struct Words<double> {
  typedef unsigned long long W;
  static constexpr W kEmpty = ~0ull;
  static constexpr W kNaN = 0x7ff8000000000000ull;
  __device__ __forceinline__ static W bits(double v) { return (W)__double_as_longlong(v); }
  __device__ __forceinline__ static double val(W w) { return __longlong_as_double((long long)w); }
};

__device__ __forceinline__ float fmaA(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double fmaA(double a, double b, double c) { return fma(a, b, c); }

template <typename Acc>
__device__ __forceinline__ void publish(typename Words<Acc>::W* p, Acc v) {
  typename Words<Acc>::W u = Words<Acc>::bits(v);
  if (u == Words<Acc>::kEmpty) u = Words<Acc>::kNaN;
  __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename Acc>
__device__ __forceinline__ typename Words<Acc>::W peek(const typename Words<Acc>::W* p) {
  return __hip_atomic_load(const_cast<typename Words<Acc>::W*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Default bound on polls of one predecessor word; beyond it the look-back gives up: the
// carry becomes NaN (the output is then visibly wrong), the stall flag is set for the host,
// and the kernel goes on instead of waiting forever.
constexpr int kMaxPolls = 1 << 20;

// Decoupled look-back for one channel, with a canonical result.  `incl`, `aggA`, `aggH`
// are indexed by chain position (0 = first chunk of the chain) times `stride`.  Position
// `pos` walks back over positions pos-1, pos-2, ... collecting published aggregates until
// it meets a published inclusive state, then applies the collected aggregates forward in
// chain order: h <- fma(A_j, h, H_j).  Every inclusive state is published as
// fma(A, carry, H), so the carry equals, bit for bit, the one a strictly sequential chain
// would compute, whatever the timing: results are reproducible run to run.  At most
// kWindow aggregates are collected; past that the walk waits for an inclusive state.
// `bufA`, `bufH` are kWindow values of scratch (LDS) owned by the calling thread.
// A wait that exceeds max_polls polls of one word (max_polls < 0: any look-back at all)
// gives up: it stores 1 to *stall and returns NaN.
constexpr int kWindow = 16;

template <typename Acc>
__device__ __forceinline__ Acc lookback_carry(const typename Words<Acc>::W* incl,
                                              const typename Words<Acc>::W* aggA,
                                              const typename Words<Acc>::W* aggH, int pos,
                                              size_t stride, Acc* bufA, Acc* bufH, int max_polls,
                                              uint32_t* stall) {
  typedef Words<Acc> Wd;
  auto give_up = [&]() {
    __hip_atomic_store(stall, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return Wd::val(Wd::kNaN);
  };
  if (max_polls < 0) return give_up();
  int j = pos - 1;
  int n = 0;
  int polls = 0;
  Acc h;
  while (true) {
    const typename Wd::W vi = peek<Acc>(incl + size_t(j) * stride);
    if (vi != Wd::kEmpty) {
      h = Wd::val(vi);
      break;
    }
    if (n < kWindow) {
      const typename Wd::W va = peek<Acc>(aggA + size_t(j) * stride);
      const typename Wd::W vh = peek<Acc>(aggH + size_t(j) * stride);
      if (va != Wd::kEmpty && vh != Wd::kEmpty) {
        bufA[n] = Wd::val(va);
        bufH[n] = Wd::val(vh);
        ++n;
        --j;   // position 0 always publishes an inclusive state, so j stays >= 0
        polls = 0;
        continue;
      }
    }
    if (++polls > max_polls) return give_up();
    __builtin_amdgcn_s_sleep(1);
  }
  for (int k = n - 1; k >= 0; --k) h = fmaA(bufA[k], h, bufH[k]);
  return h;
}

}  // namespace rglru
