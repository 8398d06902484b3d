// Causal depthwise Conv1D of temporal width 4 (Griffin model-architecture page, section
// "Recurrent block": a small separable Conv1D with only 4*D parameters placed before the
// RG-LRU).  Elementwise and HBM-bound: each thread owns four consecutive channels of one
// sequence and a run of 8 time steps; it loads the run's 11 input rows at once (the loads
// are in flight together) and writes the 8 output rows, so u is written once and x read
// from HBM about once (the 3 halo rows of each run are the previous run's rows, mostly L2
// hits), with coalesced 8/16-byte accesses along the channels.  Runs of 8 rather than 16
// steps: 41 instead of 47 us at 8 x 2048 x 2560 bf16 (fewer registers, more waves).
#include "rglru_device.h"
#include "kernels.h"

namespace rglru {

constexpr int kConvSteps = 8;   // time steps per thread

// Blocks past `conv_blocks` do not convolve: they set `fill_words` words at `fill` to all
// ones and zero the 64 words at `counter` (the look-back status and ticket counters of
// the scan that follows on the stream),
// which saves the scan a separate initialisation launch.
template <typename IO>
__global__ __launch_bounds__(256) void conv_fwd_kernel(int B, int T, int D, const IO* __restrict__ x,
                                                       const IO* __restrict__ w,
                                                       const float* __restrict__ cb,
                                                       const IO* __restrict__ state_in,
                                                       IO* __restrict__ u,
                                                       IO* __restrict__ state_out, int conv_blocks,
                                                       uint32_t* __restrict__ fill, size_t fill_words,
                                                       uint32_t* __restrict__ counter) {
  if (int(blockIdx.x) >= conv_blocks) {
    const size_t fb = blockIdx.x - conv_blocks, nfb = gridDim.x - conv_blocks;
    for (size_t i = fb * 256 + threadIdx.x; i < fill_words; i += nfb * 256) fill[i] = 0xffffffffu;
    if (fb == 0 && threadIdx.x < 64 && counter) counter[threadIdx.x] = 0u;
    return;
  }
  const int nq = D / 4;
  const int nt = (T + kConvSteps - 1) / kConvSteps;
  const long item = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= long(B) * nt * nq) return;
  const int q = int(item % nq);
  const int tc = int((item / nq) % nt);
  const int b = int(item / (long(nq) * nt));
  const int d = 4 * q;
  const float4 w0 = Io<IO>::load4(w + d), w1 = Io<IO>::load4(w + D + d),
               w2 = Io<IO>::load4(w + 2 * D + d), w3 = Io<IO>::load4(w + 3 * D + d);
  const float4 bias = cb ? *reinterpret_cast<const float4*>(cb + d) : make_float4(0, 0, 0, 0);
  // X(t) = x[b,t] for t >= 0, state_in[b,3+t] for t < 0 (zeros without a state)
  auto X = [&](int t) -> float4 {
    if (t >= 0) return Io<IO>::load4(x + (size_t(b) * T + t) * D + d);
    if (state_in) return Io<IO>::load4(state_in + (size_t(b) * 3 + 3 + t) * D + d);
    return make_float4(0, 0, 0, 0);
  };
  const int t0 = tc * kConvSteps;
  // all kConvSteps + 3 input rows are loaded before any arithmetic, so the loads are in
  // flight together; rows past the end are clamped to the last row (their outputs are not
  // stored)
  float4 xs[kConvSteps + 3];
#pragma unroll
  for (int j = 0; j < kConvSteps + 3; ++j) {
    const int t = t0 - 3 + j;
    xs[j] = (j < 3 && t0 == 0) ? X(t) : Io<IO>::load4(x + (size_t(b) * T + min(t, T - 1)) * D + d);
  }
#pragma unroll
  for (int i = 0; i < kConvSteps; ++i) {
    const int t = t0 + i;
    float4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f4set(o, j, conv_u<IO>(f4get(bias, j), f4get(w0, j), f4get(w1, j), f4get(w2, j),
                             f4get(w3, j), f4get(xs[i + 3], j), f4get(xs[i + 2], j),
                             f4get(xs[i + 1], j), f4get(xs[i], j)));
    if (t < T) Io<IO>::store4(u + (size_t(b) * T + t) * D + d, o);
  }
  if (state_out && tc == 0) {
    for (int j = 0; j < 3; ++j) Io<IO>::store4(state_out + (size_t(b) * 3 + j) * D + d, X(T - 3 + j));
  }
}

// One decode step of the conv: u_t from x_t and the three-token history, then the
// history is shifted in place (each thread touches only its own channels).
template <typename IO>
__global__ __launch_bounds__(256) void conv_decode_kernel(int B, int D, const IO* __restrict__ x,
                                                          const IO* __restrict__ w,
                                                          const float* __restrict__ cb,
                                                          IO* __restrict__ hist,
                                                          IO* __restrict__ u) {
  const int nq = D / 4;
  const long item = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= long(B) * nq) return;
  const int b = int(item / nq), d = 4 * int(item % nq);
  const float4 w0 = Io<IO>::load4(w + d), w1 = Io<IO>::load4(w + D + d),
               w2 = Io<IO>::load4(w + 2 * D + d), w3 = Io<IO>::load4(w + 3 * D + d);
  const float4 bias = cb ? *reinterpret_cast<const float4*>(cb + d) : make_float4(0, 0, 0, 0);
  IO* hb = hist + size_t(b) * 3 * D + d;
  const float4 xm3 = Io<IO>::load4(hb), xm2 = Io<IO>::load4(hb + D), xm1 = Io<IO>::load4(hb + 2 * D);
  const IO* xp = x + size_t(b) * D + d;
  const float4 x0 = Io<IO>::load4(xp);
  float4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f4set(o, j, conv_u<IO>(f4get(bias, j), f4get(w0, j), f4get(w1, j), f4get(w2, j),
                           f4get(w3, j), f4get(x0, j), f4get(xm1, j), f4get(xm2, j),
                           f4get(xm3, j)));
  Io<IO>::store4(u + size_t(b) * D + d, o);
  // shift: (x_{t-3}, x_{t-2}, x_{t-1}) <- (x_{t-2}, x_{t-1}, x_t); stores are bit copies
  const int nb = sizeof(IO) * 4;
  if (nb == 8) {
    const uint2 v1 = *reinterpret_cast<const uint2*>(hb + D), v2 = *reinterpret_cast<const uint2*>(hb + 2 * D),
                v0 = *reinterpret_cast<const uint2*>(xp);
    *reinterpret_cast<uint2*>(hb) = v1;
    *reinterpret_cast<uint2*>(hb + D) = v2;
    *reinterpret_cast<uint2*>(hb + 2 * D) = v0;
  } else {
    const uint4 v1 = *reinterpret_cast<const uint4*>(hb + D), v2 = *reinterpret_cast<const uint4*>(hb + 2 * D),
                v0 = *reinterpret_cast<const uint4*>(xp);
    *reinterpret_cast<uint4*>(hb) = v1;
    *reinterpret_cast<uint4*>(hb + D) = v2;
    *reinterpret_cast<uint4*>(hb + 2 * D) = v0;
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

// ------------------------------------------------------------------ launchers
template <typename IO>
hipError_t launch_conv_fwd(int B, int T, int D, const void* x, const void* w, const float* cb,
                           const void* state_in, void* u, void* state_out, hipStream_t s,
                           uint32_t* fill, size_t fill_words, uint32_t* counter) {
  const long items = long(B) * ((T + kConvSteps - 1) / kConvSteps) * (D / 4);
  const int blocks = int((items + 255) / 256);
  size_t fill_blocks = (fill_words + 255) / 256;
  if (fill_blocks > 1024) fill_blocks = 1024;
  if (fill_blocks == 0 && counter) fill_blocks = 1;
  conv_fwd_kernel<IO><<<blocks + int(fill_blocks), 256, 0, s>>>(
      B, T, D, static_cast<const IO*>(x), static_cast<const IO*>(w), cb,
      static_cast<const IO*>(state_in), static_cast<IO*>(u), static_cast<IO*>(state_out), blocks,
      fill, fill_words, counter);
  return hipGetLastError();
}
template hipError_t launch_conv_fwd<float>(int, int, int, const void*, const void*, const float*,
                                           const void*, void*, void*, hipStream_t, uint32_t*, size_t,
                                           uint32_t*);
template hipError_t launch_conv_fwd<bf16_t>(int, int, int, const void*, const void*, const float*,
                                            const void*, void*, void*, hipStream_t, uint32_t*,
                                            size_t, uint32_t*);

template <typename IO>
hipError_t launch_conv_decode(int B, int D, const void* x, const void* w, const float* cb,
                              void* hist, void* u, hipStream_t s) {
  const long items = long(B) * (D / 4);
  conv_decode_kernel<IO><<<int((items + 255) / 256), 256, 0, s>>>(
      B, D, static_cast<const IO*>(x), static_cast<const IO*>(w), cb, static_cast<IO*>(hist),
      static_cast<IO*>(u));
  return hipGetLastError();
}
template hipError_t launch_conv_decode<float>(int, int, const void*, const void*, const float*,
                                              void*, void*, hipStream_t);
template hipError_t launch_conv_decode<bf16_t>(int, int, const void*, const void*, const float*,
                                               void*, void*, hipStream_t);

// Look-back status words to all ones (empty) and ncounters ticket counters to zero, in one
// launch.
// 16-byte stores over the first n4 * 4 words (status is 16-byte aligned), then the tail.
__global__ __launch_bounds__(256) void fill_status_kernel(uint32_t* __restrict__ status, size_t n,
                                                          uint32_t* __restrict__ counters,
                                                          int ncounters) {
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < size_t(ncounters)) counters[i] = 0u;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  const size_t n4 = n / 4;
  uint4* s4 = reinterpret_cast<uint4*>(status);
  const uint4 ones = make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);
  for (size_t k = i; k < n4; k += stride) s4[k] = ones;
  if (i < n - n4 * 4) status[n4 * 4 + i] = 0xffffffffu;
}

hipError_t launch_fill_status(uint32_t* status, size_t words, uint32_t* counters, int ncounters,
                              hipStream_t s) {
  size_t blocks = (words / 4 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  fill_status_kernel<<<int(blocks), 256, 0, s>>>(status, words, counters, ncounters);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_u32_kernel<<<int(blocks), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace rglru
