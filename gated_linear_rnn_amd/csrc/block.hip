// Elementwise steps of the recurrent block and of the gated MLP block for fp32 I/O
// (Griffin model-architecture page, sections "Recurrent block", Fig. 2(c), and "MLP block",
// Fig. 2(b)).  In the recurrent block the two input linears arrive as one [M, 2R] product:
// its first R columns are the branch input p, GeLU of the other R columns is the
// multiplier g; after the temporal branch, z = y g feeds the output linear.  In the MLP the
// product GeLU(q1) q2 of its two branch outputs feeds its last linear.  The bf16 path fuses
// these steps into the matrix-core kernels (GEMM epilogues and the fused RG-LRU kernel), so
// these only serve the fp32 reference-precision path.
#include "kernels.h"
#include "rglru_device.h"

namespace rglru {

// p[m, r] = pq[m, r], g[m, r] = RNE_f32(GeLU(pq[m, R + r])) with GeLU evaluated in fp64.
__global__ __launch_bounds__(256) void split_gelu_f32_kernel(const float* __restrict__ pq, int M,
                                                             int R, float* __restrict__ p,
                                                             float* __restrict__ g) {
  const size_t n = size_t(M) * R;
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += size_t(gridDim.x) * blockDim.x) {
    const size_t m = o / R, r = o - m * R;
    p[o] = pq[m * 2 * R + r];
    g[o] = float(gelu_d(double(pq[m * 2 * R + R + r])));
  }
}

// y[i] = RNE_f32(y[i] * g[i])
__global__ __launch_bounds__(256) void mul_f32_kernel(float* __restrict__ y,
                                                      const float* __restrict__ g, size_t n) {
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += size_t(gridDim.x) * blockDim.x)
    y[o] = y[o] * g[o];
}

// h[i] = RNE_f32(GeLU(q1[i]) * q2[i]), the product evaluated in fp64
__global__ __launch_bounds__(256) void geglu_f32_kernel(const float* __restrict__ q1,
                                                        const float* __restrict__ q2,
                                                        float* __restrict__ h, size_t n) {
  for (size_t o = size_t(blockIdx.x) * blockDim.x + threadIdx.x; o < n;
       o += size_t(gridDim.x) * blockDim.x)
    h[o] = float(gelu_d(double(q1[o])) * double(q2[o]));
}

// Decode step of the recurrent block (bf16): the input linears' split-K partials [S][M][2R]
// added in split order; the first R columns rounded to p, GeLU of the rest (the same fp32
// approximation as the forward GEMM epilogue) rounded to g.  8 columns per thread.
__global__ __launch_bounds__(256) void inproj_finish_kernel(const float* __restrict__ partial, int S,
                                                            int M, int R, bf16_t* __restrict__ p,
                                                            bf16_t* __restrict__ g) {
  const int N = 2 * R;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= size_t(M) * (N / 8)) return;
  const int m = int(idx / (N / 8)), n = int(idx % (N / 8)) * 8;
  const float* src = partial + size_t(m) * N + n;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = src[e];
  for (int s = 1; s < S; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] += src[size_t(s) * M * N + e];
  const bool gelu = n >= R;
  bf16_t* dst = gelu ? g + size_t(m) * R + (n - R) : p + size_t(m) * R + n;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = f2bf(gelu ? gelu_fast(v[e]) : v[e]);
}

static int grid_for(size_t n) {
  const size_t blocks = (n + 255) / 256;
  return int(blocks > 8192 ? 8192 : blocks);
}

hipError_t launch_split_gelu_f32(const float* pq, int M, int R, float* p, float* g, hipStream_t s) {
  split_gelu_f32_kernel<<<grid_for(size_t(M) * R), 256, 0, s>>>(pq, M, R, p, g);
  return hipGetLastError();
}

hipError_t launch_mul_f32(float* y, const float* g, size_t n, hipStream_t s) {
  mul_f32_kernel<<<grid_for(n), 256, 0, s>>>(y, g, n);
  return hipGetLastError();
}

hipError_t launch_geglu_f32(const float* q1, const float* q2, float* h, size_t n, hipStream_t s) {
  geglu_f32_kernel<<<grid_for(n), 256, 0, s>>>(q1, q2, h, n);
  return hipGetLastError();
}

hipError_t launch_splitk_inproj_bf16(const float* partial, int S, int M, int R, void* p, void* g,
                                     hipStream_t s) {
  const size_t n = size_t(M) * (2 * R / 8);
  inproj_finish_kernel<<<int((n + 255) / 256), 256, 0, s>>>(partial, S, M, R, static_cast<bf16_t*>(p),
                                                         static_cast<bf16_t*>(g));
  return hipGetLastError();
}

}  // namespace rglru
