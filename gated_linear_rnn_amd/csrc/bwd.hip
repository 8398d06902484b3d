// Backward helpers of the RG-LRU temporal branch (the pages state no backward; these
// are the chain rule through the "Recurrent block" Conv1D and the gate projections of
// Eq. (1)-(2) of the Griffin model-architecture page).
//   * tiled transposes that put the reduction axis of the weight-gradient and
//     input-gradient products last, so both run on the same K-contiguous MFMA kernel;
//   * the conv backward: dx_tau = sum_k w[k] du_{tau+k}, and per-tile partial sums of
//     du_t x_{t-k} and du_t for dconv_w, dconv_b;
//   * one fixed-order reduction of all per-tile partials (bitwise reproducible).
#include "rglru_device.h"
#include "kernels.h"

namespace rglru {

// dst[c * ldd + r] = src[r * lds + c] for r < R; zero for R <= r < Rp.
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ src, int R, int C,
                                                        int lds, E* __restrict__ dst, int ldd,
                                                        int Rp) {
  __shared__ E tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? src[size_t(r) * lds + c] : E(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) dst[size_t(c) * ldd + r] = tile[tx][i];
  }
}

// The same with 16-byte accesses on both sides (V = 16 / sizeof(E) elements per access):
// a 64 x 64 tile goes through LDS, each thread loading one 16-byte run of a source row and
// storing one 16-byte run of a destination row.  Needs C, lds, ldd and Rp multiples of V and
// 16-byte aligned rows.
template <typename E>
__global__ __launch_bounds__(256) void transpose_vec_kernel(const E* __restrict__ src, int R, int C,
                                                            int lds, E* __restrict__ dst, int ldd,
                                                            int Rp) {
  constexpr int V = 16 / sizeof(E);
  constexpr int VPR = 64 / V;                       // 16-byte runs per 64-element tile row
  __shared__ E tile[64][64 + 2];                    // padded: column reads spread over banks
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * VPR; idx += 256) {
    const int i = idx / VPR, cv = (idx % VPR) * V;
    const int r = r0 + i, c = c0 + cv;
    E v[V];
    if (r < R && c < C) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + size_t(r) * lds + c);
      __builtin_memcpy(v, &w, 16);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) v[j] = E(0);
    }
#pragma unroll
    for (int j = 0; j < V; ++j) tile[i][cv + j] = v[j];
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * VPR; idx += 256) {
    const int i = idx / VPR, rv = (idx % VPR) * V;   // destination row c0 + i, columns r0 + rv ..
    const int c = c0 + i, r = r0 + rv;
    if (c >= C || r >= Rp) continue;
    E v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = tile[rv + j][i];
    uint4 w;
    __builtin_memcpy(&w, v, 16);
    *reinterpret_cast<uint4*>(dst + size_t(c) * ldd + r) = w;
  }
}

template <typename E>
hipError_t launch_transpose(const E* src, int R, int C, int lds, E* dst, int ldd, int Rp,
                            hipStream_t s) {
  constexpr int V = 16 / sizeof(E);
  dim3 grid((Rp + 63) / 64, (C + 63) / 64);
  const bool vec = C % V == 0 && lds % V == 0 && ldd % V == 0 && Rp % V == 0 &&
                   (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
  if (vec) transpose_vec_kernel<E><<<grid, 256, 0, s>>>(src, R, C, lds, dst, ldd, Rp);
  else transpose_kernel<E><<<grid, 256, 0, s>>>(src, R, C, lds, dst, ldd, Rp);
  return hipGetLastError();
}
template hipError_t launch_transpose<uint16_t>(const uint16_t*, int, int, int, uint16_t*, int, int,
                                               hipStream_t);
template hipError_t launch_transpose<float>(const float*, int, int, int, float*, int, int,
                                            hipStream_t);

constexpr int kBSteps = 8, kBTG = 16, kBChunk = 128, kBCh = 64;

// 4 consecutive elements moved in their storage format (global -> LDS), widened on read.
template <typename IO> struct Raw4x;
template <> struct Raw4x<bf16_t> {
  uint2 v;
  __device__ __forceinline__ void zero() { v = make_uint2(0u, 0u); }
  __device__ __forceinline__ void load(const bf16_t* g) { v = *reinterpret_cast<const uint2*>(g); }
  __device__ __forceinline__ void store(bf16_t* l) const { *reinterpret_cast<uint2*>(l) = v; }
  __device__ __forceinline__ static float4 read(const bf16_t* l) { return Io<bf16_t>::load4(l); }
};
template <> struct Raw4x<float> {
  float4 v;
  __device__ __forceinline__ void zero() { v = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load(const float* g) { v = *reinterpret_cast<const float4*>(g); }
  __device__ __forceinline__ void store(float* l) const { *reinterpret_cast<float4*>(l) = v; }
  __device__ __forceinline__ static float4 read(const float* l) { return *reinterpret_cast<const float4*>(l); }
};

template <typename IO>
__global__ __launch_bounds__(256) void conv_bwd_kernel(ConvBwdArgs p) {
  // du (fp32) and x (in its I/O type: 2 bytes at bf16, so three workgroups fit on a CU)
  // staging; after the time loop the same LDS holds the fp64 tile reduction
  constexpr int kDuBytes = (kBChunk + 3) * kBCh * 4;
  constexpr int kXBytes = (kBChunk + 3) * kBCh * int(sizeof(IO));
  constexpr int kRedBytes = int(sizeof(double)) * kBTG * 5 * kBCh;
  constexpr int kSmem = kDuBytes + kXBytes > kRedBytes ? kDuBytes + kXBytes : kRedBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  float* dus = reinterpret_cast<float*>(smem);
  IO* xs = reinterpret_cast<IO*>(smem + kDuBytes);
  double (*sRed)[5][kBCh] = reinterpret_cast<double (*)[5][kBCh]>(smem);
  const int B = p.B, T = p.T, D = p.D;
  const int nchunks = (T + kBChunk - 1) / kBChunk;
  const int nq = D / kBCh;
  const int blk = blockIdx.x % (B * nq);
  const int chunk = blockIdx.x / (B * nq);
  const int b = blk / nq, d0 = (blk % nq) * kBCh;
  const int t0 = chunk * kBChunk;
  const int tid = threadIdx.x, cg = tid & 15, tg = tid >> 4;
  const int d = d0 + 4 * cg;
  const IO* x = static_cast<const IO*>(p.x);
  const IO* cs = static_cast<const IO*>(p.conv_state);
  // du rows t0 .. t0+130 (zero past T); x rows t0-3 .. t0+127 (history for t < 0)
  for (int idx = tid; idx < (kBChunk + 3) * 16; idx += 256) {
    const int rr = idx >> 4, q = idx & 15;
    const int tdu = t0 + rr;
    float4 v = make_float4(0, 0, 0, 0);
    if (tdu < T) v = *reinterpret_cast<const float4*>(p.du + (size_t(b) * T + tdu) * D + d0 + 4 * q);
    *reinterpret_cast<float4*>(&dus[rr * kBCh + 4 * q]) = v;
    const int tx = t0 - 3 + rr;
    Raw4x<IO> xv;
    xv.zero();
    if (tx >= 0 && tx < T) xv.load(x + (size_t(b) * T + tx) * D + d0 + 4 * q);
    else if (tx < 0 && cs) xv.load(cs + (size_t(b) * 3 + 3 + tx) * D + d0 + 4 * q);
    xv.store(&xs[rr * kBCh + 4 * q]);
  }
  const IO* w = static_cast<const IO*>(p.conv_w);
  const float4 w0 = Io<IO>::load4(w + d), w1 = Io<IO>::load4(w + D + d),
               w2 = Io<IO>::load4(w + 2 * D + d), w3 = Io<IO>::load4(w + 3 * D + d);
  __syncthreads();
  double pw[4][4] = {}, pb[4] = {};
  for (int s = 0; s < kBSteps; ++s) {
    const int lt = tg * kBSteps + s;         // local time
    const int t = t0 + lt;
    if (t >= T) break;
    const float4 du0 = *reinterpret_cast<const float4*>(&dus[lt * kBCh + 4 * cg]);
    const float4 du1 = *reinterpret_cast<const float4*>(&dus[(lt + 1) * kBCh + 4 * cg]);
    const float4 du2 = *reinterpret_cast<const float4*>(&dus[(lt + 2) * kBCh + 4 * cg]);
    const float4 du3 = *reinterpret_cast<const float4*>(&dus[(lt + 3) * kBCh + 4 * cg]);
    const float4 x0 = Raw4x<IO>::read(&xs[(lt + 3) * kBCh + 4 * cg]);
    const float4 x1 = Raw4x<IO>::read(&xs[(lt + 2) * kBCh + 4 * cg]);
    const float4 x2 = Raw4x<IO>::read(&xs[(lt + 1) * kBCh + 4 * cg]);
    const float4 x3 = Raw4x<IO>::read(&xs[lt * kBCh + 4 * cg]);
    float4 dxv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = f4get(w0, j) * f4get(du0, j);
      acc = fmaf(f4get(w1, j), f4get(du1, j), acc);
      acc = fmaf(f4get(w2, j), f4get(du2, j), acc);
      acc = fmaf(f4get(w3, j), f4get(du3, j), acc);
      f4set(dxv, j, acc);
      const double g = f4get(du0, j);
      pw[0][j] = fma(g, double(f4get(x0, j)), pw[0][j]);
      pw[1][j] = fma(g, double(f4get(x1, j)), pw[1][j]);
      pw[2][j] = fma(g, double(f4get(x2, j)), pw[2][j]);
      pw[3][j] = fma(g, double(f4get(x3, j)), pw[3][j]);
      pb[j] += g;
    }
    *reinterpret_cast<float4*>(p.dx + (size_t(b) * T + t) * D + d) = dxv;
  }
  __syncthreads();   // staging reads done: the LDS is reused for the reduction
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) sRed[tg][k][4 * cg + j] = pw[k][j];
    sRed[tg][4][4 * cg + j] = pb[j];
  }
  __syncthreads();
  for (int k = tid; k < 5 * kBCh; k += 256) {
    const int qn = k / kBCh, c = k % kBCh;
    double acc = 0.0;
    for (int q = 0; q < kBTG; ++q) acc += sRed[q][qn][c];
    p.partial[(size_t(b) * nchunks + chunk) * 5 * D + size_t(qn) * D + d0 + c] = acc;
  }
}

template <typename IO>
hipError_t launch_conv_bwd(const ConvBwdArgs& a, hipStream_t s) {
  const int blocks = ((a.T + kBChunk - 1) / kBChunk) * a.B * (a.D / kBCh);
  conv_bwd_kernel<IO><<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}
template hipError_t launch_conv_bwd<float>(const ConvBwdArgs&, hipStream_t);
template hipError_t launch_conv_bwd<bf16_t>(const ConvBwdArgs&, hipStream_t);

// Sums of per-tile partials in a fixed order (tile index ascending), in fp64.
// One thread per (quantity, channel): q < 3 the scan partials (db_a, db_x, the dLambda sum),
// q = 3 .. 7 the conv partials (dconv_w rows 0..3, dconv_b).  Each sums its P partial rows
// in order, so the result does not depend on how threads are scheduled.
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs p) {
  const size_t D = p.D;
  const size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nq = p.conv_part ? 8 : 3;
  if (idx >= size_t(nq) * D) return;
  const int q = int(idx / D), d = int(idx % D);
  const double* src = q < 3 ? p.scan_part + size_t(q) * D + d : p.conv_part + size_t(q - 3) * D + d;
  const size_t stride = (q < 3 ? 3 : 5) * D;
  double acc = 0.0;
#pragma unroll 8
  for (int r = 0; r < p.P; ++r) acc += src[size_t(r) * stride];   // loads ahead, adds in order
  switch (q) {
    case 0: p.db_a[d] = float(acc); break;
    case 1: p.db_x[d] = float(acc); break;
    case 2: p.dlambda[d] = float(acc * double(sigmoid_negf(p.lam[d]))); break;
    case 7: if (p.dconv_b) p.dconv_b[d] = float(acc); break;
    default: if (p.dconv_w) p.dconv_w[size_t(q - 3) * D + d] = float(acc); break;
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  const size_t threads = size_t(a.conv_part ? 8 : 3) * a.D;
  reduce_kernel<<<int((threads + 255) / 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rglru
